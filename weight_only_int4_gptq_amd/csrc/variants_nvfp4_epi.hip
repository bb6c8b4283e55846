// NVFP4 weight-only matmul kernels that carry the epilogue modes (gate/up
// activation, row argmax, fp32 output), for every compiled shape.
#include <hip/hip_runtime.h>

#include "w4a16_variants.hpp"

namespace w4a16 {

#define W4A16_NV_V(P, MM, T, KW, D, AS) {P, MM, T, KW, D, AS, gemm_kernel<P, MM, T, KW, D, AS, true, FMT_NVFP4>},
const Variant kVariantsNvEpi[] = {W4A16_NV_VARIANT_LIST(W4A16_NV_V)};
const int kNumVariantsNvEpi = sizeof(kVariantsNvEpi) / sizeof(kVariantsNvEpi[0]);

}  // namespace w4a16
