// NVFP4 weight-only matmul kernels that carry the epilogue modes (gate/up
// activation, row argmax, fp32 output): the GEMV path.
#include <hip/hip_runtime.h>

#include "w4a16_variants.hpp"

namespace w4a16 {

#define W4A16_V(P, MM, T, KW, D, AS) {P, MM, T, KW, D, AS, gemm_kernel<P, MM, T, KW, D, AS, true, FMT_NVFP4>},
const Variant kVariantsNvEpiGemv[] = {W4A16_NV_VARIANT_LIST_GEMV(W4A16_V)};
const int kNumNvEpiGemv = sizeof(kVariantsNvEpiGemv) / sizeof(kVariantsNvEpiGemv[0]);

}  // namespace w4a16
