// NVFP4 weight-only matmul kernels that carry the epilogue modes (gate/up
// activation, row argmax, fp32 output): the matrix-core path.
#include <hip/hip_runtime.h>

#include "w4a16_variants.hpp"

namespace w4a16 {

#define W4A16_V(P, MM, T, KW, D, AS) {P, MM, T, KW, D, AS, gemm_kernel<P, MM, T, KW, D, AS, true, FMT_NVFP4>},
const Variant kVariantsNvEpiMfma[] = {W4A16_NV_VARIANT_LIST_MFMA(W4A16_V)};
const int kNumNvEpiMfma = sizeof(kVariantsNvEpiMfma) / sizeof(kVariantsNvEpiMfma[0]);

}  // namespace w4a16
