// NVFP4 weight-only matmul kernels, plain: the matrix-core path.
#include <hip/hip_runtime.h>

#include "w4a16_variants.hpp"

namespace w4a16 {

#define W4A16_V(P, MM, T, KW, D, AS) {P, MM, T, KW, D, AS, gemm_kernel<P, MM, T, KW, D, AS, false, FMT_NVFP4>},
const Variant kVariantsNvMfma[] = {W4A16_NV_VARIANT_LIST_MFMA(W4A16_V)};
const int kNumNvMfma = sizeof(kVariantsNvMfma) / sizeof(kVariantsNvMfma[0]);

}  // namespace w4a16
