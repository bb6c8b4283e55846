// NVFP4 weight-only matmul kernels for every compiled shape.
#include <hip/hip_runtime.h>

#include "w4a16_variants.hpp"

namespace w4a16 {

#define W4A16_NV_V(P, MM, T, KW, D, AS) {P, MM, T, KW, D, AS, gemm_kernel<P, MM, T, KW, D, AS, false, FMT_NVFP4>},
const Variant kVariantsNv[] = {W4A16_NV_VARIANT_LIST(W4A16_NV_V)};
const int kNumVariantsNv = sizeof(kVariantsNv) / sizeof(kVariantsNv[0]);

}  // namespace w4a16
