// Plain matmul kernels (no epilogue modes) that take the row count at run time.
#include <hip/hip_runtime.h>

#include "w4a16_variants.hpp"

namespace w4a16 {

#define W4A16_V(P, MM, T, KW, D, AS) {P, MM, T, KW, D, AS, gemm_kernel<P, MM, T, KW, D, AS, false>},
const Variant kVariantsPlainRt[] = {W4A16_VARIANT_LIST_RT(W4A16_V)};
const int kNumPlainRt = sizeof(kVariantsPlainRt) / sizeof(kVariantsPlainRt[0]);

}  // namespace w4a16
