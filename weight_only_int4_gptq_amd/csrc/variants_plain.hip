// Plain matmul kernels (no epilogue modes) with compile-time row counts.
#include <hip/hip_runtime.h>

#include "w4a16_variants.hpp"

namespace w4a16 {

#define W4A16_V(P, MM, T, KW, D, AS) {P, MM, T, KW, D, AS, gemm_kernel<P, MM, T, KW, D, AS, false>},
const Variant kVariantsPlainCt[] = {W4A16_VARIANT_LIST_CT(W4A16_V)};
const int kNumPlainCt = sizeof(kVariantsPlainCt) / sizeof(kVariantsPlainCt[0]);

}  // namespace w4a16
