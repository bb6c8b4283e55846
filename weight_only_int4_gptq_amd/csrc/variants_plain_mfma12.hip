// Plain matmul kernels (no epilogue modes): the matrix-core path for one or
// two rows, compile-time row counts.
#include <hip/hip_runtime.h>

#include "w4a16_variants.hpp"

namespace w4a16 {

#define W4A16_V(P, MM, T, KW, D, AS) {P, MM, T, KW, D, AS, gemm_kernel<P, MM, T, KW, D, AS, false>},
const Variant kVariantsPlainMfma12[] = {W4A16_VARIANT_LIST_CT_MFMA12(W4A16_V)};
const int kNumPlainMfma12 = sizeof(kVariantsPlainMfma12) / sizeof(kVariantsPlainMfma12[0]);

}  // namespace w4a16
