// Plain matmul kernels (no epilogue modes): the GEMV path, compile-time row
// counts.
#include <hip/hip_runtime.h>

#include "w4a16_variants.hpp"

namespace w4a16 {

#define W4A16_V(P, MM, T, KW, D, AS) {P, MM, T, KW, D, AS, gemm_kernel<P, MM, T, KW, D, AS, false>},
const Variant kVariantsPlainGemv[] = {W4A16_VARIANT_LIST_CT_GEMV(W4A16_V)};
const int kNumPlainGemv = sizeof(kVariantsPlainGemv) / sizeof(kVariantsPlainGemv[0]);

}  // namespace w4a16
