// Matmul kernels that carry the epilogue modes (gate/up activation, row
// argmax, fp32 output): the GEMV path, compile-time row counts.
#include <hip/hip_runtime.h>

#include "w4a16_variants.hpp"

namespace w4a16 {

#define W4A16_V(P, MM, T, KW, D, AS) {P, MM, T, KW, D, AS, gemm_kernel<P, MM, T, KW, D, AS, true>},
const Variant kVariantsEpiGemv[] = {W4A16_VARIANT_LIST_CT_GEMV(W4A16_V)};
const int kNumEpiGemv = sizeof(kVariantsEpiGemv) / sizeof(kVariantsEpiGemv[0]);

}  // namespace w4a16
