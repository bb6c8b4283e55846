// Matmul kernels that carry the epilogue modes (gate/up activation, row
// argmax, fp32 output): the matrix-core path for one or two rows.
#include <hip/hip_runtime.h>

#include "w4a16_variants.hpp"

namespace w4a16 {

#define W4A16_V(P, MM, T, KW, D, AS) {P, MM, T, KW, D, AS, gemm_kernel<P, MM, T, KW, D, AS, true>},
const Variant kVariantsEpiMfma12[] = {W4A16_VARIANT_LIST_CT_MFMA12(W4A16_V)};
const int kNumEpiMfma12 = sizeof(kVariantsEpiMfma12) / sizeof(kVariantsEpiMfma12[0]);

}  // namespace w4a16
