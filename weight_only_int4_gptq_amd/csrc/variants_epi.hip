// Matmul kernels that carry the epilogue modes (gate/up activation, row
// argmax, fp32 output), for every compiled shape.
#include <hip/hip_runtime.h>

#include "w4a16_variants.hpp"

namespace w4a16 {

#define W4A16_V(P, MM, T, KW, D, AS) {P, MM, T, KW, D, AS, gemm_kernel<P, MM, T, KW, D, AS, true>},
const Variant kVariantsEpi[] = {W4A16_VARIANT_LIST(W4A16_V)};

}  // namespace w4a16
