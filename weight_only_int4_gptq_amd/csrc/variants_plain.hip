// Plain matmul kernels (no epilogue modes) for every compiled shape.
#include <hip/hip_runtime.h>

#include "w4a16_variants.hpp"

namespace w4a16 {

#define W4A16_V(P, MM, T, KW, D, AS) {P, MM, T, KW, D, AS, gemm_kernel<P, MM, T, KW, D, AS, false>},
const Variant kVariantsPlain[] = {W4A16_VARIANT_LIST(W4A16_V)};
const int kNumVariants = sizeof(kVariantsPlain) / sizeof(kVariantsPlain[0]);

}  // namespace w4a16
