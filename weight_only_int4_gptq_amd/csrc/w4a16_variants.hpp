// The compiled kernel shapes of the W4A16 matmul, shared by the two
// instantiation units (variants_plain.hip, variants_epi.hip) and the host
// code that picks a kernel for a plan.
#pragma once

#include "w4a16_kernels.hpp"

namespace w4a16 {

using KernelFn = void (*)(GemmArgs);

struct Variant {
    int path, mm, tiles, kwaves, depth, asrc;   // mm: compile-time row count (0: run time)
    KernelFn fn;
};

// (tiles, kwaves, depth) shapes instantiated for every path / row count
#define W4A16_SHAPES(X, P, MM, AS) \
    X(P, MM, 1, 1, 8, AS) X(P, MM, 1, 4, 8, AS) X(P, MM, 1, 8, 4, AS) X(P, MM, 1, 8, 8, AS) \
    X(P, MM, 2, 4, 4, AS) X(P, MM, 2, 8, 4, AS) X(P, MM, 2, 4, 8, AS) X(P, MM, 4, 4, 2, AS) \
    X(P, MM, 4, 4, 4, AS)

// A streamed per group through a per-wavefront LDS ring (matrix-core path)
#define W4A16_RINGS(X, P, MM, AS) \
    X(P, MM, 1, 4, 4, AS) X(P, MM, 1, 8, 4, AS) X(P, MM, 2, 4, 2, AS) X(P, MM, 2, 4, 4, AS) \
    X(P, MM, 4, 4, 2, AS) X(P, MM, 4, 2, 2, AS) X(P, MM, 4, 4, 4, AS) X(P, MM, 8, 1, 4, AS) \
    X(P, MM, 8, 2, 2, AS) X(P, MM, 8, 4, 2, AS)

// eight-tile strips: A read once per eight tiles (matrix-core paths)
#define W4A16_WIDE(X, P, MM, AS) \
    X(P, MM, 8, 4, 2, AS) X(P, MM, 8, 2, 2, AS) X(P, MM, 8, 2, 4, AS) X(P, MM, 8, 1, 4, AS)

// deeper rings for one row: a wavefront's groups in one or few rounds
#define W4A16_ONESHOT(X, P, MM, AS) \
    X(P, MM, 2, 4, 10, AS) X(P, MM, 2, 4, 5, AS) X(P, MM, 4, 4, 5, AS) X(P, MM, 4, 8, 5, AS) \
    X(P, MM, 1, 4, 10, AS) X(P, MM, 2, 2, 10, AS) X(P, MM, 4, 2, 5, AS) X(P, MM, 1, 8, 17, AS) \
    X(P, MM, 2, 8, 17, AS) X(P, MM, 2, 4, 17, AS) X(P, MM, 4, 4, 10, AS) X(P, MM, 2, 2, 17, AS)

#define W4A16_VARIANT_LIST(X)                                                                       \
    W4A16_ONESHOT(X, PATH_GEMV, 1, ASRC_LDS) W4A16_ONESHOT(X, PATH_MFMA, 1, ASRC_LDS)               \
    W4A16_ONESHOT(X, PATH_MFMA, 1, ASRC_GLOBAL)                                                     \
    W4A16_SHAPES(X, PATH_GEMV, 1, ASRC_LDS) W4A16_SHAPES(X, PATH_GEMV, 2, ASRC_LDS)                 \
    W4A16_SHAPES(X, PATH_GEMV, 3, ASRC_LDS) W4A16_SHAPES(X, PATH_GEMV, 4, ASRC_LDS)                 \
    W4A16_RINGS(X, PATH_MFMA, 0, ASRC_RING)                                                         \
    W4A16_WIDE(X, PATH_MFMA, 0, ASRC_LDS) W4A16_WIDE(X, PATH_MFMA, 0, ASRC_GLOBAL)                  \
    W4A16_WIDE(X, PATH_MFMA, 2, ASRC_LDS) W4A16_WIDE(X, PATH_MFMA, 3, ASRC_LDS)                     \
    W4A16_WIDE(X, PATH_MFMA, 4, ASRC_LDS)                                                           \
    W4A16_SHAPES(X, PATH_MFMA, 0, ASRC_LDS) W4A16_SHAPES(X, PATH_MFMA, 0, ASRC_GLOBAL)              \
    W4A16_SHAPES(X, PATH_MFMA, 1, ASRC_LDS) W4A16_SHAPES(X, PATH_MFMA, 1, ASRC_GLOBAL)              \
    W4A16_SHAPES(X, PATH_MFMA, 2, ASRC_LDS) W4A16_SHAPES(X, PATH_MFMA, 2, ASRC_GLOBAL)              \
    W4A16_SHAPES(X, PATH_MFMA, 3, ASRC_LDS) W4A16_SHAPES(X, PATH_MFMA, 3, ASRC_GLOBAL)              \
    W4A16_SHAPES(X, PATH_MFMA, 4, ASRC_LDS) W4A16_SHAPES(X, PATH_MFMA, 4, ASRC_GLOBAL)

// kVariantsPlain: plain matmuls; kVariantsEpi: the same shapes with the
// epilogue modes.  Both tables list the shapes in W4A16_VARIANT_LIST order.
extern const Variant kVariantsPlain[];
extern const Variant kVariantsEpi[];
extern const int kNumVariants;

}  // namespace w4a16
