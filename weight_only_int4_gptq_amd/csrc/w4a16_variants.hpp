// The compiled kernel shapes of the W4A16 matmul, shared by the
// instantiation units (variants_*.hip) and the host code that picks a kernel
// for a plan.
#pragma once

#include "w4a16_kernels.hpp"

namespace w4a16 {

using KernelFn = void (*)(GemmArgs);

struct Variant {
    int path, mm, tiles, kwaves, depth, asrc;   // mm: compile-time row count (0: run time;
                                                // < 0: run time, ceil(M/4) = -mm)
    KernelFn fn;
};

// (tiles, kwaves, depth) shapes instantiated for every path / row count
#define W4A16_SHAPES(X, P, MM, AS) \
    X(P, MM, 1, 1, 8, AS) X(P, MM, 1, 4, 8, AS) X(P, MM, 1, 8, 4, AS) X(P, MM, 1, 8, 8, AS) \
    X(P, MM, 2, 4, 4, AS) X(P, MM, 2, 8, 4, AS) X(P, MM, 2, 4, 8, AS) X(P, MM, 4, 4, 2, AS) \
    X(P, MM, 4, 4, 4, AS)

// A streamed per group through a per-wavefront LDS ring (matrix-core path);
// the two-tile depth-2 shapes are compiled only with their DMA count fixed
// (W4A16_RINGS_ND, one kernel per ceil(M/4))
#define W4A16_RINGS(X, P, MM, AS) \
    X(P, MM, 1, 4, 4, AS) X(P, MM, 1, 8, 4, AS) X(P, MM, 2, 4, 4, AS) \
    X(P, MM, 4, 4, 2, AS) X(P, MM, 4, 2, 2, AS) X(P, MM, 4, 4, 4, AS) X(P, MM, 8, 1, 4, AS) \
    X(P, MM, 8, 2, 2, AS) X(P, MM, 8, 4, 2, AS) X(P, MM, 1, 8, 2, AS)

// eight-tile strips: A read once per eight tiles (matrix-core paths)
#define W4A16_WIDE(X, P, MM, AS) \
    X(P, MM, 8, 4, 2, AS) X(P, MM, 8, 2, 2, AS) X(P, MM, 8, 2, 4, AS) X(P, MM, 8, 1, 4, AS)

// deeper rings for one row: a wavefront's groups in one or few rounds
#define W4A16_ONESHOT(X, P, MM, AS) \
    X(P, MM, 2, 4, 10, AS) X(P, MM, 2, 4, 5, AS) X(P, MM, 4, 4, 5, AS) X(P, MM, 4, 8, 5, AS) \
    X(P, MM, 1, 4, 10, AS) X(P, MM, 2, 2, 10, AS) X(P, MM, 4, 2, 5, AS) X(P, MM, 1, 8, 17, AS) \
    X(P, MM, 2, 8, 17, AS) X(P, MM, 2, 4, 17, AS) X(P, MM, 4, 4, 10, AS) X(P, MM, 2, 2, 17, AS)

// Kernels with compile-time rows (GEMV, and matrix-core kernels for one to
// four rows) and kernels that take the row count at run time (matrix cores,
// five rows and more, and ring A) sit in separate instantiation units,
// compiled with different register choices for the matrix-core results
// (build.py).

// more wavefronts per SIMD for one row: shallow rings, eight or sixteen along K
#define W4A16_MANYWAVE(X, P, MM, AS) \
    X(P, MM, 2, 8, 2, AS) X(P, MM, 2, 8, 3, AS) X(P, MM, 4, 8, 2, AS) X(P, MM, 2, 16, 2, AS) \
    X(P, MM, 1, 16, 2, AS) X(P, MM, 4, 4, 3, AS) X(P, MM, 2, 8, 5, AS) X(P, MM, 1, 8, 2, AS)

// The compile-time-row list in three parts, one instantiation unit each (the
// units compile in parallel): GEMV kernels, matrix-core kernels for one or
// two rows, and matrix-core kernels for three or four rows.
#define W4A16_VARIANT_LIST_CT_GEMV(X)                                                               \
    W4A16_MANYWAVE(X, PATH_GEMV, 1, ASRC_LDS) W4A16_ONESHOT(X, PATH_GEMV, 1, ASRC_LDS)              \
    W4A16_SHAPES(X, PATH_GEMV, 1, ASRC_LDS) W4A16_SHAPES(X, PATH_GEMV, 2, ASRC_LDS)                 \
    W4A16_SHAPES(X, PATH_GEMV, 3, ASRC_LDS) W4A16_SHAPES(X, PATH_GEMV, 4, ASRC_LDS)
#define W4A16_VARIANT_LIST_CT_MFMA12(X)                                                             \
    W4A16_ONESHOT(X, PATH_MFMA, 1, ASRC_LDS) W4A16_ONESHOT(X, PATH_MFMA, 1, ASRC_GLOBAL)            \
    W4A16_WIDE(X, PATH_MFMA, 2, ASRC_LDS)                                                           \
    W4A16_SHAPES(X, PATH_MFMA, 1, ASRC_LDS) W4A16_SHAPES(X, PATH_MFMA, 1, ASRC_GLOBAL)              \
    W4A16_SHAPES(X, PATH_MFMA, 2, ASRC_LDS) W4A16_SHAPES(X, PATH_MFMA, 2, ASRC_GLOBAL)
#define W4A16_VARIANT_LIST_CT_MFMA34(X)                                                             \
    W4A16_WIDE(X, PATH_MFMA, 3, ASRC_LDS) W4A16_WIDE(X, PATH_MFMA, 4, ASRC_LDS)                     \
    W4A16_SHAPES(X, PATH_MFMA, 3, ASRC_LDS) W4A16_SHAPES(X, PATH_MFMA, 3, ASRC_GLOBAL)              \
    W4A16_SHAPES(X, PATH_MFMA, 4, ASRC_LDS) W4A16_SHAPES(X, PATH_MFMA, 4, ASRC_GLOBAL)
// four wavefronts splitting the columns around one shared ring of A
#define W4A16_SPLITN(X, P, MM, AS) \
    X(P, MM, 1, 4, 2, AS) X(P, MM, 1, 4, 4, AS) X(P, MM, 2, 4, 2, AS) X(P, MM, 2, 4, 3, AS) \
    X(P, MM, 2, 4, 4, AS) X(P, MM, 4, 4, 2, AS)

// rings of depth 2 with the DMA count per group fixed (MM = -ceil(M/4)):
// every two-tile one, and one tile for 9..12 rows (measured faster; the
// one-tile depth-4 ring measured slower with its count fixed)
#define W4A16_RINGS_ND(X, P, AS) \
    X(P, -1, 2, 8, 2, AS) X(P, -2, 2, 8, 2, AS) X(P, -3, 2, 8, 2, AS) X(P, -4, 2, 8, 2, AS) \
    X(P, -1, 2, 4, 2, AS) X(P, -2, 2, 4, 2, AS) X(P, -3, 2, 4, 2, AS) X(P, -4, 2, 4, 2, AS) \
    X(P, -3, 1, 8, 2, AS)

#define W4A16_VARIANT_LIST_RT(X)                                                                    \
    W4A16_RINGS(X, PATH_MFMA, 0, ASRC_RING) W4A16_SPLITN(X, PATH_MFMA, 0, ASRC_SPLITN)             \
    W4A16_RINGS_ND(X, PATH_MFMA, ASRC_RING)                                                         \
    W4A16_WIDE(X, PATH_MFMA, 0, ASRC_LDS) W4A16_WIDE(X, PATH_MFMA, 0, ASRC_GLOBAL)                  \
    W4A16_SHAPES(X, PATH_MFMA, 0, ASRC_LDS) W4A16_SHAPES(X, PATH_MFMA, 0, ASRC_GLOBAL)

// Kernel tables, one per instantiation unit: plain matmuls and kernels that
// also carry the epilogue modes, each in the three compile-time-row parts
// and one run-time-row (Rt) table.
struct VariantTable {
    const Variant *v;
    int n;
};
extern const Variant kVariantsPlainGemv[], kVariantsPlainMfma12[], kVariantsPlainMfma34[], kVariantsPlainRt[];
extern const Variant kVariantsEpiGemv[], kVariantsEpiMfma12[], kVariantsEpiMfma34[], kVariantsEpiRt[];
extern const int kNumPlainGemv, kNumPlainMfma12, kNumPlainMfma34, kNumPlainRt;
extern const int kNumEpiGemv, kNumEpiMfma12, kNumEpiMfma34, kNumEpiRt;

// NVFP4 weight-only kernels (one table plain, one with the epilogue modes;
// A staged in LDS, read from global memory or through the LDS ring): the
// GEMV path for one to four rows, the matrix-core path for every row count.
#define W4A16_NV_GEMV(X, MM) \
    X(PATH_GEMV, MM, 1, 1, 8, ASRC_LDS) X(PATH_GEMV, MM, 1, 8, 4, ASRC_LDS) X(PATH_GEMV, MM, 2, 4, 4, ASRC_LDS) \
    X(PATH_GEMV, MM, 2, 8, 4, ASRC_LDS) X(PATH_GEMV, MM, 1, 4, 8, ASRC_LDS) X(PATH_GEMV, MM, 4, 4, 2, ASRC_LDS)
#define W4A16_NV_MFMA(X, MM, AS) \
    X(PATH_MFMA, MM, 1, 1, 8, AS) X(PATH_MFMA, MM, 1, 8, 4, AS) X(PATH_MFMA, MM, 2, 4, 4, AS) \
    X(PATH_MFMA, MM, 2, 8, 4, AS) X(PATH_MFMA, MM, 4, 4, 2, AS) X(PATH_MFMA, MM, 1, 4, 8, AS)
// in two parts, one unit each: the GEMV kernels and the matrix-core kernels
#define W4A16_NV_VARIANT_LIST_GEMV(X)                                                             \
    W4A16_NV_GEMV(X, 1) W4A16_NV_GEMV(X, 2) W4A16_NV_GEMV(X, 3) W4A16_NV_GEMV(X, 4)               \
    X(PATH_GEMV, 1, 2, 4, 5, ASRC_LDS) X(PATH_GEMV, 1, 1, 4, 10, ASRC_LDS)                         \
    X(PATH_GEMV, 1, 2, 8, 2, ASRC_LDS) X(PATH_GEMV, 1, 2, 2, 8, ASRC_LDS)                           \
    X(PATH_GEMV, 1, 1, 8, 2, ASRC_LDS) X(PATH_GEMV, 1, 1, 8, 3, ASRC_LDS)                           \
    X(PATH_GEMV, 1, 1, 16, 2, ASRC_LDS) X(PATH_GEMV, 1, 2, 8, 3, ASRC_LDS)
#define W4A16_NV_VARIANT_LIST_MFMA(X)                                                             \
    W4A16_NV_MFMA(X, 0, ASRC_LDS) W4A16_NV_MFMA(X, 0, ASRC_GLOBAL)                                 \
    X(PATH_MFMA, 0, 8, 1, 4, ASRC_GLOBAL) X(PATH_MFMA, 0, 8, 2, 2, ASRC_GLOBAL)                    \
    X(PATH_MFMA, 0, 8, 1, 2, ASRC_GLOBAL) X(PATH_MFMA, 0, 8, 1, 3, ASRC_GLOBAL)                    \
    X(PATH_MFMA, 0, 2, 4, 2, ASRC_RING) X(PATH_MFMA, 0, 2, 4, 4, ASRC_RING)                        \
    X(PATH_MFMA, 0, 4, 4, 2, ASRC_RING) X(PATH_MFMA, 0, 4, 2, 2, ASRC_RING)                        \
    X(PATH_MFMA, 0, 2, 4, 2, ASRC_SPLITN) X(PATH_MFMA, 0, 2, 4, 4, ASRC_SPLITN)                    \
    X(PATH_MFMA, 0, 1, 4, 4, ASRC_SPLITN) X(PATH_MFMA, 0, 4, 4, 2, ASRC_SPLITN)                    \
    W4A16_NV_MFMA(X, 1, ASRC_LDS) W4A16_NV_MFMA(X, 2, ASRC_LDS) W4A16_NV_MFMA(X, 3, ASRC_LDS)     \
    W4A16_NV_MFMA(X, 4, ASRC_LDS) W4A16_NV_MFMA(X, 2, ASRC_GLOBAL) W4A16_NV_MFMA(X, 4, ASRC_GLOBAL)

// W4A16_VARIANT_SUBSET: a handful of shapes per table instead of all of
// them, for quick builds of the host side under the address and
// undefined-behaviour sanitizers (the planner then falls back where a shape
// is missing; the library itself is always built with every shape).
#ifdef W4A16_VARIANT_SUBSET
#undef W4A16_VARIANT_LIST_CT_GEMV
#undef W4A16_VARIANT_LIST_CT_MFMA12
#undef W4A16_VARIANT_LIST_CT_MFMA34
#undef W4A16_VARIANT_LIST_RT
#undef W4A16_NV_VARIANT_LIST_GEMV
#undef W4A16_NV_VARIANT_LIST_MFMA
#define W4A16_VARIANT_LIST_CT_GEMV(X) X(PATH_GEMV, 1, 1, 8, 2, ASRC_LDS)
#define W4A16_VARIANT_LIST_CT_MFMA12(X) X(PATH_MFMA, 2, 2, 4, 4, ASRC_LDS)
#define W4A16_VARIANT_LIST_CT_MFMA34(X) X(PATH_MFMA, 4, 2, 4, 4, ASRC_LDS)
#define W4A16_VARIANT_LIST_RT(X) X(PATH_MFMA, 0, 2, 4, 2, ASRC_RING) X(PATH_MFMA, 0, 2, 4, 4, ASRC_LDS)
#define W4A16_NV_VARIANT_LIST_GEMV(X) X(PATH_GEMV, 1, 1, 8, 2, ASRC_LDS)
#define W4A16_NV_VARIANT_LIST_MFMA(X) X(PATH_MFMA, 0, 2, 4, 2, ASRC_RING)
#endif

// plain, and with the epilogue modes; GEMV and matrix-core parts
extern const Variant kVariantsNvGemv[], kVariantsNvMfma[], kVariantsNvEpiGemv[], kVariantsNvEpiMfma[];
extern const int kNumNvGemv, kNumNvMfma, kNumNvEpiGemv, kNumNvEpiMfma;

}  // namespace w4a16
