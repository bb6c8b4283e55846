// C ABI, argument checks and row-count dispatcher of the W4A16 library.
//
// The backbone and output-projection matmuls of the decode engine described on
// the page "Qwen3.8-27B on single DGX Spark ..." (section "How.") are
// dispatched by row count; here the row count M picks between a VALU path
// (v_dot2_f32_bf16 with a cross-lane reduction) and a matrix-core path
// (v_mfma_f32_16x16x32_bf16), and (M, N, K) pick the work decomposition.
// Everything is launched on the caller's stream; nothing is allocated.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "w4a16.h"
#include "w4a16_kernels.hpp"
#include "w4a16_variants.hpp"

namespace {

using namespace w4a16;

constexpr int kLdsBudget = 64 * 1024;    // automatic GEMV plans: at least two workgroups per CU
constexpr int kLdsMax = 160 * 1024;      // explicit plans: gfx950's LDS per workgroup
constexpr int kMaxVariants = 2048;       // bound on the kernel count over all tables (checked before use)
constexpr int kPlanCUs = 256;            // CUs the plans are balanced for (MI355X)

// ---------------------------------------------------------------- kernel table
// Two instantiations of every kernel shape (w4a16_variants.hpp): plain
// matmuls, and kernels that also carry the epilogue modes (gate/up
// activation, row argmax, fp32 output), compiled in their own translation
// units.  The plain ones have no mode code at all.

int default_depth(int tiles) { return tiles == 1 ? 8 : (tiles == 2 ? 4 : 2); }

// The kernel for a plan: GEMV kernels are compiled per row count (1..4);
// MFMA kernels too for M <= 4 (LDS or global A), and take M at run time
// above and with ring A.
// epi: a kernel that carries the epilogue modes (else a plain matmul);
// fmt: the weight format
const Variant *find_variant(const w4a16_plan_t &p, int M, bool epi = false, int fmt = FMT_GPTQ) {
    // ring and split-N kernels take M at run time for every row count
    const int mm = (p.path == W4A16_PATH_GEMV ||
                    (M <= 4 && p.asrc != W4A16_ASRC_RING && p.asrc != W4A16_ASRC_SPLITN))
                       ? M
                       : 0;
    const int asrc = (p.path == W4A16_PATH_GEMV) ? ASRC_LDS : p.asrc;
    const int depth = p.depth ? p.depth : default_depth(p.tiles);
    const VariantTable plain[] = {{kVariantsPlainGemv, kNumPlainGemv}, {kVariantsPlainMfma12, kNumPlainMfma12},
                                  {kVariantsPlainMfma34, kNumPlainMfma34}, {kVariantsPlainRt, kNumPlainRt}};
    const VariantTable with_epi[] = {{kVariantsEpiGemv, kNumEpiGemv}, {kVariantsEpiMfma12, kNumEpiMfma12},
                                     {kVariantsEpiMfma34, kNumEpiMfma34}, {kVariantsEpiRt, kNumEpiRt}};
    const VariantTable nv[] = {{kVariantsNvGemv, kNumNvGemv}, {kVariantsNvMfma, kNumNvMfma}};
    const VariantTable nv_epi[] = {{kVariantsNvEpiGemv, kNumNvEpiGemv}, {kVariantsNvEpiMfma, kNumNvEpiMfma}};
    const VariantTable *tabs = fmt == FMT_NVFP4 ? (epi ? nv_epi : nv) : (epi ? with_epi : plain);
    const int ntabs = fmt == FMT_NVFP4 ? 2 : 4;
    auto find = [&](int want_mm) -> const Variant * {
        for (int ti = 0; ti < ntabs; ++ti)
            for (int i = 0; i < tabs[ti].n; ++i) {
                const Variant &v = tabs[ti].v[i];
                if (v.path == p.path && v.mm == want_mm && v.tiles == p.tiles && v.kwaves == p.kwaves &&
                    v.depth == depth && v.asrc == asrc)
                    return &v;
            }
        return nullptr;
    };
    // ring A: the kernel with this M's DMA count per group fixed, if compiled
    if (p.path == W4A16_PATH_MFMA && asrc == ASRC_RING)
        if (const Variant *v = find(-((M + 3) / 4))) return v;
    return find(mm);
}

// A dense index of a kernel over every table (for per-kernel host caches), or
// -1 if it is in none.
int variant_slot(const Variant *v) {
    const VariantTable tabs[] = {{kVariantsPlainGemv, kNumPlainGemv},   {kVariantsPlainMfma12, kNumPlainMfma12},
                                 {kVariantsPlainMfma34, kNumPlainMfma34}, {kVariantsPlainRt, kNumPlainRt},
                                 {kVariantsEpiGemv, kNumEpiGemv},       {kVariantsEpiMfma12, kNumEpiMfma12},
                                 {kVariantsEpiMfma34, kNumEpiMfma34},   {kVariantsEpiRt, kNumEpiRt},
                                 {kVariantsNvGemv, kNumNvGemv},         {kVariantsNvMfma, kNumNvMfma},
                                 {kVariantsNvEpiGemv, kNumNvEpiGemv},   {kVariantsNvEpiMfma, kNumNvEpiMfma}};
    int base = 0;
    for (const VariantTable &t : tabs) {
        if (v >= t.v && v < t.v + t.n) return base + (int)(v - t.v);
        base += t.n;
    }
    return -1;
}

// ---------------------------------------------------------------- checks

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_shape(int M, int N, int K) {
    if (M < 1 || M > W4A16_MAX_M) return W4A16_ERR_SHAPE;
    if (K <= 0 || (K % W4A16_GROUP) != 0 || K > W4A16_MAX_K) return W4A16_ERR_SHAPE;
    if (N <= 0 || (N % 16) != 0) return W4A16_ERR_SHAPE;
    if ((unsigned long long)K * (unsigned long long)N / 2ull >= (1ull << 40)) return W4A16_ERR_SHAPE;
    // the scales [K/128][N] are addressed with 32-bit byte offsets
    if ((unsigned long long)(K / W4A16_GROUP) * (unsigned long long)N * 2ull >= (1ull << 31)) return W4A16_ERR_SHAPE;
    return W4A16_OK;
}

int check_weight_shape(int K, int N) { return check_shape(1, N, K); }

// Current device must be a gfx950; answers are cached per device id.
// Current device: W4A16_OK if it is a gfx950, with its LDS bytes per
// workgroup in *lds_max (cached per device).
int check_device(int *lds_max = nullptr) {
    static std::atomic<int> cache[64];   // 0 unknown, -1 not gfx950, else LDS bytes per workgroup
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return W4A16_ERR_DEVICE;
    if (dev >= 64) return W4A16_ERR_DEVICE;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess ||
            std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
            v = -1;
        else
            v = (int)prop.sharedMemPerBlock > 0 ? (int)prop.sharedMemPerBlock : 65536;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    if (v < 0) return W4A16_ERR_DEVICE;
    if (lds_max) *lds_max = v;
    return W4A16_OK;
}

// ---------------------------------------------------------------- planning

// K groups of the widest workgroup K range of a plan
int plan_gwg(const w4a16_plan_t &p, int G) {
    return (p.splits > 1 && p.whole == 0) ? (G + p.splits - 1) / p.splits : G;
}

int plan_lds(const w4a16_plan_t &p, int M, int G) {
    const int Gwg = plan_gwg(p, G);
    const int asrc = (p.path == W4A16_PATH_GEMV) ? ASRC_LDS : p.asrc;
    const int depth = p.depth ? p.depth : default_depth(p.tiles);
    return lds_layout(p.path, asrc, M, Gwg, p.tiles, p.kwaves, depth).total;
}

// 16-column tiles of one workgroup's strip
long long strip_tiles(const w4a16_plan_t &p) {
    const bool splitn = p.path == W4A16_PATH_MFMA && p.asrc == W4A16_ASRC_SPLITN;
    return (long long)p.tiles * (splitn ? p.kwaves : 1);
}

int validate_plan(const w4a16_plan_t &p, int M, int N, int K, int fmt = FMT_GPTQ) {
    const int G = K / W4A16_GROUP;
    if (p.path != W4A16_PATH_GEMV && p.path != W4A16_PATH_MFMA) return W4A16_ERR_PLAN;
    if (p.path == W4A16_PATH_GEMV && M > 4) return W4A16_ERR_PLAN;
    if (p.splits < 1 || p.splits > G || (p.splits & (p.splits - 1)) != 0) return W4A16_ERR_PLAN;
    if (p.asrc != W4A16_ASRC_LDS && p.asrc != W4A16_ASRC_GLOBAL && p.asrc != W4A16_ASRC_RING &&
        p.asrc != W4A16_ASRC_SPLITN)
        return W4A16_ERR_PLAN;
    if (p.depth < 0) return W4A16_ERR_PLAN;
    if (!find_variant(p, M, false, fmt)) return W4A16_ERR_PLAN;
    if (plan_lds(p, M, G) + 256 > kLdsMax) return W4A16_ERR_PLAN;
    const long long nstrips = (N / 16 + strip_tiles(p) - 1) / strip_tiles(p);
    if (nstrips * p.splits >= (1ll << 31)) return W4A16_ERR_PLAN;
    if (p.whole < 0 || (p.splits > 1 && p.whole > nstrips)) return W4A16_ERR_PLAN;
    if (p.splits > 1 && nstrips > W4A16_SPLIT_COUNTER_BYTES / 4) return W4A16_ERR_PLAN;
    return W4A16_OK;
}

// The row-count dispatcher.  Plan choice, from graph-replayed timings of
// every compiled plan on MI355X (cold weights) over the decoder shapes
// K x N = 5120 x 8192, 6144 x 5120, 5120 x 34816, 17408 x 5120 and
// 5120 x 248320 and their tensor-parallel shards (N / 2, 4, 8 for the first
// and third, K / 2, 4, 8 for the second and fourth), M = 1..16.
// Widths: "narrow" up to 384 tiles of 16 columns, "mid" 513..2047, "wide"
// from 2048, "very wide" from 8192; "long" K from 128 groups of 128.
//  * M = 1: the GEMV kernel; eight wavefronts with a ring of depth 2 and one
//    tile per strip almost everywhere (two wavefronts or more per SIMD);
//    two tiles for the attention output and QKV (257..512 tiles, 32..63
//    groups);
//    two tiles, four wavefronts, depth 4 below 16 groups; the very wide
//    output head keeps two tiles, four wavefronts, depth 5;
//  * M = 2..4: matrix cores; long K: the whole K range of A staged in LDS,
//    two tiles, eight wavefronts; very wide N: four tiles, depth 2, A in
//    LDS (the ring with two wavefronts at M = 2); wide and mid N: A through
//    the per-wavefront LDS ring, two tiles, depth 2; narrow N from 16
//    groups: A in LDS, eight wavefronts, depth 4, one tile (two from 64
//    groups); otherwise A in LDS, two tiles, depth 4;
//  * M >= 5, matrix cores:
//      - very wide N: four wavefronts split the columns (two tiles each up
//        to 8 rows, four above) around one shared ring of A, depth 2;
//      - wide N from 32 groups: the same with one tile each (two above 8
//        rows), depth 4, the strips beyond a whole number per CU split four
//        ways along K;
//      - mid N: A through the ring, two tiles, depth 2, with the same
//        remainder split;
//      - long K: A through the ring from M = 8; below, a quarter of K of A
//        staged in LDS (split four ways);
//      - narrow N up to 256 tiles: one tile, eight wavefronts, A in LDS up
//        to 7 rows, through the ring above;
//      - narrow N with 8..31 groups: A through the ring, two tiles, depth 4;
//      - otherwise two tiles: all of A in LDS up to 7 rows and from 64
//        groups (depth 4, eight wavefronts from 64 groups), A through the
//        ring otherwise (depth 2; depth 4 for narrow N from 32 groups).
//  Three rules override these (below): the QKV and attention-output widths,
//  the remainder split of narrow N with long K, and split-N with K pieces
//  for narrow N with long K from 13 rows.  Staged A that does
//  not fit in LDS goes through the ring with four wavefronts.
void auto_plan(int M, int N, int K, w4a16_plan_t *out) {
    const int NT = N / 16, G = K / W4A16_GROUP;
    const bool wide = NT >= 2048, vwide = NT >= 8192, deep = G >= 128;
    const bool narrow = NT <= 384;             // few strips: one tile each, more waves along K
    const bool mid = NT > 512 && NT < 2048;    // between the QKV and gate/up widths
    w4a16_plan_t p{};
    p.kwaves = 4;
    p.splits = 1;
    p.asrc = W4A16_ASRC_LDS;
    if (M == 1) {
        // eight wavefronts with shallow rings below the gate/up width: two
        // wavefronts per SIMD, one's dequantization overlaps the other's wait
        p.path = W4A16_PATH_GEMV;
        p.kwaves = 8;
        if (wide && !vwide && !deep) {         // gate/up width: one tile, eight shallow wavefronts
            p.tiles = 1;
            p.depth = 2;
        } else if (wide) {
            p.tiles = 2;
            p.kwaves = deep ? 8 : 4;
            p.depth = deep ? 4 : 5;
        } else if (NT > 256 && NT <= 512 && G >= 32 && G < 64) {   // attention out, QKV: two tiles, shallow
            p.tiles = 2;
            p.depth = 2;
        } else if (G >= 16) {                  // one tile, eight shallow wavefronts
            p.tiles = 1;
            p.depth = 2;
        } else {                               // few groups: two tiles, four wavefronts
            p.tiles = 2;
            p.kwaves = 4;
            p.depth = 4;
        }
    } else if (M <= 4) {
        p.path = W4A16_PATH_MFMA;
        if (deep && !wide) {                   // the whole long K range of A in LDS
            p.tiles = 2;
            p.kwaves = 8;
            p.depth = 4;
        } else if (vwide) {
            p.tiles = 4;
            p.depth = 2;
            if (M == 2) {                      // A through the ring, two wavefronts
                p.asrc = W4A16_ASRC_RING;
                p.kwaves = 2;
            }
        } else if (wide || mid) {              // A through the ring, shallow
            p.asrc = W4A16_ASRC_RING;
            p.tiles = 2;
            p.depth = 2;
        } else if (narrow && G >= 16) {        // eight wavefronts (two per SIMD): one tile, two from 64 groups
            p.tiles = G >= 64 ? 2 : 1;
            p.kwaves = 8;
            p.depth = 4;
        } else {
            p.tiles = 2;
            p.depth = 4;
        }
    } else {
        p.path = W4A16_PATH_MFMA;
        if (vwide) {                           // four wavefronts split 8 (16 above 8 rows) tiles, shared A
            p.asrc = W4A16_ASRC_SPLITN;
            p.tiles = M <= 8 ? 2 : 4;
            p.depth = 2;
        } else if (wide && G >= 32) {          // four wavefronts split 4 (8 above 8 rows) tiles, shared A
            p.asrc = W4A16_ASRC_SPLITN;
            p.tiles = M <= 8 ? 1 : 2;
            p.depth = 4;
            // strips beyond a whole number per CU: split four ways along K
            const int ns = (NT + 4 * p.tiles - 1) / (4 * p.tiles), R = ns % kPlanCUs;
            if (ns > kPlanCUs && R != 0 && 4 * R <= kPlanCUs) {
                p.splits = 4;
                p.whole = ns - R;
            }
        } else if (wide && M >= 9) {           // four wavefronts split 4 tiles, shared A, depth 4
            p.asrc = W4A16_ASRC_SPLITN;
            p.tiles = 1;
            p.depth = 4;
        } else if (wide) {                     // A through the ring: two tiles up to 8 rows, four above
            p.asrc = W4A16_ASRC_RING;
            p.tiles = M <= 8 ? 2 : 4;
            p.depth = 2;
        } else if (mid) {                      // A through the ring, two tiles; strips beyond a whole
            p.asrc = W4A16_ASRC_RING;          // number per CU split four ways along K
            p.tiles = 2;
            p.depth = 2;
            const int ns = (NT + 1) / 2, R = ns % kPlanCUs;
            if (ns > kPlanCUs && R != 0 && 4 * R <= kPlanCUs && G >= 32) {
                p.splits = 4;
                p.whole = ns - R;
            }
        } else if (deep) {
            p.tiles = 2;
            p.depth = 4;
            if (M >= 8) {
                p.asrc = W4A16_ASRC_RING;
            } else {                           // a quarter of K of A in LDS
                p.asrc = W4A16_ASRC_LDS;
                p.splits = 4;
            }
        } else if (narrow && NT <= 256) {      // one tile, eight wavefronts: A in LDS to 7 rows, the ring above
            p.tiles = 1;
            p.kwaves = 8;
            p.depth = 4;
            if (M >= 8) p.asrc = W4A16_ASRC_RING;
        } else if (narrow && G >= 8 && G < 32) {    // 8-31 groups: two tiles, ring A, depth 4
            p.asrc = W4A16_ASRC_RING;
            p.tiles = 2;
            p.depth = 4;
        } else if (M <= 7 || G >= 64) {       // all of A in LDS (eight wavefronts from 64 groups)
            p.tiles = 2;
            p.depth = 4;
            if (G >= 64) p.kwaves = 8;
        } else {                               // A through the ring (depth 4 for narrow N from 32 groups)
            p.asrc = W4A16_ASRC_RING;
            p.tiles = 2;
            p.depth = (narrow && G >= 32) ? 4 : 2;
        }
    }
    // Between one and two strips of two tiles per CU with 32 to 127 groups
    // (the attention output projection 6144 x 5120 and QKV 5120 x 8192):
    // two tiles, eight wavefronts (two per SIMD), A through the ring, depth 2
    // (its kernels with the DMA count fixed beat A staged whole in LDS from
    // two rows).
    if (M >= 2 && NT > kPlanCUs && NT <= 2 * kPlanCUs && G >= 32 && !deep) {
        p.path = W4A16_PATH_MFMA;
        p.asrc = W4A16_ASRC_RING;
        p.tiles = 2;
        p.kwaves = 8;
        p.depth = 2;
        p.splits = 1;
        p.whole = 0;
    }
    // Narrow N with long K, one row, from three rows with 128 groups and
    // more, or from five rows with 64: one tile per strip, eight wavefronts
    // along K, and the strips beyond one per CU split into K pieces, so that
    // every CU gets one whole strip and one piece (17408 x 5120: 256 whole
    // strips and 64 strips in four pieces).  The pieces' hand-off finishes
    // long before the whole strips do.  Ring depth 4 up to 8 rows with 128
    // groups (slots of one or two KiB), 2 otherwise.  (Two rows, and three
    // and four below 128 groups, keep the whole K range of A in LDS.)
    if (narrow && (M == 1 ? deep : (deep ? M >= 3 : (M >= 5 && G >= 64))) && NT > kPlanCUs &&
        NT % kPlanCUs != 0) {
        const int R = NT % kPlanCUs;
        int S = 1;
        while (S * 2 * R <= kPlanCUs && S * 2 <= G / 16) S *= 2;
        if (S >= 2) {
            p.path = (M == 1) ? W4A16_PATH_GEMV : W4A16_PATH_MFMA;
            p.asrc = (M == 1) ? W4A16_ASRC_LDS : W4A16_ASRC_RING;
            p.tiles = 1;
            p.kwaves = 8;
            p.depth = (deep && M >= 3 && M <= 8) ? 4 : 2;
            p.splits = S;
            p.whole = NT - R;
        }
    }
    // Narrow N with long K from 13 rows: four wavefronts split four
    // one-tile columns around one shared ring of A (a quarter of the A
    // traffic of the per-wavefront ring), every strip split along K into
    // pieces of at least 16 groups, at most eight (17408 x 5120: 80 strips
    // in eight pieces of 17 groups).
    if (narrow && deep && M >= 13) {
        p.path = W4A16_PATH_MFMA;
        p.asrc = W4A16_ASRC_SPLITN;
        p.tiles = 1;
        p.kwaves = 4;
        p.depth = 4;
        p.splits = 1;
        while (p.splits < 8 && G / (p.splits * 2) >= 16) p.splits *= 2;
        p.whole = 0;
    }
    // short K: no more wavefronts along K than groups per workgroup
    // (split-N wavefronts split the columns)
    if (p.asrc != W4A16_ASRC_SPLITN && p.kwaves * p.splits > G) {
        p.splits = 1;
        if (p.kwaves > G) {
            if (G >= 4) {
                p.kwaves = 4;
                p.depth = 0;
            } else {
                p.tiles = 1;
                p.kwaves = 1;
                p.depth = 8;
            }
        }
    }
    if (p.path == W4A16_PATH_GEMV && plan_lds(p, M, G) > kLdsBudget) {
        p.path = W4A16_PATH_MFMA;
        p.depth = 0;
    }
    // staged A may take a whole workgroup's LDS (one workgroup per CU);
    // beyond that A streams through the ring
    if (p.path == W4A16_PATH_MFMA && p.asrc == W4A16_ASRC_LDS && plan_lds(p, M, G) + 256 > kLdsMax) {
        p.asrc = M >= 5 ? W4A16_ASRC_RING : W4A16_ASRC_GLOBAL;
        p.splits = 1;
        if (p.asrc == W4A16_ASRC_RING) p.kwaves = 4;   // the ring measures best with four
    }
    // ring A has fewer compiled shapes (none for the short-K fallback)
    if (p.asrc == W4A16_ASRC_RING && !find_variant(p, M)) p.asrc = W4A16_ASRC_GLOBAL;
    *out = p;
}

// NVFP4 plans, from graph-replayed timings of every compiled NVFP4 plan on
// MI355X (cold weights) over the decoder shapes, M = 1..16.  The matrix-core
// path pays one scale multiply per 16-row block and output, so it wins later
// than for GPTQ on narrow N and favours split K for long K:
//  * M = 1, GEMV: the gate/up width: one tile, eight wavefronts, depth 2;
//    other wide N: two tiles, four wavefronts, depth 5; narrow N with long
//    K (the down projection): one tile, eight wavefronts, the strips beyond
//    one per CU split four ways along K; other long K: two tiles, eight
//    wavefronts, depth 3; otherwise one tile, eight wavefronts, depth 2;
//  * M = 2 on the down projection: the same remainder split with matrix
//    cores, A in LDS, depth 4;
//  * M = 2..4, A in LDS: very wide N: four tiles, depth 2; long K: two
//    tiles, eight wavefronts; the gate/up width: four tiles, four
//    wavefronts, depth 2, the strips beyond a whole number per CU split
//    eight ways along K; otherwise one tile, eight wavefronts;
//  * M >= 5: very wide N: four wavefronts split the columns (two tiles
//    each) around one shared ring of A, depth 2; wide N: the same with one
//    tile each, depth 4, the strips beyond a whole number per CU split four
//    ways along K; narrow N with long K: the same with every strip in eight
//    K pieces; other long K: four tiles split four ways with A in LDS up to
//    7 rows, from 8 the ring (two tiles, split two ways); fewer than 64
//    groups up to 6 rows (the QKV and attention-out widths): one tile,
//    eight wavefronts, A in LDS, depth 4; narrow N up to 8 rows: the same
//    with two tiles from 64 groups or past 256 tiles; otherwise two tiles,
//    eight wavefronts, A in LDS up to 7 rows, and from 8 rows the ring, two
//    tiles, four wavefronts, depth 2 (4 for narrow N from 64 groups).
// The first of these that the library has a kernel for and that fits is taken, else
// the first compiled fallback.
void auto_plan_nv(int M, int N, int K, w4a16_plan_t *out) {
    const int NT = N / 16, G = K / W4A16_GROUP;
    const bool wide = NT >= 2048, vwide = NT >= 8192, deep = G >= 128, narrow = NT <= 384;
    w4a16_plan_t p{};
    p.path = W4A16_PATH_MFMA;
    p.tiles = 2;
    p.kwaves = 4;
    p.splits = 1;
    p.asrc = W4A16_ASRC_LDS;
    p.depth = 4;
    auto set = [&](int path, int t, int kw, int s, int asrc, int d) {
        p.path = path, p.tiles = t, p.kwaves = kw, p.splits = s, p.asrc = asrc, p.depth = d;
    };
    // narrow N with long K and more one-tile strips than CUs (the down
    // projection): the strips beyond one per CU split four ways along K
    const int R = NT % kPlanCUs;
    const bool remainder = narrow && deep && NT > kPlanCUs && R != 0 && 4 * R <= kPlanCUs && G >= 64;
    if (M == 1) {
        if (wide && !vwide && !deep) set(W4A16_PATH_GEMV, 1, 8, 1, W4A16_ASRC_LDS, 2);
        else if (wide) set(W4A16_PATH_GEMV, 2, 4, 1, W4A16_ASRC_LDS, 5);
        else if (remainder) set(W4A16_PATH_GEMV, 1, 8, 4, W4A16_ASRC_LDS, 2), p.whole = NT - R;
        else if (deep) set(W4A16_PATH_GEMV, 2, 8, 1, W4A16_ASRC_LDS, 3);
        else set(W4A16_PATH_GEMV, 1, 8, 1, W4A16_ASRC_LDS, 2);
    } else if (M == 2 && remainder) {
        set(W4A16_PATH_MFMA, 1, 8, 4, W4A16_ASRC_LDS, 4);
        p.whole = NT - R;
    } else if (M <= 4) {
        if (vwide) set(W4A16_PATH_MFMA, 4, 4, 1, W4A16_ASRC_LDS, 2);
        else if (deep) set(W4A16_PATH_MFMA, 2, 8, 1, W4A16_ASRC_LDS, 4);
        else if (!wide) set(W4A16_PATH_MFMA, 1, 8, 1, W4A16_ASRC_LDS, 4);
        else {
            // the gate/up width: four-tile strips, the strips beyond a whole
            // number per CU split eight ways along K
            set(W4A16_PATH_MFMA, 4, 4, 1, W4A16_ASRC_LDS, 2);
            const int ns = (NT + 3) / 4, r = ns % kPlanCUs;
            if (ns > kPlanCUs && r != 0 && 8 * r <= kPlanCUs) {
                p.splits = 8;
                p.whole = ns - r;
            }
        }
    } else {
        // A through the LDS ring (two tiles, depth 2) wherever it measured
        // best; four wavefronts splitting the columns around one shared ring
        // for the widest N (and wide N from 9 rows)
        if (vwide) {
            set(W4A16_PATH_MFMA, 2, 4, 1, W4A16_ASRC_SPLITN, 2);
        } else if (wide) {
            // four wavefronts split 4 tiles around a shared ring; the
            // strips beyond a whole number per CU split four ways along K
            set(W4A16_PATH_MFMA, 1, 4, 1, W4A16_ASRC_SPLITN, 4);
            const int ns = (NT + 3) / 4, r = ns % kPlanCUs;
            if (G >= 32 && ns > kPlanCUs && r != 0 && 4 * r <= kPlanCUs) {
                p.splits = 4;
                p.whole = ns - r;
            }
        } else if (deep && narrow) {
            // four wavefronts split four one-tile columns around a shared
            // ring, every strip in eight K pieces
            set(W4A16_PATH_MFMA, 1, 4, 8, W4A16_ASRC_SPLITN, 4);
        } else if (deep) {
            if (M <= 7) set(W4A16_PATH_MFMA, 4, 4, 4, W4A16_ASRC_LDS, 2);
            else set(W4A16_PATH_MFMA, 2, 4, 2, W4A16_ASRC_RING, 2);
        } else if (M <= 6 && G < 64) {         // QKV and attention-out widths: one tile, eight wavefronts
            set(W4A16_PATH_MFMA, 1, 8, 1, W4A16_ASRC_LDS, 4);
        } else if (narrow && M <= 8) {         // one tile (two from 64 groups or past 256 tiles), eight wavefronts
            set(W4A16_PATH_MFMA, (G >= 64 || NT > kPlanCUs) ? 2 : 1, 8, 1, W4A16_ASRC_LDS, 4);
        } else if (M <= 7) {
            set(W4A16_PATH_MFMA, 2, 8, 1, W4A16_ASRC_LDS, 4);
        } else {
            set(W4A16_PATH_MFMA, 2, 4, 1, W4A16_ASRC_RING, (narrow && G >= 64) ? 4 : 2);
        }
    }
    // splits no larger than the groups allow (a power of two), and no more
    // wavefronts along K than each split's groups
    // (one row: up to two wavefronts per group, the idle ones finish at once)
    const int kwmax = (M == 1) ? 2 * G : G;
    while (p.splits > 1 && p.splits * p.kwaves > G) p.splits >>= 1;
    if (p.splits == 1) p.whole = 0;
    while (p.asrc != W4A16_ASRC_SPLITN && p.kwaves > 1 && p.kwaves > kwmax) p.kwaves >>= 1;
    // fallbacks: A from global memory; the LDS ring (its kernels take any
    // row count, so they also cover K ranges of A too long to stage); the
    // common shapes; the short-K shapes
    w4a16_plan_t cand[9] = {p, p, p, p, p, p, p, p, p};
    cand[1].asrc = W4A16_ASRC_GLOBAL;
    cand[2].path = W4A16_PATH_MFMA, cand[2].asrc = W4A16_ASRC_RING, cand[2].tiles = 2, cand[2].kwaves = 4;
    cand[2].depth = 2;
    cand[3] = cand[2], cand[3].splits = 1;
    cand[4].tiles = 2, cand[4].kwaves = 4, cand[4].depth = 4, cand[4].splits = 1;
    cand[5] = cand[4], cand[5].asrc = W4A16_ASRC_GLOBAL;
    cand[6] = cand[4], cand[6].path = M <= 4 ? W4A16_PATH_GEMV : W4A16_PATH_MFMA;
    cand[7].tiles = 1, cand[7].kwaves = 1, cand[7].depth = 8, cand[7].splits = 1, cand[7].asrc = W4A16_ASRC_LDS;
    cand[8] = cand[7], cand[8].path = W4A16_PATH_MFMA, cand[8].asrc = W4A16_ASRC_GLOBAL;
    for (const w4a16_plan_t &c : cand)
        if (validate_plan(c, M, N, K, FMT_NVFP4) == W4A16_OK) {
            *out = c;
            return;
        }
    *out = cand[3];
}

size_t workspace_for(const w4a16_plan_t &p, int M, int N) {
    if (p.splits <= 1) return 0;
    return (size_t)W4A16_SPLIT_COUNTER_BYTES + (size_t)p.splits * (size_t)M * (size_t)N * sizeof(float);
}

hipError_t launch(const void *fn, unsigned grid, unsigned block, size_t lds, hipStream_t stream,
                  void **args) {
    return hipLaunchKernel(fn, dim3(grid), dim3(block), args, lds, stream);
}

static_assert(kArgmaxBinOffset + kArgmaxBins * 16 * 8 <= W4A16_ARGMAX_WORKSPACE_BYTES &&
                  W4A16_ARGMAX_WORKSPACE_BYTES <= W4A16_SPLIT_COUNTER_BYTES,
              "argmax counter and bins live in the workspace's counter region");

// The gate/up epilogue needs strips of gate/up tile pairs: an even tile
// count.  The automatic plan is moved to two tiles when it has one.
void fuse_plan(int M, w4a16_plan_t *p, int fmt = FMT_GPTQ) {
    if (p->tiles % 2 == 0) return;
    w4a16_plan_t q = *p;
    if (q.whole > 0) {                         // the strip count changes with the tile count
        q.splits = 1;
        q.whole = 0;
    }
    if (q.asrc == W4A16_ASRC_SPLITN) {         // one-tile split-N: the ring plan of the same width
        q.asrc = W4A16_ASRC_RING;
        q.tiles = (fmt == FMT_GPTQ && M >= 9) ? 4 : 2;
        q.kwaves = 4;
        q.depth = 2;
    } else {
        q.tiles = 2;                           // same wavefronts and ring depth if compiled
    }
    if (!find_variant(q, M, true, fmt)) q.depth = 0;
    if (!find_variant(q, M, true, fmt)) q.kwaves = 4;
    if (!find_variant(q, M, true, fmt)) q.asrc = W4A16_ASRC_GLOBAL;
    if (!find_variant(q, M, true, fmt)) q.asrc = W4A16_ASRC_RING, q.depth = 2;
    *p = q;
}

// Workspace bytes that serve every call kind at (M, N, K) with its automatic
// plan: the plain and fp32-output calls, the gate/up call (N a multiple of
// 32) and the argmax call (the counter region alone).
size_t workspace_any_call(int M, int N, int K, int fmt) {
    if (check_shape(M, N, K) != W4A16_OK) return 0;
    w4a16_plan_t p{};
    if (fmt == FMT_NVFP4) auto_plan_nv(M, N, K, &p);
    else auto_plan(M, N, K, &p);
    size_t need = workspace_for(p, M, N);
    if (N % 32 == 0) {
        fuse_plan(M, &p, fmt);
        const size_t f = workspace_for(p, M, N);
        if (f > need) need = f;
    }
    return need > (size_t)W4A16_ARGMAX_WORKSPACE_BYTES ? need : (size_t)W4A16_ARGMAX_WORKSPACE_BYTES;
}

// fuse: 0 plain C[M][N]; 1 the gate/up epilogue, C is H[M][N/2]; 2 the row
// argmax (C unused, results in idx / val); 3 C as fp32 [M][N]
// fmt: FMT_GPTQ (group 128, bf16 scales) or FMT_NVFP4 (group 16, E4M3
// scales, alpha the per-tensor factor)
int run_gemm(const void *A, const void *wq, const void *scales, void *C, int M, int N, int K,
             int group, void *workspace, size_t workspace_bytes, const w4a16_plan_t *user,
             void *stream, int fuse = 0, int *idx = nullptr, float *val = nullptr,
             int fmt = FMT_GPTQ, float alpha = 1.0f) {
    if (!A || !wq || !scales) return W4A16_ERR_NULL;
    if (fuse == 2 ? (!idx || !val) : !C) return W4A16_ERR_NULL;
    int st = check_shape(M, N, K);
    if (st != W4A16_OK) return st;
    if (fuse == 1 && N % 32 != 0) return W4A16_ERR_SHAPE;
    if (group != (fmt == FMT_NVFP4 ? W4A16_NVFP4_GROUP : W4A16_GROUP)) return W4A16_ERR_GROUP;
    if (!aligned16(A) || !aligned16(wq) || !aligned16(scales) || (fuse != 2 && !aligned16(C)))
        return W4A16_ERR_ALIGN;
    if (fuse == 2 && (((uintptr_t)idx | (uintptr_t)val) & 3)) return W4A16_ERR_ALIGN;
    w4a16_plan_t p{};
    if (user) {
        p = *user;
        st = validate_plan(p, M, N, K, fmt);
        if (st != W4A16_OK) return st;
        if (fuse == 1 && p.tiles % 2 != 0) return W4A16_ERR_PLAN;
        if (fuse == 2 && p.splits != 1) return W4A16_ERR_PLAN;
        if (fuse != 0 && !find_variant(p, M, true, fmt)) return W4A16_ERR_PLAN;
    } else {
        if (fmt == FMT_NVFP4) auto_plan_nv(M, N, K, &p);
        else auto_plan(M, N, K, &p);
        if (fuse == 1) fuse_plan(M, &p, fmt);
        if (fuse == 2 && p.splits != 1) {
            p.splits = 1;
            if (validate_plan(p, M, N, K, fmt) != W4A16_OK) p.asrc = W4A16_ASRC_RING;
            if (validate_plan(p, M, N, K, fmt) != W4A16_OK) p.asrc = W4A16_ASRC_GLOBAL;
        }
    }
    const size_t need = fuse == 2 ? (size_t)W4A16_ARGMAX_WORKSPACE_BYTES : workspace_for(p, M, N);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return W4A16_ERR_WORKSPACE;
        if (!aligned16(workspace)) return W4A16_ERR_ALIGN;
    }
    const Variant *v = find_variant(p, M, fuse != 0, fmt);
    if (!v) return W4A16_ERR_PLAN;
    int lds_max = 0;
    st = check_device(&lds_max);
    if (st != W4A16_OK) return st;

    const int lds = plan_lds(p, M, K / W4A16_GROUP);
    if (lds + 256 > lds_max) return W4A16_ERR_PLAN;   // 256: the kernel's static LDS
    if (lds > 65536) {
        // above 64 KiB the kernel must be allowed its dynamic LDS first (once)
        static std::atomic<uint8_t> raised[kMaxVariants];
        const int vi = variant_slot(v);
        if (vi < 0 || vi >= kMaxVariants) return W4A16_ERR_LAUNCH;
        if (!raised[vi].load(std::memory_order_relaxed)) {
            const void *fn = reinterpret_cast<const void *>(v->fn);
            hipFuncAttributes fa;
            if (hipFuncGetAttributes(&fa, fn) != hipSuccess ||
                hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                    lds_max - (int)fa.sharedSizeBytes) != hipSuccess)
                return W4A16_ERR_LAUNCH;
            raised[vi].store(1, std::memory_order_relaxed);
        }
    }
    GemmArgs a;
    a.A = static_cast<const uint16_t *>(A);
    a.blob = static_cast<const u32x4 *>(wq);
    a.scales = static_cast<const uint16_t *>(scales);
    a.C = static_cast<uint16_t *>(C);
    a.M = M;
    a.N = N;
    a.K = K;
    a.G = K / W4A16_GROUP;
    a.S = p.splits;
    a.Slog2 = 0;
    while ((1 << a.Slog2) < a.S) ++a.Slog2;
    a.NT = N / 16;
    a.nstrips = (int)((a.NT + strip_tiles(p) - 1) / strip_tiles(p));
    a.nwhole = a.S > 1 ? p.whole : 0;
    a.nunits = a.nwhole + (a.nstrips - a.nwhole) * a.S;
    a.fuse = fuse;
    a.amax_idx = idx;
    a.amax_val = val;
    a.alpha = alpha;
    if (need > 0) {   // split-K partials or argmax bins: the counter region first
        a.count = static_cast<uint32_t *>(workspace);
        a.part = reinterpret_cast<float *>(static_cast<char *>(workspace) + W4A16_SPLIT_COUNTER_BYTES);
    } else {
        a.part = nullptr;
        a.count = nullptr;
    }
    void *args[] = {&a};
    hipError_t e = launch(reinterpret_cast<const void *>(v->fn), (unsigned)a.nunits,
                          64u * (unsigned)p.kwaves, (size_t)lds, static_cast<hipStream_t>(stream), args);
    if (e == hipSuccess && fuse == 2) {
        // fold the per-bin row maxima (stream order: after every atomic above)
        unsigned long long *bins = reinterpret_cast<unsigned long long *>(
            static_cast<char *>(workspace) + kArgmaxBinOffset);
        hipLaunchKernelGGL(argmax_fold_kernel, dim3(1), dim3(kArgmaxBins * 16), 0,
                           static_cast<hipStream_t>(stream), bins, M, idx, val);
        e = hipGetLastError();
    }
    return e == hipSuccess ? W4A16_OK : W4A16_ERR_LAUNCH;
}

// ---------------------------------------------------------------- allocation-free calls
// The workspace of w4a16_gemm_noalloc: a static device array, one copy per
// GPU the library runs on, held until the process ends.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in
// for the symbol); it passes the device address found for the current GPU.
__device__ __align__(256) uint8_t scratch[W4A16_NOALLOC_SCRATCH_BYTES];

__global__ void __launch_bounds__(256) clear_words_kernel(uint32_t *__restrict__ p, int n) {
    const int i = (int)blockIdx.x * 256 + (int)threadIdx.x;
    if (i < n) p[i] = 0u;
}

// The scratch array's address on the current device.  The first call on a
// device looks it up with that device current and clears the counter region
// with a kernel on `stream` (calls leave that region zero after that).
void *scratch_for_device(hipStream_t stream, int *status) {
    static std::mutex mu;
    static void *addr[64];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        *status = W4A16_ERR_DEVICE;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
            *status = W4A16_ERR_DEVICE;
            return nullptr;
        }
        const int n = W4A16_SPLIT_COUNTER_BYTES / 4;
        hipLaunchKernelGGL(clear_words_kernel, dim3((n + 255) / 256), dim3(256), 0, stream,
                           static_cast<uint32_t *>(p), n);
        if (hipGetLastError() != hipSuccess) {
            *status = W4A16_ERR_LAUNCH;
            return nullptr;
        }
        addr[dev] = p;
    }
    *status = W4A16_OK;
    return addr[dev];
}

}  // namespace

extern "C" {

const char *w4a16_status_string(int status) {
    switch (status) {
        case W4A16_OK: return "ok";
        case W4A16_ERR_NULL: return "null pointer argument";
        case W4A16_ERR_SHAPE: return "invalid shape (need 1<=M<=16, K%128==0, K<=2^24, N%16==0, (K/128)*N*2 < 2^31)";
        case W4A16_ERR_GROUP: return "group size must be 128 (GPTQ) or 16 (NVFP4)";
        case W4A16_ERR_ALIGN: return "device pointer not 16-byte aligned";
        case W4A16_ERR_WORKSPACE: return "workspace missing or too small";
        case W4A16_ERR_DEVICE: return "no gfx950 HIP device";
        case W4A16_ERR_LAUNCH: return "kernel launch failed";
        case W4A16_ERR_PLAN: return "no compiled kernel for this plan";
        default: return "unknown status";
    }
}

size_t w4a16_repacked_bytes(int K, int N) {
    if (check_weight_shape(K, N) != W4A16_OK) return 0;
    return (size_t)K * (size_t)N / 2;
}

int w4a16_repack_weights(const void *qweight, void *wq_repacked, int K, int N, void *stream) {
    if (!qweight || !wq_repacked) return W4A16_ERR_NULL;
    int st = check_weight_shape(K, N);
    if (st != W4A16_OK) return st;
    if (!aligned16(qweight) || !aligned16(wq_repacked)) return W4A16_ERR_ALIGN;
    st = check_device();
    if (st != W4A16_OK) return st;
    const long long npieces = (long long)K * N / 32;
    const unsigned grid = (unsigned)((npieces + 255) / 256);
    const uint32_t *q = static_cast<const uint32_t *>(qweight);
    u32x4 *b = static_cast<u32x4 *>(wq_repacked);
    int n = N, g = K / W4A16_GROUP;
    long long np = npieces;
    void *args[] = {&q, &b, &n, &g, &np};
    const hipError_t e = launch(reinterpret_cast<const void *>(repack_kernel), grid, 256, 0,
                                static_cast<hipStream_t>(stream), args);
    return e == hipSuccess ? W4A16_OK : W4A16_ERR_LAUNCH;
}

int w4a16_get_plan(int M, int N, int K, w4a16_plan_t *plan) {
    if (!plan) return W4A16_ERR_NULL;
    const int st = check_shape(M, N, K);
    if (st != W4A16_OK) return st;
    auto_plan(M, N, K, plan);
    return W4A16_OK;
}

int w4a16_check_plan(int M, int N, int K, const w4a16_plan_t *plan) {
    if (!plan) return W4A16_ERR_NULL;
    const int st = check_shape(M, N, K);
    if (st != W4A16_OK) return st;
    return validate_plan(*plan, M, N, K);
}

size_t w4a16_workspace_bytes_plan(int M, int N, int K, const w4a16_plan_t *plan) {
    if (check_shape(M, N, K) != W4A16_OK) return 0;
    w4a16_plan_t p{};
    if (plan) {
        p = *plan;
        if (validate_plan(p, M, N, K) != W4A16_OK) return 0;
    } else {
        auto_plan(M, N, K, &p);
    }
    return workspace_for(p, M, N);
}

size_t w4a16_workspace_bytes(int M, int N, int K) {
    return workspace_any_call(M, N, K, FMT_GPTQ);
}

int w4a16_gemm(const void *A, const void *wq_repacked, const void *scales, void *C, int M, int N,
               int K, int group, void *workspace, size_t workspace_bytes, void *stream) {
    return run_gemm(A, wq_repacked, scales, C, M, N, K, group, workspace, workspace_bytes, nullptr,
                    stream);
}

int w4a16_gemm_plan(const void *A, const void *wq_repacked, const void *scales, void *C, int M,
                    int N, int K, int group, void *workspace, size_t workspace_bytes,
                    const w4a16_plan_t *plan, void *stream) {
    return run_gemm(A, wq_repacked, scales, C, M, N, K, group, workspace, workspace_bytes, plan,
                    stream);
}

int w4a16_gemm_noalloc(const void *A, const void *wq_repacked, const void *scales, void *C, int M,
                       int N, int K, int group, const w4a16_plan_t *plan, void *stream) {
    // every check that needs no device comes first, so a rejected call
    // touches neither the device nor the scratch array
    if (!A || !wq_repacked || !scales || !C) return W4A16_ERR_NULL;
    int st = check_shape(M, N, K);
    if (st != W4A16_OK) return st;
    if (group != W4A16_GROUP) return W4A16_ERR_GROUP;
    if (!aligned16(A) || !aligned16(wq_repacked) || !aligned16(scales) || !aligned16(C)) return W4A16_ERR_ALIGN;
    w4a16_plan_t p{};
    if (plan) {
        p = *plan;
        st = validate_plan(p, M, N, K);
        if (st != W4A16_OK) return st;
    } else {
        auto_plan(M, N, K, &p);
        if (workspace_for(p, M, N) > (size_t)W4A16_NOALLOC_SCRATCH_BYTES) {
            p.splits = 1;                      // partials too large: every strip whole
            p.whole = 0;
        }
    }
    if (workspace_for(p, M, N) > (size_t)W4A16_NOALLOC_SCRATCH_BYTES) return W4A16_ERR_WORKSPACE;
    st = check_device();
    if (st != W4A16_OK) return st;
    void *ws = scratch_for_device(static_cast<hipStream_t>(stream), &st);
    if (st != W4A16_OK) return st;
    return run_gemm(A, wq_repacked, scales, C, M, N, K, group, ws, W4A16_NOALLOC_SCRATCH_BYTES, &p, stream);
}

int w4a16_gemm_f32(const void *A, const void *wq_repacked, const void *scales, float *C, int M,
                   int N, int K, int group, void *workspace, size_t workspace_bytes, void *stream) {
    return run_gemm(A, wq_repacked, scales, C, M, N, K, group, workspace, workspace_bytes, nullptr,
                    stream, 3);
}

int w4a16_gemm_f32_plan(const void *A, const void *wq_repacked, const void *scales, float *C, int M,
                        int N, int K, int group, void *workspace, size_t workspace_bytes,
                        const w4a16_plan_t *plan, void *stream) {
    return run_gemm(A, wq_repacked, scales, C, M, N, K, group, workspace, workspace_bytes, plan,
                    stream, 3);
}

int w4a16_gemm_argmax(const void *A, const void *wq_repacked, const void *scales, int *idx,
                      float *val, int M, int N, int K, int group, void *workspace,
                      size_t workspace_bytes, void *stream) {
    return run_gemm(A, wq_repacked, scales, nullptr, M, N, K, group, workspace, workspace_bytes,
                    nullptr, stream, 2, idx, val);
}

int w4a16_gemm_argmax_plan(const void *A, const void *wq_repacked, const void *scales, int *idx,
                           float *val, int M, int N, int K, int group, void *workspace,
                           size_t workspace_bytes, const w4a16_plan_t *plan, void *stream) {
    return run_gemm(A, wq_repacked, scales, nullptr, M, N, K, group, workspace, workspace_bytes,
                    plan, stream, 2, idx, val);
}

int w4a16_gemm_silu_mul(const void *A, const void *wq_repacked, const void *scales, void *H, int M,
                        int N, int K, int group, void *workspace, size_t workspace_bytes,
                        void *stream) {
    return run_gemm(A, wq_repacked, scales, H, M, N, K, group, workspace, workspace_bytes, nullptr,
                    stream, 1);
}

int w4a16_gemm_silu_mul_plan(const void *A, const void *wq_repacked, const void *scales, void *H,
                             int M, int N, int K, int group, void *workspace,
                             size_t workspace_bytes, const w4a16_plan_t *plan, void *stream) {
    return run_gemm(A, wq_repacked, scales, H, M, N, K, group, workspace, workspace_bytes, plan,
                    stream, 1);
}

static int run_export(const void *wq, const void *scales, float *W, uint8_t *codes, int K, int N,
                      void *stream) {
    int st = check_weight_shape(K, N);
    if (st != W4A16_OK) return st;
    if (!aligned16(wq) || (scales && !aligned16(scales)) || (W && !aligned16(W)) ||
        (codes && !aligned16(codes)))
        return W4A16_ERR_ALIGN;
    st = check_device();
    if (st != W4A16_OK) return st;
    const long long npieces = (long long)K * N / 32;
    const unsigned grid = (unsigned)((npieces + 255) / 256);
    const u32x4 *b = static_cast<const u32x4 *>(wq);
    const uint16_t *s = static_cast<const uint16_t *>(scales);
    int n = N, g = K / W4A16_GROUP;
    long long np = npieces;
    void *args[] = {&b, &s, &W, &codes, &n, &g, &np};
    const void *fn = codes ? reinterpret_cast<const void *>(export_kernel<true>)
                           : reinterpret_cast<const void *>(export_kernel<false>);
    const hipError_t e = launch(fn, grid, 256, 0, static_cast<hipStream_t>(stream), args);
    return e == hipSuccess ? W4A16_OK : W4A16_ERR_LAUNCH;
}

int w4a16_dequant_debug(const void *wq_repacked, const void *scales, float *W, int K, int N,
                        void *stream) {
    if (!wq_repacked || !scales || !W) return W4A16_ERR_NULL;
    return run_export(wq_repacked, scales, W, nullptr, K, N, stream);
}

int w4a16_unpack_debug(const void *wq_repacked, uint8_t *codes, int K, int N, void *stream) {
    if (!wq_repacked || !codes) return W4A16_ERR_NULL;
    return run_export(wq_repacked, nullptr, nullptr, codes, K, N, stream);
}

// ---------------------------------------------------------------- NVFP4

size_t w4a16_nvfp4_repacked_bytes(int K, int N) {
    if (check_weight_shape(K, N) != W4A16_OK) return 0;
    return (size_t)K * (size_t)N / 2;
}

size_t w4a16_nvfp4_repacked_scale_bytes(int K, int N) {
    if (check_weight_shape(K, N) != W4A16_OK) return 0;
    return (size_t)(K / W4A16_NVFP4_GROUP) * (size_t)N;
}

int w4a16_nvfp4_repack_weights(const void *packed, void *wq_repacked, int K, int N, void *stream) {
    if (!packed || !wq_repacked) return W4A16_ERR_NULL;
    int st = check_weight_shape(K, N);
    if (st != W4A16_OK) return st;
    if (!aligned16(packed) || !aligned16(wq_repacked)) return W4A16_ERR_ALIGN;
    st = check_device();
    if (st != W4A16_OK) return st;
    const long long npieces = (long long)K * N / 32;
    const unsigned grid = (unsigned)((npieces + 255) / 256);
    const uint8_t *in = static_cast<const uint8_t *>(packed);
    u32x4 *b = static_cast<u32x4 *>(wq_repacked);
    int k = K, g = K / W4A16_GROUP;
    long long np = npieces;
    void *args[] = {&in, &b, &k, &g, &np};
    const hipError_t e = launch(reinterpret_cast<const void *>(nv_repack_kernel), grid, 256, 0,
                                static_cast<hipStream_t>(stream), args);
    return e == hipSuccess ? W4A16_OK : W4A16_ERR_LAUNCH;
}

int w4a16_nvfp4_repack_scales(const void *scales, void *scales_repacked, int K, int N, void *stream) {
    if (!scales || !scales_repacked) return W4A16_ERR_NULL;
    int st = check_weight_shape(K, N);
    if (st != W4A16_OK) return st;
    if (!aligned16(scales) || !aligned16(scales_repacked)) return W4A16_ERR_ALIGN;
    st = check_device();
    if (st != W4A16_OK) return st;
    const long long count = (long long)(K / W4A16_NVFP4_GROUP) * N;
    const unsigned grid = (unsigned)((count + 255) / 256);
    const uint8_t *in = static_cast<const uint8_t *>(scales);
    uint8_t *out = static_cast<uint8_t *>(scales_repacked);
    int k = K, g = K / W4A16_GROUP;
    long long cnt = count;
    void *args[] = {&in, &out, &k, &g, &cnt};
    const hipError_t e = launch(reinterpret_cast<const void *>(nv_repack_scales_kernel), grid, 256, 0,
                                static_cast<hipStream_t>(stream), args);
    return e == hipSuccess ? W4A16_OK : W4A16_ERR_LAUNCH;
}

int w4a16_nvfp4_get_plan(int M, int N, int K, w4a16_plan_t *plan) {
    if (!plan) return W4A16_ERR_NULL;
    const int st = check_shape(M, N, K);
    if (st != W4A16_OK) return st;
    auto_plan_nv(M, N, K, plan);
    return W4A16_OK;
}

int w4a16_nvfp4_check_plan(int M, int N, int K, const w4a16_plan_t *plan) {
    if (!plan) return W4A16_ERR_NULL;
    const int st = check_shape(M, N, K);
    if (st != W4A16_OK) return st;
    return validate_plan(*plan, M, N, K, FMT_NVFP4);
}

size_t w4a16_nvfp4_workspace_bytes_plan(int M, int N, int K, const w4a16_plan_t *plan) {
    if (check_shape(M, N, K) != W4A16_OK) return 0;
    w4a16_plan_t p{};
    if (plan) {
        p = *plan;
        if (validate_plan(p, M, N, K, FMT_NVFP4) != W4A16_OK) return 0;
    } else {
        auto_plan_nv(M, N, K, &p);
    }
    return workspace_for(p, M, N);
}

size_t w4a16_nvfp4_workspace_bytes(int M, int N, int K) {
    return workspace_any_call(M, N, K, FMT_NVFP4);
}

int w4a16_nvfp4_gemm(const void *A, const void *wq_repacked, const void *scales, float alpha, void *C,
                     int M, int N, int K, int group, void *workspace, size_t workspace_bytes,
                     void *stream) {
    return run_gemm(A, wq_repacked, scales, C, M, N, K, group, workspace, workspace_bytes, nullptr,
                    stream, 0, nullptr, nullptr, FMT_NVFP4, alpha);
}

int w4a16_nvfp4_gemm_plan(const void *A, const void *wq_repacked, const void *scales, float alpha,
                          void *C, int M, int N, int K, int group, void *workspace,
                          size_t workspace_bytes, const w4a16_plan_t *plan, void *stream) {
    return run_gemm(A, wq_repacked, scales, C, M, N, K, group, workspace, workspace_bytes, plan,
                    stream, 0, nullptr, nullptr, FMT_NVFP4, alpha);
}

int w4a16_nvfp4_gemm_silu_mul(const void *A, const void *wq_repacked, const void *scales, float alpha,
                              void *H, int M, int N, int K, int group, void *workspace,
                              size_t workspace_bytes, void *stream) {
    return run_gemm(A, wq_repacked, scales, H, M, N, K, group, workspace, workspace_bytes, nullptr,
                    stream, 1, nullptr, nullptr, FMT_NVFP4, alpha);
}

int w4a16_nvfp4_gemm_silu_mul_plan(const void *A, const void *wq_repacked, const void *scales,
                                   float alpha, void *H, int M, int N, int K, int group,
                                   void *workspace, size_t workspace_bytes, const w4a16_plan_t *plan,
                                   void *stream) {
    return run_gemm(A, wq_repacked, scales, H, M, N, K, group, workspace, workspace_bytes, plan,
                    stream, 1, nullptr, nullptr, FMT_NVFP4, alpha);
}

int w4a16_nvfp4_gemm_argmax(const void *A, const void *wq_repacked, const void *scales, float alpha,
                            int *idx, float *val, int M, int N, int K, int group, void *workspace,
                            size_t workspace_bytes, void *stream) {
    return run_gemm(A, wq_repacked, scales, nullptr, M, N, K, group, workspace, workspace_bytes,
                    nullptr, stream, 2, idx, val, FMT_NVFP4, alpha);
}

int w4a16_nvfp4_gemm_argmax_plan(const void *A, const void *wq_repacked, const void *scales,
                                 float alpha, int *idx, float *val, int M, int N, int K, int group,
                                 void *workspace, size_t workspace_bytes, const w4a16_plan_t *plan,
                                 void *stream) {
    return run_gemm(A, wq_repacked, scales, nullptr, M, N, K, group, workspace, workspace_bytes,
                    plan, stream, 2, idx, val, FMT_NVFP4, alpha);
}

int w4a16_nvfp4_gemm_f32(const void *A, const void *wq_repacked, const void *scales, float alpha,
                         float *C, int M, int N, int K, int group, void *workspace,
                         size_t workspace_bytes, void *stream) {
    return run_gemm(A, wq_repacked, scales, C, M, N, K, group, workspace, workspace_bytes, nullptr,
                    stream, 3, nullptr, nullptr, FMT_NVFP4, alpha);
}

int w4a16_nvfp4_gemm_f32_plan(const void *A, const void *wq_repacked, const void *scales, float alpha,
                              float *C, int M, int N, int K, int group, void *workspace,
                              size_t workspace_bytes, const w4a16_plan_t *plan, void *stream) {
    return run_gemm(A, wq_repacked, scales, C, M, N, K, group, workspace, workspace_bytes, plan,
                    stream, 3, nullptr, nullptr, FMT_NVFP4, alpha);
}

int w4a16_nvfp4_dequant(const void *wq_repacked, const void *scales, float *W, int K, int N,
                        void *stream) {
    if (!wq_repacked || !scales || !W) return W4A16_ERR_NULL;
    int st = check_weight_shape(K, N);
    if (st != W4A16_OK) return st;
    if (!aligned16(wq_repacked) || !aligned16(scales) || !aligned16(W)) return W4A16_ERR_ALIGN;
    st = check_device();
    if (st != W4A16_OK) return st;
    const long long npieces = (long long)K * N / 32;
    const unsigned grid = (unsigned)((npieces + 255) / 256);
    const u32x4 *b = static_cast<const u32x4 *>(wq_repacked);
    const uint8_t *sc = static_cast<const uint8_t *>(scales);
    int n = N, g = K / W4A16_GROUP;
    long long np = npieces;
    void *args[] = {&b, &sc, &W, &n, &g, &np};
    const hipError_t e = launch(reinterpret_cast<const void *>(nv_export_kernel), grid, 256, 0,
                                static_cast<hipStream_t>(stream), args);
    return e == hipSuccess ? W4A16_OK : W4A16_ERR_LAUNCH;
}

}  // extern "C"
