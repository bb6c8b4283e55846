// Device code of the W4A16 decode/verify matmul for gfx950 (CDNA4, wave64).
//
// C[M,N] = A[M,K] . W[K,N] with W[k,n] = (q[k,n] - 8) * s[k/128, n]: symmetric
// GPTQ 4-bit codes, group 128 along K, bf16 activations and scales (checkpoint
// contract on the page "Qwen3.8-27B on single DGX Spark ...", section
// "Quality.").  Decode is bound by the bytes of the weights (page "One Config
// Line Made My 27B Model 2.7x Faster", section "Gotcha #2"), so everything
// here is arranged around one streaming read of the repacked blob.
//
// Dequantization without a subtraction per weight: OR-ing a 4-bit code q into
// the low mantissa bits of bf16 128.0 (0x4300) gives exactly the bf16 value
// 128 + q.  The contraction runs on these biased values, and the bias is
// removed once per group and row:
//     sum_k a_k (q_k - 8) = sum_k a_k (128 + q_k) - sum_k a_k * 136.
// The bias sum is column independent, so it is formed once per group (per
// workgroup in the GEMV path, per wavefront in the MFMA path), never per
// weight.  It is formed by the very instruction sequence that forms the
// weight sum, in the same order, with every code replaced by 8: a group whose
// codes are all 8 therefore contributes exactly zero, as it must.  The group
// scale multiplies the group's partial sum, so no dequantized weight is ever
// rounded.
//
// The same kernels also run the NVFP4 weight-only variant (FMT_NVFP4): 4-bit
// E2M1 codes with one E4M3 scale per 16 consecutive rows of a column and one
// fp32 factor per tensor (the nvfp4-pack-quantized checkpoints of the page
// "Qwen3.8 27B - NVFP4 for veloGB10", section "Specifications"; group size 16
// on the page "SuperQwen3.8-27b-abliterated-NVFP4-2xDGX", table "Release
// highlights").  E2M1 -> bf16 is one hardware conversion per code pair, exact
// and signed, so no bias is needed; the block scale multiplies the 16-row
// block's partial sum (one 16x16x16 matrix-core product, or two dot2, per
// block), and the per-tensor factor multiplies the final sum.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace w4a16 {

constexpr int kGroup = 128;
constexpr uint32_t kMagicPair = 0x43004300u;   // bf16 pair (128.0, 128.0)
constexpr uint32_t kNibblePair = 0x000F000Fu;  // the low nibble of each half
constexpr uint32_t kBiasPair = 0x43084308u;    // bf16 pair (136.0, 136.0) = codes of 8
constexpr float kBias = 136.0f;                // 128 (magic) + 8 (code midpoint)
constexpr int kXcds = 8;                       // MI355X: 8 XCDs, 32 CUs each
constexpr int kRowPad = 16;                    // bytes of padding per staged A row
constexpr int kRingSlotBytes = 16 * kGroup * 2; // one group of A, 16 rows, in the shared (split-N) LDS ring

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

enum { PATH_GEMV = 1, PATH_MFMA = 2 };
// ASRC_SPLITN: the four wavefronts of a workgroup split the strip's columns
// (T tiles each) instead of its K range, and A goes per group through one
// LDS ring shared by them: each group of A is fetched once for 4 * T tiles
// (matrix-core path)
enum { ASRC_LDS = 0, ASRC_GLOBAL = 1, ASRC_RING = 2, ASRC_SPLITN = 3 };
enum { FMT_GPTQ = 0, FMT_NVFP4 = 1 };
constexpr int kNvBlock = 16;                   // NVFP4 rows per block scale

struct GemmArgs {
    const uint16_t *A;       // bf16 [M][K]
    const u32x4 *blob;       // repacked weights, 64 pieces of 16 B per (tile, group)
    const uint16_t *scales;  // bf16 scales as in the checkpoint: [K/128][N]
                             // (NVFP4: E4M3 bytes [tile][group][16 columns][8 blocks])
    uint16_t *C;             // bf16 [M][N]
    float *part;             // split-K partials [S][M][N] (S > 1 only)
    uint32_t *count;         // split-K arrival counters [nstrips] (S > 1 only)
    int M, N, K, G;          // G = K / 128
    int S;                   // workgroups along K per split column strip (a power of two)
    int Slog2;               // log2(S)
    int NT;                  // 16-column tiles = N / 16
    int nstrips;             // column strips = ceil(NT / tiles)
    int nwhole;              // strips 0 .. nwhole-1 are computed whole by one workgroup each;
                             // the others are split S ways along K
    int nunits;              // nwhole + (nstrips - nwhole) * S = grid size
    int fuse;                // epilogue: 0 plain C, 1 gate/up activation, 2 row argmax,
                             // 3 C as fp32 (unrounded partial sums of a K shard)
    int *amax_idx;           // row argmax: column of each row's maximum [M]
    float *amax_val;         // row argmax: its fp32 value [M]
    float alpha;             // NVFP4: per-tensor factor of the sum
};

// Row argmax: per-row maxima meet in kArgmaxBins 64-bit slots per row
// (workgroup index modulo the bin count), kept in the workspace's counter
// region at byte kArgmaxBinOffset; its counter is the region's first word.
// Every call leaves the region zero, whichever kind of call it is.
constexpr int kArgmaxBins = 64;
constexpr int kArgmaxBinOffset = 256;

// ---------------------------------------------------------------- LDS plan
// Shared by host (sizing) and device (carving).  Offsets in bytes.
struct LdsLayout {
    int keys;   // row argmax: one 64-bit key per row [16]
    int a;      // staged A rows [M][Gwg*128 bf16 + pad]; ring: [KW][D][4 ceil(M/4) rows][256 B] + pad
    int bias;   // GEMV: bias of each 32-row quarter [M][Gwg][4] fp32;
                // MFMA with staged A: bias tile rows [Gwg][16] fp32
    int red;    // cross-wavefront reduction [KW][T*M*16] fp32
    int total;
    int row;    // bytes per staged A row
};

// Slots of the shared split-N ring: D + 1 rounded up to a power of two, so
// that a group's slot is its index masked (a modulo by D + 1 cost several
// scalar instructions per group, twice)
__host__ __device__ constexpr int shared_slots(int D) {
    int n = 1;
    while (n < D + 1) n <<= 1;
    return n;
}

__host__ __device__ inline LdsLayout lds_layout(int path, int asrc, int M, int Gwg, int T, int KW, int D) {
    LdsLayout L;
    const bool stage = (path == PATH_GEMV) || (asrc == ASRC_LDS);
    L.row = Gwg * kGroup * 2 + kRowPad;
    int off = 0;
    L.keys = off;
    off += 16 * 8;
    L.a = off;
    if (stage) off += M * L.row;
    else if (path == PATH_MFMA && asrc == ASRC_RING) {
        // ceil(M/4) KiB per slot (four rows per KiB); the matrix-core reads
        // take 16 rows from a slot, so the last slot's reads of rows past
        // 4 ceil(M/4) need (4 - ceil(M/4)) KiB after it
        const int nd = (M + 3) / 4;
        off += KW * D * nd * 1024 + (4 - nd) * 1024;
    }
    else if (path == PATH_MFMA && asrc == ASRC_SPLITN) off += shared_slots(D) * kRingSlotBytes;
    L.bias = off;
    if (path == PATH_GEMV) off += M * Gwg * 4 * 4;
    else if (stage) off += Gwg * 16 * 4;
    L.red = off;
    if (KW > 1 && asrc != ASRC_SPLITN) off += KW * T * M * 16 * 4;
    L.total = off;
    return L;
}

// ---------------------------------------------------------------- helpers

// Register-held constants of the dequantization.  gfx9-family VOP3
// instructions take no 32-bit literal, so v_and_or_b32 needs its mask and
// magic in registers; made opaque once per kernel, they stay there (with
// literal constants the compiler would split each into v_and + v_or).
struct DequantConsts {
    uint32_t nib;     // SGPR: 0x000F000F
    uint32_t magic;   // VGPR: 0x43004300
};

__device__ __forceinline__ DequantConsts dequant_consts() {
    DequantConsts k;
    asm volatile("s_mov_b32 %0, 0x000f000f" : "=s"(k.nib));
    asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(k.magic));
    return k;
}

// Plain C on purpose: the compiler selects v_and_or_b32 from it (the operands
// are registers) and so knows the instruction when it places the wait states
// an MFMA reading its result needs.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t nib, uint32_t magic) {
    return (x & nib) | magic;
}

// Two repacked words (each: codes of 8 consecutive rows e = 0..7; even e in
// bits 0..15, odd e in bits 16..31, 4 bits each) -> four bf16 pairs
// (128 + q_e, 128 + q_{e+1}), e = 0, 2, 4, 6, per word.
//
// SHIFT64: the words share their shifts: one v_lshrrev_b64 by 4 moves both,
// and the bits it carries from w1 into the low word land in bits 28..31,
// which the mask drops (eleven VALU operations for sixteen codes).  The shift
// is written out because the compiler otherwise splits it into a funnel shift
// and a 32-bit shift; only kernels without matrix-core instructions use this
// form, since the compiler cannot see an inline-asm write when it places the
// wait states that protect registers an in-flight MFMA still reads.
// Without SHIFT64 the compiler forms the shifts (fourteen operations).
template <bool SHIFT64>
__device__ __forceinline__ void words_to_bf16x8(uint32_t w0, uint32_t w1, const DequantConsts &k,
                                                uint32_t (&b0)[4], uint32_t (&b1)[4]) {
    uint64_t x = ((uint64_t)w1 << 32) | w0;
    b0[0] = and_or(w0, k.nib, k.magic);
    b1[0] = and_or(w1, k.nib, k.magic);
#pragma unroll
    for (int v = 1; v < 4; ++v) {
        if constexpr (SHIFT64)
            asm("v_lshrrev_b64 %0, 4, %1" : "=v"(x) : "v"(x));
        else
            x >>= 4;
        b0[v] = and_or((uint32_t)x, k.nib, k.magic);
        b1[v] = and_or((uint32_t)(x >> 32), k.nib, k.magic);
    }
}

// Byte selector for v_perm_b32 that moves a lane's bf16 scale (low half of
// the dword for even columns, high half for odd) to the top of an fp32 with
// zero low bits.
__device__ __forceinline__ uint32_t scale_selector(int c) { return (c & 1) ? 0x03020C0Cu : 0x01000C0Cu; }
__device__ __forceinline__ float scale_from(uint32_t dword, uint32_t sel) {
    return __uint_as_float(__builtin_amdgcn_perm(dword, dword, sel));
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ float pair_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float pair_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// Order-preserving 64-bit key of (value, column): a larger value gives a
// larger key, and for equal values the lower column does (-0 counts as +0).
__device__ __forceinline__ unsigned long long argmax_key(float v, uint32_t col) {
    uint32_t u = __float_as_uint(v == 0.0f ? 0.0f : v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((unsigned long long)u << 32) | (0xFFFFFFFFu - col);
}
__device__ __forceinline__ float argmax_key_value(unsigned long long k) {
    uint32_t u = (uint32_t)(k >> 32);
    u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
    return __uint_as_float(u);
}

// fp32 -> bf16, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Workgroups are dispatched to the 8 XCDs round robin (block b -> XCD b % 8).
// Give each XCD one contiguous range of work units, so the K splits of one
// strip meet in one L2.
__device__ __forceinline__ int xcd_unit(int b, int nunits) {
    const int q = nunits / kXcds, r = nunits % kXcds;
    const int x = b % kXcds, slot = b / kXcds;
    return x * q + (x < r ? x : r) + slot;
}

__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
}

// ---------------------------------------------------------------- NVFP4 helpers
// E2M1 code pair (byte SEL of w, low nibble first) -> bf16 pair, by the
// gfx950 conversion instruction with scale 1.0.  Its scale operand only
// contributes a power of two, so an E4M3 block scale (three mantissa bits)
// cannot be folded in here; it multiplies the block's partial sum instead,
// and every converted weight is exact.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1x2_to_bf16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL));
}

// Block B (0..7) of a lane's 16 repacked bytes: rows 4h .. 4h+3 of the
// block as two bf16 pairs (byte 2B holds rows 4h, 4h+1; byte 2B+1 rows
// 4h+2, 4h+3).
template <int B>
__device__ __forceinline__ u32x2 nv_block(const u32x4 &w) {
    const uint32_t x = w[B >> 1];
    return u32x2{e2m1x2_to_bf16x2<2 * (B & 1)>(x), e2m1x2_to_bf16x2<2 * (B & 1) + 1>(x)};
}

// The eight E4M3 block scales of a lane's 8 scale bytes (gfx950 converts
// OCP E4M3), two per instruction: out[b] is byte b.
__device__ __forceinline__ void nv_scales(const uint32_t *s, float (&out)[8]) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const f32x2 v0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)s[0], false);
    const f32x2 v1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)s[0], true);
    const f32x2 v2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)s[1], false);
    const f32x2 v3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)s[1], true);
    out[0] = v0[0], out[1] = v0[1], out[2] = v1[0], out[3] = v1[1];
    out[4] = v2[0], out[5] = v2[1], out[6] = v3[0], out[7] = v3[1];
}

// 16x16x16 bf16 product: lane l supplies A[l % 16][4 (l / 16) + i] and
// B[4 (l / 16) + i][l % 16], i = 0..3, and receives rows 4 (l / 16) + v of
// column l % 16.
__device__ __forceinline__ f32x4 mfma16x16x16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// Sum of a value over the 4 lanes l, l^16, l^32, l^48 (the four K quarters of
// one column in the GEMV lane layout), in the fixed order
// (x[l] + x[l^32]) + (x[l^16] + x[l^16^32]); every one of the 4 lanes gets
// bitwise the same result.
__device__ __forceinline__ float sum_quarters(float x) {
    uint32_t u = __float_as_uint(x);
    auto s32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    float y = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
    uint32_t v = __float_as_uint(y);
    auto s16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
}

// s_waitcnt immediates (gfx9 encoding): vmcnt <= n only; LDS/scalar only.
constexpr int waitcnt_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
constexpr int kWaitLgkm0 = 15 | (7 << 4) | (0 << 8) | (3 << 14);

// Barrier for LDS traffic only: unlike __syncthreads() it does not wait for
// outstanding global loads, so the weight ring stays in flight across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
}

// Workgroup barrier that also orders LDS accesses for the compiler: no LDS
// read after it is moved above it, none before it below it.  At workgroup
// scope the fences wait for no global memory operation.
__device__ __forceinline__ void wg_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at lds_base + 16*l (lds_base wave-uniform).  Written as inline assembly so
// that the compiler's wait insertion does not track it: the caller waits for
// it explicitly (it is older than every load issued after it).
// M0 is a reserved register to the compiler; nothing else in these kernels
// uses it (no LDS-DMA builtins, messages or relative register moves), so
// setting it here cannot disturb compiler-generated code.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const void *gsrc, uint32_t lds_base) {
    // one wait state between the SALU write of M0 and the LDS-DMA load reading it
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(gsrc), "s"(lds_base)
                 : "memory", "m0");
}
// The same with a wave-uniform 64-bit base (SGPRs) and a 32-bit per-lane
// byte offset: no vector address arithmetic when only the base moves.
__device__ __forceinline__ void lds_dma16_sbase(uint32_t voff, const void *sbase, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(lds_base)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Buffer resource of `bytes` bytes at `base` (gfx9 raw buffer: stride 0,
// dword 3 = 0x00020000).  Loads through it take a per-lane offset (VGPR)
// plus a wave-uniform offset (SGPR); offsets past `bytes` read zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr int kCachePolicyNt = 2;   // non-temporal: streamed weights

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// ---------------------------------------------------------------- row argmax fold
// One workgroup of kArgmaxBins * 16 threads: thread (b, m) reads bin b of row
// m and clears it; the rows' maxima meet in LDS; thread m < M writes the
// column and value of row m.
static __global__ void __launch_bounds__(kArgmaxBins * 16) argmax_fold_kernel(unsigned long long *__restrict__ bins,
                                                                       int M, int *__restrict__ idx,
                                                                       float *__restrict__ val) {
    __shared__ unsigned long long best[16];
    const int m = threadIdx.x & 15, b = threadIdx.x >> 4;
    if (threadIdx.x < 16) best[threadIdx.x] = 0ull;
    __syncthreads();
    if (m < M) {
        const unsigned long long k = bins[b * 16 + m];
        bins[b * 16 + m] = 0ull;
        if (k) __hip_atomic_fetch_max(&best[m], k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    __syncthreads();
    if (threadIdx.x < (unsigned)M) {
        const unsigned long long k = best[threadIdx.x];
        idx[threadIdx.x] = (int)(0xFFFFFFFFu - (uint32_t)k);
        val[threadIdx.x] = argmax_key_value(k);
    }
}

// ---------------------------------------------------------------- repack
// One thread per 16-byte piece of the blob (see the layout in w4a16.h).
__device__ __forceinline__ uint32_t gptq_word_to_tile_word(uint32_t x) {
    uint32_t out = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t q = (x >> (4 * j)) & 0xFu;
        const int pos = (j & 1) ? 16 + 4 * (j >> 1) : 4 * (j >> 1);
        out |= q << pos;
    }
    return out;
}

static __global__ void __launch_bounds__(256) repack_kernel(const uint32_t *__restrict__ qweight,
                                                     u32x4 *__restrict__ blob, int N, int G,
                                                     long long npieces) {
    const long long pc = (long long)blockIdx.x * 256 + threadIdx.x;
    if (pc >= npieces) return;
    const int c = (int)(pc & 15), h = (int)((pc >> 4) & 3);
    const long long tg = pc >> 6;
    const int g = (int)(tg % G);
    const long long t = tg / G;
    const long long n = t * 16 + c;
    u32x4 out;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const long long kb = (long long)g * 16 + h * 4 + r;
        out[r] = gptq_word_to_tile_word(qweight[kb * N + n]);
    }
    blob[pc] = out;
}

// Test exports: the same words_to_bf16x8 the GEMM kernels use, and the
// checkpoint's scales [K/128][N].  Both instruction forms run (the shared
// 64-bit shift of the GEMV kernels and the compiler's shifts of the
// matrix-core kernels); where they disagree the export writes a value no
// exact dequantization has (NaN, or code 255), so an export that matches
// the oracle pins both.
template <bool CODES>
__global__ void __launch_bounds__(256) export_kernel(const u32x4 *__restrict__ blob,
                                                     const uint16_t *__restrict__ scales,
                                                     float *__restrict__ W, uint8_t *__restrict__ codes,
                                                     int N, int G, long long npieces) {
    const long long pc = (long long)blockIdx.x * 256 + threadIdx.x;
    if (pc >= npieces) return;
    const int c = (int)(pc & 15), h = (int)((pc >> 4) & 3);
    const long long tg = pc >> 6;
    const int g = (int)(tg % G);
    const long long t = tg / G;
    const long long n = t * 16 + c;
    const u32x4 w = blob[pc];
    const DequantConsts kc = dequant_consts();
    const float s = CODES ? 0.0f : bf16_bits_to_f32(scales[(long long)g * N + n]);
    uint32_t bw[4][4], bx[4][4];
    words_to_bf16x8<true>(w[0], w[1], kc, bw[0], bw[1]);
    words_to_bf16x8<true>(w[2], w[3], kc, bw[2], bw[3]);
    words_to_bf16x8<false>(w[0], w[1], kc, bx[0], bx[1]);
    words_to_bf16x8<false>(w[2], w[3], kc, bx[2], bx[3]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t (&b)[4] = bw[r];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const long long k = (long long)g * kGroup + h * 32 + r * 8 + 2 * v;
            const bool same = b[v] == bx[r][v];
            const float lo = pair_lo(b[v]), hi = pair_hi(b[v]);
            if (CODES) {
                codes[k * N + n] = same ? (uint8_t)(int)(lo - 128.0f) : (uint8_t)255;
                codes[(k + 1) * N + n] = same ? (uint8_t)(int)(hi - 128.0f) : (uint8_t)255;
            } else {
                W[k * N + n] = same ? (lo - kBias) * s : __builtin_nanf("");
                W[(k + 1) * N + n] = same ? (hi - kBias) * s : __builtin_nanf("");
            }
        }
    }
}

// ---------------------------------------------------------------- NVFP4 repack
// One thread per 16-byte piece (t, g, h, c) of column n = 16 t + c: byte
// 2 b + p is byte 64 g + 8 b + 2 h + p of column n's packed codes [N][K/2]
// (rows 128 g + 16 b + 4 h + 2 p and the next one).
static __global__ void __launch_bounds__(256) nv_repack_kernel(const uint8_t *__restrict__ packed,
                                                        u32x4 *__restrict__ blob, int K, int G,
                                                        long long npieces) {
    const long long pc = (long long)blockIdx.x * 256 + threadIdx.x;
    if (pc >= npieces) return;
    const int c = (int)(pc & 15), h = (int)((pc >> 4) & 3);
    const long long tg = pc >> 6;
    const int g = (int)(tg % G);
    const long long t = tg / G;
    const uint8_t *src = packed + (t * 16 + c) * (long long)(K / 2) + 64 * g + 2 * h;
    u32x4 out;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t lo = *reinterpret_cast<const uint16_t *>(src + 16 * r);
        const uint32_t hi = *reinterpret_cast<const uint16_t *>(src + 16 * r + 8);
        out[r] = lo | (hi << 16);
    }
    blob[pc] = out;
}

// NVFP4 scales [N][K/16] -> [tile][superblock][16 columns][8 blocks]: one
// thread per byte.
static __global__ void __launch_bounds__(256) nv_repack_scales_kernel(const uint8_t *__restrict__ scales,
                                                               uint8_t *__restrict__ out, int K, int G,
                                                               long long count) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= count) return;
    const int b = (int)(i & 7), c = (int)((i >> 3) & 15);
    const long long tg = i >> 7;
    const int g = (int)(tg % G);
    const long long t = tg / G;
    out[i] = scales[(t * 16 + c) * (long long)(K / kNvBlock) + 8 * g + b];
}

// Test export: fp32 W[k][n] = e2m1 * e4m3 through the GEMM kernels' own
// conversions (exact: at most six significant bits).
static __global__ void __launch_bounds__(256) nv_export_kernel(const u32x4 *__restrict__ blob,
                                                        const uint8_t *__restrict__ scales,
                                                        float *__restrict__ W, int N, int G,
                                                        long long npieces) {
    const long long pc = (long long)blockIdx.x * 256 + threadIdx.x;
    if (pc >= npieces) return;
    const int c = (int)(pc & 15), h = (int)((pc >> 4) & 3);
    const long long tg = pc >> 6;
    const int g = (int)(tg % G);
    const long long n = (tg / G) * 16 + c;
    const u32x4 w = blob[pc];
    const u32x2 sraw = *reinterpret_cast<const u32x2 *>(scales + (tg * 16 + c) * 8);
    const uint32_t s[2] = {sraw[0], sraw[1]};
    float scl[8];
    nv_scales(s, scl);
    [&]<int... B>(std::integer_sequence<int, B...>) {
        (([&] {
             const u32x2 v = nv_block<B>(w);
             const float sc = scl[B];
             const long long k = (long long)g * kGroup + B * kNvBlock + 4 * h;
             W[k * N + n] = pair_lo(v[0]) * sc;
             W[(k + 1) * N + n] = pair_hi(v[0]) * sc;
             W[(k + 2) * N + n] = pair_lo(v[1]) * sc;
             W[(k + 3) * N + n] = pair_hi(v[1]) * sc;
         }()),
         ...);
    }(std::make_integer_sequence<int, 8>{});
}

// ---------------------------------------------------------------- GEMM
//
// Work decomposition.  A workgroup owns one column strip of T 16-column tiles
// and one of S contiguous ranges of K groups; its KW wavefronts split that
// range further.  (Split-N, ASRC_SPLITN: the strip has KW * T tiles, and
// each wavefront takes T of them over the whole range.)  Every wavefront streams, for each of its groups, T pieces
// of 1 KiB (one 16-byte load per lane, the whole 1 KiB contiguous) plus the
// 16 scales of each tile, through a D-deep register ring, so D*T KiB per
// wavefront are in flight from the start.  All addresses are a wave-uniform
// base (scalar registers) plus a fixed per-lane offset, so the stream costs
// no vector instructions for address arithmetic.
//
// Issue order at start: first the asynchronous LDS fill of A (global -> LDS
// without passing through registers), then the weight ring.  Memory
// operations complete in order, so waiting for the A fill does not wait for
// any weight load, and the first group can be computed as soon as its own
// bytes arrive.
//
// Lane l of a wavefront owns column c = l % 16 of each tile and quarter
// h = l / 16 of each group (32 rows, 4 words).  In the MFMA path these are
// exactly the B operands of four v_mfma_f32_16x16x32_bf16 (lane l holds
// B[8*(l/16) + e][l % 16], e = 0..7, word r feeding instruction r), A rows
// are lanes l % 16, and the 16x16 fp32 result puts row 4*(l/16)+v of column
// l % 16 in register v.  In the GEMV path each lane forms dot products of its
// 32 rows with v_dot2_f32_bf16, and the four quarters of a column are summed
// across lanes at the very end.
//
// MM is the row count when it is known at compile time (1..4; the GEMV path
// always has it): then only the live rows are scaled and accumulated.  MM = 0
// (MFMA only) takes M at run time, up to 16.  MM < 0 (ring A only) also takes
// M at run time, with ceil(M/4) = -MM fixed: the group's DMA loads are then
// issued without a run-time count.
//
// The partial sums of the KW wavefronts meet in LDS and are added in a fixed
// order (split-N wavefronts hold whole sums of their own tiles); with S > 1 the workgroups of one strip meet in the workspace, where
// the last one to arrive adds the S partials in a fixed order.  No float
// atomics: the result does not depend on timing.
// EPI: the kernel carries the epilogue modes of GemmArgs::fuse; without it
// the mode is 0 (plain C) and no other mode's code is compiled in.
// FMT: the weight format.  NVFP4 pieces have the same geometry (one
// 1 KiB piece set per 16 columns x 128 rows); lane l holds rows 4h .. 4h+3 of
// each of the eight 16-row blocks, and 8 scale bytes per (tile, group).
template <int PATH, int MM, int T, int KW, int D, int ASRC, bool EPI, int FMT = FMT_GPTQ>
__global__ void __launch_bounds__(64 * KW) gemm_kernel(GemmArgs p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ int s_last;

    constexpr bool kNv = FMT == FMT_NVFP4;
    constexpr bool kGlobalA = (PATH == PATH_MFMA && ASRC == ASRC_GLOBAL);
    constexpr bool kRingA = (PATH == PATH_MFMA && ASRC == ASRC_RING);
    constexpr bool kSplitN = (PATH == PATH_MFMA && ASRC == ASRC_SPLITN);
    constexpr bool kStage = !kGlobalA && !kRingA && !kSplitN;
    static_assert(!kSplitN || KW == 4, "split-N: four wavefronts, one DMA load of A each per group");
    // wavefronts whose partial sums meet in LDS (split-N wavefronts each
    // hold whole sums of their own tiles)
    constexpr int KWR = kSplitN ? 1 : KW;
    constexpr int kLoadsPerGroup = 2 * T + (kGlobalA ? (kNv ? 8 : 4) : 0);   // loads the compiler sees
    // Matrix-core bias: formed in the loop from the A fragments already
    // loaded (four more MFMAs per group, shared by the T tiles), except for
    // four-tile strips of one or two rows, where one pass over the staged A
    // before the loop measures faster.
    constexpr bool kBiasInLoop = !kNv && PATH == PATH_MFMA && !(kStage && MM >= 1 && MM <= 2 && T >= 4);
    // rows of the 4-row block held by lane group h that are ever stored
    constexpr int kRowsV = (MM >= 1 && MM <= 4) ? MM : 4;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int M = (MM >= 1) ? MM : p.M;
    constexpr int kScaleBytes = kNv ? 128 : 32;   // scale bytes per (tile, group)
    const int c = lane & 15, h = lane >> 4;
    const int arow_m = min(c, M - 1);   // MFMA A-operand row of this lane

    // Work unit of this workgroup.  Units below nwhole are whole strips; the
    // others are the S pieces (contiguous K ranges) of the remaining strips.
    // Each XCD gets one contiguous range of units, so neighbouring strips
    // (which share the 128-byte lines of the scales) and the pieces of a
    // strip meet in one L2.  With whole strips, the first nwhole workgroups
    // (nwhole a multiple of 8) take them and the rest take the pieces, so
    // the hardware's placement gives each CU one whole strip and one piece.
    const int u = blockIdx.x < (unsigned)p.nwhole
                      ? xcd_unit(blockIdx.x, p.nwhole)
                      : p.nwhole + xcd_unit(blockIdx.x - p.nwhole, p.nunits - p.nwhole);
    const bool whole = u < p.nwhole;
    const bool split = !whole && p.S > 1;                     // this workgroup writes a partial sum
    const int ur = u - p.nwhole;
    const int strip = whole ? u : p.nwhole + (ur >> p.Slog2);
    const int z = whole ? 0 : (ur & (p.S - 1));
    const int slog2 = whole ? 0 : p.Slog2;
    const int gw0 = (p.G * z) >> slog2, gw1 = (p.G * (z + 1)) >> slog2;
    const int Gwg = gw1 - gw0;
    const int gk0 = kSplitN ? gw0 : gw0 + (Gwg * wave) / KW;
    const int gk1 = kSplitN ? gw1 : gw0 + (Gwg * (wave + 1)) / KW;
    const int ng = gk1 - gk0;
    const LdsLayout L = lds_layout(PATH, ASRC, M, Gwg, T, KW, D);
    const DequantConsts kc = dequant_consts();

    // Tiles of this strip.  Plain: T consecutive tiles.  Gate/up epilogue
    // (T even): the first T/2 slots hold gate tiles strip*T/2 + t, the last
    // T/2 the up tiles of the same columns, NT/2 tiles further on.
    // Split-N: wavefront w of strip s takes the tiles of sub-strip s*KW + w.
    constexpr int kHalfT = T / 2;
    const int fuse = EPI ? p.fuse : 0;
    const int vs = kSplitN ? strip * KW + wave : strip;
    auto tile_of = [&](int t) {
        if (fuse == 1) return t < kHalfT ? vs * kHalfT + t : (p.NT >> 1) + vs * kHalfT + (t - kHalfT);
        return vs * T + t;
    };
    auto tile_ok = [&](int t) {
        return fuse == 1 ? vs * kHalfT + (t < kHalfT ? t : t - kHalfT) < (p.NT >> 1) : vs * T + t < p.NT;
    };

    // Buffer resources (scalar): each tile's weights and scales, and A.
    // Every load is resource + fixed per-lane offset + the group's
    // wave-uniform offset, so the stream costs no vector address arithmetic.
    __amdgpu_buffer_rsrc_t wres[T], sres[T];
    const uint32_t s_gstride = kNv ? (uint32_t)kScaleBytes : (uint32_t)p.N * 2u;   // scale bytes between groups
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const size_t tile = (size_t)min(tile_of(t), p.NT - 1);
        wres[t] = buffer_rsrc(reinterpret_cast<const uint8_t *>(p.blob) + tile * (size_t)p.G * 1024,
                              (uint32_t)p.G * 1024u);
        // GPTQ: the checkpoint's scales [G][N]: tile t's 16 scales of group g
        // are the 32 bytes at g*2N + 32t.  NVFP4: repacked, one tile's
        // groups after each other.
        if constexpr (kNv)
            sres[t] = buffer_rsrc(reinterpret_cast<const uint8_t *>(p.scales) + tile * (size_t)p.G * kScaleBytes,
                                  (uint32_t)p.G * (uint32_t)kScaleBytes);
        else
            sres[t] = buffer_rsrc(reinterpret_cast<const uint8_t *>(p.scales) + tile * (size_t)kScaleBytes,
                                  (uint32_t)(p.G - 1) * s_gstride + (uint32_t)kScaleBytes);
    }
    const uint32_t w_lane = (uint32_t)lane * 16;             // this lane's 16 B of a 1 KiB piece
    // GPTQ: the dword holding this column's bf16 scale, and its half;
    // NVFP4: this column's 8 block-scale bytes
    const uint32_t s_lane = kNv ? (uint32_t)c * 8 : (uint32_t)(c >> 1) * 4;
    const uint32_t s_sel = scale_selector(c);
    // MFMA A from global memory: row arow_m, this lane group's rows of a
    // group.  GPTQ reads its four 16-byte pieces through a pointer, NVFP4
    // its eight 8-byte pieces through a buffer resource (each measured the
    // faster for its format).
    const uint8_t *abase = reinterpret_cast<const uint8_t *>(p.A) +
                           ((size_t)arow_m * p.K + (size_t)h * (kNv ? 4 : 32)) * 2;
    const __amdgpu_buffer_rsrc_t ares = buffer_rsrc(p.A, (uint32_t)M * (uint32_t)p.K * 2u);
    const uint32_t a_lane = ((uint32_t)arow_m * (uint32_t)p.K + (uint32_t)h * (kNv ? 4u : 32u)) * 2u;

    // ---- 1. asynchronous LDS fill of this wavefront's own K range of A
    // (all M rows), at its place in the workgroup's staged rows.  Each
    // wavefront reads only the A it fills itself, so no workgroup barrier
    // stands between the fill and the first group.
    if constexpr (kStage) {
        const int start = (gk0 - gw0) * kGroup * 2;          // byte offset of the range in a row
        const int bytes = ng * kGroup * 2;
        for (int m = 0; m < M; ++m)
            for (int q = 0; (q << 10) < bytes; ++q) {
                const int off = (q << 10) + lane * 16;
                const uint32_t dst =
                    __builtin_amdgcn_readfirstlane(lds_addr(smem + L.a + m * L.row + start + (q << 10)));
                if (off < bytes) {
                    const uint8_t *src = reinterpret_cast<const uint8_t *>(p.A + (size_t)m * p.K +
                                                                           (size_t)gk0 * kGroup) + off;
                    lds_dma16(src, dst);
                }
            }
    }

    // ---- 2. weight ring, D groups deep, issued in slot order
    u32x4 wv[D][T];
    uint32_t sv[D][T][kNv ? 2 : 1];
    u32x4 av[kGlobalA ? D : 1][4];   // NVFP4: av[j][q] = the A fragments of blocks 2q, 2q+1

    // Ring A: the group's rows go to this wavefront's LDS slot of ceil(M/4)
    // KiB as contiguous 1 KiB DMA loads (four rows each; rows >= M repeat
    // row M-1).  The matrix-core reads take rows 0..15 of the slot: rows
    // past the slot's last are the next slot's bytes (or the padding after
    // the last slot) and only reach output rows that are never stored.  Inside a
    // row the 16-byte pieces are XOR-swizzled by the row index, so the
    // matrix-core reads below (16 rows, one piece each) hit distinct banks.
    const int nd = (MM < 0) ? -MM : (M + 3) >> 2;           // DMA loads per group
    auto ring_slot = [&](int j) { return L.a + (wave * D + j) * (nd << 10); };
    // this lane's byte offset inside a group of A for DMA load i (rows
    // 4i + h, swizzled piece c), fixed for the whole loop
    uint32_t ring_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = min(4 * i + h, M - 1);
        ring_off[i] = (uint32_t)row * (uint32_t)p.K * 2u + (uint32_t)((c ^ (row & 15)) << 4);
    }
    // Split-N: one ring of P = shared_slots(D) >= D + 1 slots for the
    // workgroup; group g (the i-th of the range) in slot i % P.  Wavefront w
    // loads rows 4w .. 4w+3 of every group (rows >= M repeat row M-1), so
    // each wavefront issues exactly one DMA load per group and the wait
    // counts stay static.  The refill issued after computing group i (group
    // i + D) goes to the slot of group i + D - P <= i - 1, which every
    // wavefront has finished reading once it passed group i's barrier;
    // hence at least one spare slot.
    auto shared_slot = [&](int g) { return L.a + ((g - gk0) & (shared_slots(D) - 1)) * kRingSlotBytes; };
    const int sh_row = min(4 * wave + h, M - 1);
    const uint32_t sh_off = (uint32_t)sh_row * (uint32_t)p.K * 2u + (uint32_t)((c ^ (sh_row & 15)) << 4);

    auto load_group = [&](auto jc, int g) {
        constexpr int j = decltype(jc)::value;
        if constexpr (kRingA) {
            const uint32_t dst0 = __builtin_amdgcn_readfirstlane(lds_addr(smem + ring_slot(j)));
            const uint8_t *gbase = reinterpret_cast<const uint8_t *>(p.A) + (size_t)g * kGroup * 2;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (i < nd) lds_dma16_sbase(ring_off[i], gbase, dst0 + (i << 10));
        } else if constexpr (kSplitN) {
            const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(smem + shared_slot(g))) + (wave << 10);
            const uint8_t *gbase = reinterpret_cast<const uint8_t *>(p.A) + (size_t)g * kGroup * 2;
            lds_dma16_sbase(sh_off, gbase, dst);
        }
#pragma unroll
        for (int t = 0; t < T; ++t) {
            wv[j][t] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(wres[t], w_lane, g * 1024, kCachePolicyNt));
            if constexpr (kNv) {
                const u32x2 x = __builtin_bit_cast(
                    u32x2, __builtin_amdgcn_raw_buffer_load_b64(sres[t], s_lane, g * s_gstride, 0));
                sv[j][t][0] = x[0];
                sv[j][t][1] = x[1];
            } else {
                // the aligned dword that holds this lane's bf16 scale (a 16-bit
                // load would be re-extended at the loop latch, which stalls the ring)
                sv[j][t][0] = __builtin_amdgcn_raw_buffer_load_b32(sres[t], s_lane, g * s_gstride, 0);
            }
        }
        if constexpr (kGlobalA && kNv) {
            // rows 16b + 4h .. +3 of the group, b = 0..7: eight 8-byte pieces
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x2 lo = __builtin_bit_cast(
                    u32x2, __builtin_amdgcn_raw_buffer_load_b64(ares, a_lane + (2 * q) * kNvBlock * 2, g * kGroup * 2, 0));
                const u32x2 hi = __builtin_bit_cast(
                    u32x2, __builtin_amdgcn_raw_buffer_load_b64(ares, a_lane + (2 * q + 1) * kNvBlock * 2, g * kGroup * 2, 0));
                av[j][q] = u32x4{lo[0], lo[1], hi[0], hi[1]};
            }
        } else if constexpr (kGlobalA) {
            // A rows >= M repeat row M-1: their results land in output rows
            // that are never written, and the loads stay branch free
            const u32x4 *ap = reinterpret_cast<const u32x4 *>(abase + (size_t)g * kGroup * 2);
#pragma unroll
            for (int r = 0; r < 4; ++r) av[j][r] = ap[r];   // rows 32h + 8r .. +8: 16 B
        }
    };
    auto gat = [&](int i) { return gk0 + i; };
    auto gidx = [&](int i) { return gat(min(i, ng - 1)); };

    if (ng > 0) {
        [&]<int... J>(std::integer_sequence<int, J...>) {
            ((load_group(std::integral_constant<int, J>{}, gidx(J)),
              __builtin_amdgcn_sched_barrier(0)),
             ...);
        }(std::make_integer_sequence<int, D>{});
    }

    // ---- 3. this wavefront's A is in LDS once its own fill has landed; then
    //         the bias of each of its groups, formed by the wavefront itself
    if constexpr (kStage) {
        // this wavefront's fill is older than its ring loads (ng == 0: no ring)
        if (ng > 0)
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(D * kLoadsPerGroup));
        else
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        float *bias = reinterpret_cast<float *>(smem + L.bias);
        const int gl0 = gk0 - gw0, gl1 = gk1 - gw0;          // own groups, relative to the range
        if constexpr (kNv) {
            // exact signed weights: no bias
        } else if constexpr (PATH == PATH_GEMV) {
            // each 32-row quarter: the GEMV lane's dot2 chain with every code 8
            for (int m = 0; m < M; ++m)
            for (int rem = gl0 * 4 + lane; rem < gl1 * 4; rem += 64) {
                const int b = m * Gwg * 4 + rem;
                const u32x4 *src = reinterpret_cast<const u32x4 *>(smem + L.a + m * L.row + rem * 64);
                float s = 0.0f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const u32x4 x = src[i];
#pragma unroll
                    for (int e = 0; e < 4; ++e) s = dot2_bf16(kBiasPair, x[e], s);
                }
                bias[b] = s;
            }
        } else if constexpr (!kBiasInLoop) {
            // each group: the MFMA lanes' four-instruction chain with every code
            // 8, exactly as the main loop would form it; rows 4h..4h+3 of column
            // 0 are stored (all 16 columns are equal)
            // Four groups per pass so that four independent chains fill the
            // matrix pipeline; a pass past the last group repeats it and
            // skips the store.
            const u32x4 bconst = {kBiasPair, kBiasPair, kBiasPair, kBiasPair};
            constexpr int kB = 4;
            for (int gb = gl0; gb < gl1; gb += kB) {
                u32x4 a[kB][4];
#pragma unroll
                for (int i = 0; i < kB; ++i) {
                    const int gl = min(gb + i, gl1 - 1);
                    const uint8_t *arow = smem + L.a + arow_m * L.row + (gl * kGroup + h * 32) * 2;
#pragma unroll
                    for (int r = 0; r < 4; ++r) a[i][r] = reinterpret_cast<const u32x4 *>(arow)[r];
                }
                f32x4 Q[kB];
#pragma unroll
                for (int i = 0; i < kB; ++i) Q[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int i = 0; i < kB; ++i) Q[i] = mfma16x16x32(a[i][r], bconst, Q[i]);
#pragma unroll
                for (int i = 0; i < kB; ++i) {
                    const int gl = gb + i;
                    if (c == 0 && gl < gl1) reinterpret_cast<f32x4 *>(bias)[gl * 4 + h] = Q[i];
                }
            }
        }
        // the wavefront's own LDS writes precede its reads (LDS operations of
        // one wavefront complete in order); keep the compiler from moving
        // the reads above the writes
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        asm volatile("" ::: "memory");
    }

    // ---- 4. main loop over this wavefront's groups
    constexpr int NACC = (PATH == PATH_GEMV) ? MM : kRowsV;
    float acc[T][NACC];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int i = 0; i < NACC; ++i) acc[t][i] = 0.0f;

    // later_c: how many younger groups have their loads in flight when this
    // slot is computed (the explicit waits for DMA loads count on it)
    auto compute_group = [&](auto jc, int g, auto later_c) {
        constexpr int j = decltype(jc)::value;
        const int gl = g - gw0;
        if constexpr (kNv) {
            // Eight 16-row blocks per group; each block's partial sum is
            // scaled by its E4M3 scale and added, so converted weights stay
            // exact and no bias arises.
            if constexpr (PATH == PATH_MFMA) {
                // A fragments: row arow_m, rows 16b + 4h .. +3 of the group
                u32x2 a[8];
                if constexpr (kStage) {
                    const uint8_t *arow = smem + L.a + arow_m * L.row + (gl * kGroup + 4 * h) * 2;
#pragma unroll
                    for (int b = 0; b < 8; ++b) a[b] = *reinterpret_cast<const u32x2 *>(arow + b * kNvBlock * 2);
                } else if constexpr (kRingA || kSplitN) {
                    // as for GPTQ: wait for this slot's DMA loads explicitly;
                    // rows 16b + 4h .. +3 are bytes 32b + 8h of row c, in
                    // logical piece 2b + h/2, stored at piece (2b + h/2) ^ c
                    constexpr int later = decltype(later_c)::value;
                    __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * T + later * (2 * T + 1)));
                    if constexpr (kSplitN) wg_barrier();   // every wavefront's rows have landed
                    const uint8_t *slot = smem + (kSplitN ? shared_slot(g) : ring_slot(j)) + c * (kGroup * 2) +
                                          ((h & 1) << 3);
#pragma unroll
                    for (int b = 0; b < 8; ++b)
                        a[b] = *reinterpret_cast<const u32x2 *>(slot + (((2 * b + (h >> 1)) ^ c) << 4));
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        a[2 * q] = u32x2{av[j][q][0], av[j][q][1]};
                        a[2 * q + 1] = u32x2{av[j][q][2], av[j][q][3]};
                    }
                }
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    float scl[8];
                    nv_scales(sv[j][t], scl);
                    [&]<int... B>(std::integer_sequence<int, B...>) {
                        (([&] {
                             const f32x4 P = mfma16x16x16(a[B], nv_block<B>(wv[j][t]), f32x4{0.0f, 0.0f, 0.0f, 0.0f});
                             const float sc = scl[B];
#pragma unroll
                             for (int v = 0; v < kRowsV; ++v) acc[t][v] = __builtin_fmaf(sc, P[v], acc[t][v]);
                         }()),
                         ...);
                    }(std::make_integer_sequence<int, 8>{});
                }
            } else {
                // GEMV: per block, two dot2 per row on the lane's four rows,
                // then the scale
                float scl[T][8];
#pragma unroll
                for (int t = 0; t < T; ++t) nv_scales(sv[j][t], scl[t]);
                [&]<int... B>(std::integer_sequence<int, B...>) {
                    (([&] {
                         u32x2 ar[MM];
#pragma unroll
                         for (int m = 0; m < MM; ++m)
                             ar[m] = *reinterpret_cast<const u32x2 *>(smem + L.a + m * L.row +
                                                                     (gl * kGroup + B * kNvBlock + 4 * h) * 2);
#pragma unroll
                         for (int t = 0; t < T; ++t) {
                             const u32x2 w = nv_block<B>(wv[j][t]);
                             const float sc = scl[t][B];
#pragma unroll
                             for (int m = 0; m < MM; ++m) {
                                 const float part = dot2_bf16(w[1], ar[m][1], dot2_bf16(w[0], ar[m][0], 0.0f));
                                 acc[t][m] = __builtin_fmaf(sc, part, acc[t][m]);
                             }
                         }
                     }()),
                     ...);
                }(std::make_integer_sequence<int, 8>{});
            }
        } else if constexpr (PATH == PATH_MFMA) {
            u32x4 a[4];
            f32x4 Q;
            if constexpr (kStage) {
                const uint8_t *arow = smem + L.a + arow_m * L.row + (gl * kGroup + h * 32) * 2;
#pragma unroll
                for (int r = 0; r < 4; ++r) a[r] = reinterpret_cast<const u32x4 *>(arow)[r];
                if constexpr (kBiasInLoop) {
                    const u32x4 bconst = {kBiasPair, kBiasPair, kBiasPair, kBiasPair};
                    Q = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int r = 0; r < 4; ++r) Q = mfma16x16x32(a[r], bconst, Q);
                } else {
                    Q = reinterpret_cast<const f32x4 *>(smem + L.bias)[gl * 4 + h];
                }
            } else {
                if constexpr (kRingA || kSplitN) {
                    // the compiler does not see the DMA loads: wait for this
                    // slot's explicitly (every load issued after them counted
                    // as if each later group had one DMA load: never fewer)
                    constexpr int later = decltype(later_c)::value;
                    __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * T + later * (2 * T + 1)));
                    if constexpr (kSplitN) wg_barrier();   // every wavefront's rows have landed
                    const uint8_t *slot = smem + (kSplitN ? shared_slot(g) : ring_slot(j)) + c * (kGroup * 2);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        a[r] = *reinterpret_cast<const u32x4 *>(slot + (((h * 4 + r) ^ c) << 4));
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) a[r] = av[j][r];
                }
                // bias: the same four-MFMA chain with every code 8
                const u32x4 bconst = {kBiasPair, kBiasPair, kBiasPair, kBiasPair};
                Q = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int r = 0; r < 4; ++r) Q = mfma16x16x32(a[r], bconst, Q);
            }
#pragma unroll
            for (int t = 0; t < T; ++t) {
                f32x4 P = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int rp = 0; rp < 2; ++rp) {
                    uint32_t b0[4], b1[4];
                    words_to_bf16x8<false>(wv[j][t][2 * rp], wv[j][t][2 * rp + 1], kc, b0, b1);
                    P = mfma16x16x32(a[2 * rp], u32x4{b0[0], b0[1], b0[2], b0[3]}, P);
                    P = mfma16x16x32(a[2 * rp + 1], u32x4{b1[0], b1[1], b1[2], b1[3]}, P);
                }
                const float s = scale_from(sv[j][t][0], s_sel);
#pragma unroll
                for (int v = 0; v < kRowsV; ++v) acc[t][v] = __builtin_fmaf(s, P[v] - Q[v], acc[t][v]);
            }
        } else {
            // Word pairs outermost (they share their shifts), then r: one
            // 16-byte A sub-block per row is live at a time.  Per (tile, row)
            // the dot2 chain runs r = 0..3, v = 0..3, the same order the bias
            // was formed in.
            float part[T][MM];
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int m = 0; m < MM; ++m) part[t][m] = 0.0f;
#pragma unroll
            for (int rp = 0; rp < 2; ++rp) {
                uint32_t b[T][2][4];
#pragma unroll
                for (int t = 0; t < T; ++t)
                    words_to_bf16x8<true>(wv[j][t][2 * rp], wv[j][t][2 * rp + 1], kc, b[t][0], b[t][1]);
#pragma unroll
                for (int rr = 0; rr < 2; ++rr) {
                    const int r = 2 * rp + rr;
                    u32x4 ar[MM];
#pragma unroll
                    for (int m = 0; m < MM; ++m)
                        ar[m] = reinterpret_cast<const u32x4 *>(smem + L.a + m * L.row +
                                                               (gl * kGroup + h * 32) * 2)[r];
#pragma unroll
                    for (int t = 0; t < T; ++t)
#pragma unroll
                        for (int v = 0; v < 4; ++v)
#pragma unroll
                            for (int m = 0; m < MM; ++m)
                                part[t][m] = dot2_bf16(b[t][rr][v], ar[m][v], part[t][m]);
                }
            }
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const float s = scale_from(sv[j][t][0], s_sel);
#pragma unroll
                for (int m = 0; m < MM; ++m) {
                    const float corr = reinterpret_cast<const float *>(smem + L.bias)[(m * Gwg + gl) * 4 + h];
                    acc[t][m] = __builtin_fmaf(s, part[t][m] - corr, acc[t][m]);
                }
            }
        }
    };

    using Full = std::integral_constant<int, D - 1>;   // every younger slot in flight
    // (The NVFP4 matrix-core kernels keep the clamped refills for fewer
    // groups than slots: the extra code path crashes this compiler's
    // AGPR-copy rewrite pass on some of their shapes.)
    constexpr bool kFewerThanSlots = !kNv || PATH == PATH_GEMV;
    // One full round: compute each slot, refill it with the group D ahead.
    auto full_round = [&](int base) {
        [&]<int... J>(std::integer_sequence<int, J...>) {
            ((compute_group(std::integral_constant<int, J>{}, gat(base + J), Full{}),
              load_group(std::integral_constant<int, J>{}, gat(base + J + D)),
              __builtin_amdgcn_sched_barrier(0)),
             ...);
        }(std::make_integer_sequence<int, D>{});
    };
    // The last groups, with RT of the last round's refills still real
    // (0 <= RT < D): the round computes its D slots and refills only the
    // first RT of them, then those RT are computed.  Every load issued is a
    // real group, and each wait count is still a compile-time constant.
    auto tail = [&](auto rtc, int base) {
        constexpr int RT = decltype(rtc)::value;
        [&]<int... J>(std::integer_sequence<int, J...>) {
            (([&] {
                 // younger loads: slots J+1..D-1 of the previous round, and
                 // this round's refills of slots 0..min(J, RT)-1
                 compute_group(std::integral_constant<int, J>{}, gat(base + J),
                               std::integral_constant<int, (D - 1 - J) + (J < RT ? J : RT)>{});
                 if constexpr (J < RT) load_group(std::integral_constant<int, J>{}, gat(base + J + D));
                 __builtin_amdgcn_sched_barrier(0);
             }()),
             ...);
        }(std::make_integer_sequence<int, D>{});
        [&]<int... J>(std::integer_sequence<int, J...>) {
            (([&] {
                 if constexpr (J < RT)
                     compute_group(std::integral_constant<int, J>{}, gat(base + D + J),
                                   std::integral_constant<int, RT - 1 - J>{});
             }()),
             ...);
        }(std::make_integer_sequence<int, D>{});
    };

    if (ng > 0) {
        if (ng % D == 0 || (D <= 4 && ng > D)) {
            // exact: every refill is a real group.  Full rounds while two
            // rounds' groups remain, then the tail for the remainder (one of
            // D compiled tails; shallow rings only, for code size).
            int base = 0;
            for (; base + 2 * D <= ng; base += D) full_round(base);
            const int rt = ng - base - D;
            [&]<int... R>(std::integer_sequence<int, R...>) {
                ((rt == R ? tail(std::integral_constant<int, R>{}, base) : void()), ...);
            }(std::make_integer_sequence<int, (D <= 4 ? D : 1)>{});
        } else if (kFewerThanSlots && ng < D) {
            // fewer groups than slots: the prologue loaded every group (its
            // slots past the last re-read the last group); compute them, no
            // refills
            [&]<int... J>(std::integer_sequence<int, J...>) {
                ((J < ng ? compute_group(std::integral_constant<int, J>{}, gat(J),
                                         std::integral_constant<int, D - 1 - J>{})
                         : void()),
                 ...);
            }(std::make_integer_sequence<int, D>{});
        } else {
            // ragged deep rings: past the last group the refill re-reads the
            // last group (clamped; it is in flight or in L2 already), so every
            // iteration issues the same loads and the wait counts stay static
            for (int base = 0; base < ng; base += D) {
                [&]<int... J>(std::integer_sequence<int, J...>) {
                    ((base + J < ng ? compute_group(std::integral_constant<int, J>{}, gat(base + J), Full{})
                                    : void(),
                      load_group(std::integral_constant<int, J>{}, gidx(base + J + D)),
                      __builtin_amdgcn_sched_barrier(0)),
                     ...);
                }(std::make_integer_sequence<int, D>{});
            }
        }
    }

    // ---- GEMV: sum the four K quarters of each column across lanes
    if constexpr (PATH == PATH_GEMV) {
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int m = 0; m < MM; ++m) acc[t][m] = sum_quarters(acc[t][m]);
    }

    // ---- 5. epilogue: fixed-order reduction over wavefronts, then C, the
    //         gate/up output, or split-K partials
    //
    // Gate/up epilogue: H[m][j] = silu(C[m][j]) * C[m][j + N/2] for
    // j < N/2, silu(x) = x / (1 + exp(-x)), on the fp32 sums, one bf16
    // rounding at the end; H has N/2 columns.
    const int NV = T * M * 16;   // values (t, m, c) of this workgroup
    auto col_of = [&](int t, int cc) { return (size_t)tile_of(t) * 16 + cc; };
    // NVFP4: the per-tensor factor multiplies every finished sum before its
    // epilogue (rounding, activation, argmax key)
    auto fin = [&](float v) {
        if constexpr (kNv) return v * p.alpha;
        else return v;
    };
    auto emit_c = [&](int t, int m, int cc, float val) {      // plain, one split
        val = fin(val);
        if (fuse == 3)
            reinterpret_cast<float *>(p.C)[(size_t)m * p.N + col_of(t, cc)] = val;
        else
            p.C[(size_t)m * p.N + col_of(t, cc)] = f32_to_bf16_rne(val);
    };
    auto emit_h = [&](int t, int m, int cc, float g, float u) {   // gate/up, one split
        g = fin(g);
        u = fin(u);
        const float hv = g / (1.0f + expf(-g)) * u;
        p.C[(size_t)m * (p.N >> 1) + col_of(t, cc)] = f32_to_bf16_rne(hv);
    };
    auto emit_part = [&](int t, int m, int cc, float val) {   // split-K partial
        // device-coherent store (the XCDs' L2s are not coherent with each other)
        __hip_atomic_store(&p.part[((size_t)z * M + m) * p.N + col_of(t, cc)], val, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    };

    if constexpr (KWR == 1) {
        // lane (c, h) holds rows 4h + v (MFMA) or, in lanes h == 0, all rows (GEMV)
        auto row_val = [&](int t, int i) { return acc[t][i]; };
        constexpr int kRows = (PATH == PATH_MFMA) ? kRowsV : MM;
        const bool holder = (PATH == PATH_MFMA) || h == 0;
        auto row_of = [&](int i) { return PATH == PATH_MFMA ? 4 * h + i : i; };
        if (fuse == 2) {
            unsigned long long *keys = reinterpret_cast<unsigned long long *>(smem + L.keys);
            if (threadIdx.x < 16) keys[threadIdx.x] = 0ull;
            lds_barrier();
            if (holder) {
#pragma unroll
                for (int t = 0; t < T; ++t)
#pragma unroll
                    for (int i = 0; i < kRows; ++i)
                        if (row_of(i) < M && tile_ok(t))
                            __hip_atomic_fetch_max(&keys[row_of(i)], argmax_key(fin(row_val(t, i)), (uint32_t)col_of(t, c)),
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        } else if (holder) {
            if (split || fuse != 1) {
#pragma unroll
                for (int t = 0; t < T; ++t)
#pragma unroll
                    for (int i = 0; i < kRows; ++i)
                        if (row_of(i) < M && tile_ok(t)) {
                            if (split) emit_part(t, row_of(i), c, row_val(t, i));
                            else emit_c(t, row_of(i), c, row_val(t, i));
                        }
            } else {
#pragma unroll
                for (int t = 0; t < kHalfT; ++t)
#pragma unroll
                    for (int i = 0; i < kRows; ++i)
                        if (row_of(i) < M && tile_ok(t))
                            emit_h(t, row_of(i), c, row_val(t, i), row_val(t + kHalfT, i));
            }
        }
    } else {
        float *red = reinterpret_cast<float *>(smem + L.red);
        float *mine = red + wave * NV;
#pragma unroll
        for (int t = 0; t < T; ++t) {
            if constexpr (PATH == PATH_MFMA) {
#pragma unroll
                for (int v = 0; v < kRowsV; ++v)
                    if (4 * h + v < M) mine[(t * M + 4 * h + v) * 16 + c] = acc[t][v];
            } else {
                if (h == 0) {
#pragma unroll
                    for (int m = 0; m < MM; ++m) mine[(t * MM + m) * 16 + c] = acc[t][m];
                }
            }
        }
        lds_barrier();   // LDS only: the clamped refills still in flight need no wait
        auto reduced = [&](int t, int mc) {
            const int e = t * M * 16 + mc;
            float s = red[e];
#pragma unroll
            for (int w = 1; w < KW; ++w) s += red[w * NV + e];
            return s;
        };
        if (fuse == 2) {
            unsigned long long *keys = reinterpret_cast<unsigned long long *>(smem + L.keys);
            if (threadIdx.x < 16) keys[threadIdx.x] = 0ull;
            lds_barrier();
#pragma unroll
            for (int t = 0; t < T; ++t)
                for (int mc = threadIdx.x; mc < M * 16; mc += 64 * KW) {
                    if (!tile_ok(t)) continue;
                    __hip_atomic_fetch_max(&keys[mc >> 4], argmax_key(fin(reduced(t, mc)), (uint32_t)col_of(t, mc & 15)),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                }
        } else if (split || fuse != 1) {
#pragma unroll
            for (int t = 0; t < T; ++t)
                for (int mc = threadIdx.x; mc < M * 16; mc += 64 * KW) {
                    if (!tile_ok(t)) continue;
                    const float s = reduced(t, mc);
                    if (split) emit_part(t, mc >> 4, mc & 15, s);
                    else emit_c(t, mc >> 4, mc & 15, s);
                }
        } else {
#pragma unroll
            for (int t = 0; t < kHalfT; ++t)
                for (int mc = threadIdx.x; mc < M * 16; mc += 64 * KW) {
                    if (!tile_ok(t)) continue;
                    emit_h(t, mc >> 4, mc & 15, reduced(t, mc), reduced(t + kHalfT, mc));
                }
        }
    }

    if (fuse == 2) {
        // Row argmax across workgroups (single split): this workgroup's row
        // maxima go to its bin with device-scope 64-bit max atomics, issued
        // and not waited for; the fold kernel that follows on the stream
        // reads the bins.  Max is order-independent: the result does not
        // depend on timing.
        unsigned long long *keys = reinterpret_cast<unsigned long long *>(smem + L.keys);
        unsigned long long *bins =
            reinterpret_cast<unsigned long long *>(reinterpret_cast<uint8_t *>(p.count) + kArgmaxBinOffset);
        lds_barrier();
        if (threadIdx.x < (unsigned)M)
            __hip_atomic_fetch_max(&bins[(blockIdx.x % kArgmaxBins) * 16 + threadIdx.x], keys[threadIdx.x],
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }

    if (split) {
        // Hand-off between the S workgroups of a strip without flushing any
        // L2.  Every partial is written with an agent-scope atomic store,
        // which gfx950 writes through its XCD's L2 to the device-coherent
        // level; the wait for vmcnt 0 returns once each of this thread's
        // stores is acknowledged there.  Only then, after the workgroup
        // barrier, does one thread increment the strip's counter (an
        // agent-scope RMW, performed at that same level).  The last to
        // arrive reads the S partials with agent-scope atomic loads, which
        // do not take a stale line from its own L2, and adds them in the
        // fixed order z = 0..S-1.  An agent-scope release/acquire pair would
        // add a write-back of this XCD's whole L2 and an invalidate of it,
        // both of which only matter for data written or read with ordinary
        // (non-atomic) accesses, and there is none in this exchange.  The
        // signal fences keep the compiler from moving memory accesses across
        // the wait and the counter; they emit no instruction.
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_barrier();
        if (threadIdx.x == 0) {
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            const uint32_t prev = __hip_atomic_fetch_add(&p.count[strip], 1u, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            s_last = (prev == (uint32_t)(p.S - 1));
        }
        wg_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (s_last) {
            // The S partials of an output are added in the fixed order
            // z = 0..S-1.  Every load of a batch (eight partials of two
            // outputs; past z = S-1 the index is clamped and the value
            // unused) is issued before the first add, so the batch costs one
            // round trip to the device-coherent level instead of one per
            // partial.
            constexpr int kB = 8;
            const size_t zstride = (size_t)M * p.N;
            auto load_b = [&](size_t col, int m, int z0, float (&v)[kB]) {
                const float *src = p.part + (size_t)m * p.N + col;
#pragma unroll
                for (int i = 0; i < kB; ++i)
                    v[i] = __hip_atomic_load(src + (size_t)min(z0 + i, p.S - 1) * zstride, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
            };
            auto add_b = [&](const float (&v)[kB], int z0, float s) {
#pragma unroll
                for (int i = 0; i < kB; ++i)
                    if (z0 + i < p.S) s += v[i];
                return s;
            };
            // split-N: each wavefront adds its own tiles
            const int mc0 = kSplitN ? lane : (int)threadIdx.x;
            constexpr int kMcStep = kSplitN ? 64 : 64 * KW;
            // outputs e = t * 16M + mc of this thread, two at a time; gate/up:
            // the gate tile t and its up tile t + T/2 together
            const int nT = fuse == 1 ? kHalfT : T;
            const int ne = nT * M * 16;
            for (int e0 = mc0; e0 < ne; e0 += 2 * kMcStep) {
                int te[2], me[2], ce[2];
                size_t col0[2], col1[2];   // plain (or gate) column, and the up column
                bool live[2];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int e = min(e0 + q * kMcStep, ne - 1);
                    te[q] = e / (M * 16);
                    me[q] = (e % (M * 16)) >> 4;
                    ce[q] = e & 15;
                    live[q] = e0 + q * kMcStep < ne && tile_ok(te[q]);
                    // an output that is not written still loads, from column 0
                    col0[q] = live[q] ? col_of(te[q], ce[q]) : 0;
                    col1[q] = live[q] && fuse == 1 ? col_of(te[q] + kHalfT, ce[q]) : 0;
                }
                float s0[2] = {0.0f, 0.0f}, s1[2] = {0.0f, 0.0f};
                for (int z0 = 0; z0 < p.S; z0 += kB) {
                    float v0[2][kB], v1[2][kB];
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        load_b(col0[q], me[q], z0, v0[q]);
                        if (fuse == 1) load_b(col1[q], me[q], z0, v1[q]);
                    }
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        s0[q] = add_b(v0[q], z0, s0[q]);
                        if (fuse == 1) s1[q] = add_b(v1[q], z0, s1[q]);
                    }
                }
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    if (!live[q]) continue;
                    if (fuse == 1) emit_h(te[q], me[q], ce[q], s0[q], s1[q]);
                    else emit_c(te[q], me[q], ce[q], s0[q]);
                }
            }
            if (threadIdx.x == 0)
                __hip_atomic_store(&p.count[strip], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

}  // namespace w4a16
