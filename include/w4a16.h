/*
 * w4a16.h - C ABI of a gfx950 (MI355X) library for the weight-only INT4
 * decode/verify matmul
 *
 *     C[M, N] = A[M, K] . dequant(Wq)[K, N],   1 <= M <= 16,
 *
 * with BF16 activations A, BF16 output C and weights Wq in the symmetric GPTQ
 * 4-bit format: group size 128 along K, no zero points, no act-order.  That
 * checkpoint contract is stated on the page "Qwen3.8-27B on single DGX Spark
 * ..." (section "Quality."); the same page (section "How.") describes the
 * backbone and output-projection matmuls as kernels dispatched by row count,
 * and the page "One Config Line Made My 27B Model 2.7x Faster" (section "The
 * fix: use the MTP head you already downloaded") explains why decode calls it
 * with one row and speculative verify with a handful of rows.
 *
 * Formats
 *   qweight  uint32 [K/8][N], N contiguous.  Nibble j of word (kb, n), i.e.
 *            bits 4j..4j+3 (low nibble first), is the code q in [0, 15] of
 *            row k = 8*kb + j.  The weight is w = (q - 8) * s.
 *   scales   bf16 [K/128][N], N contiguous: s for (group floor(k/128), column n),
 *            exactly as the checkpoint stores them.  The GEMM reads them in
 *            place (tile t's 16 scales of group g are the 32 bytes at
 *            g*2N + 32t); they are never repacked.
 *   A        bf16 [M][K], K contiguous (row stride K).
 *   C        bf16 [M][N], N contiguous (row stride N); fp32 accumulation,
 *            rounded to nearest even once at the end.
 *   blob     the repacked weights: exactly K*N/2 bytes.  Layout: 16-byte
 *            pieces; piece (t, g, h, c) at piece index ((t*G + g)*4 + h)*16 + c
 *            (G = K/128) holds column n = 16t + c, rows k = 128g + 32h + 8r + e
 *            in its word r = 0..3; inside a word the code of row offset e sits
 *            at bit 4*(e/2) for even e and 16 + 4*(e/2) for odd e.
 *
 * Conventions shared by every entry point
 *   - Every pointer argument except `stream` is DEVICE memory owned by the
 *     caller.  The library allocates nothing and keeps no state between calls
 *     other than a lazily filled cache of device properties.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     is asynchronous: a return of W4A16_OK means the launch was accepted,
 *     not that the kernel has finished.  Nothing synchronizes.
 *   - Arguments are validated before any device work; an invalid call returns
 *     a negative status and enqueues nothing.  No call aborts the process and
 *     no unsupported case falls back silently to another path.
 *   - Device pointers must be 16-byte aligned.  Output buffers must not
 *     overlap any input (not checked).
 *   - Valid shapes: 1 <= M <= 16, K a positive multiple of 128 up to
 *     W4A16_MAX_K (2^24; the kernels address a tile's weights and the rows of
 *     A through 32-bit buffer offsets), N a positive multiple of 16,
 *     K*N/2 < 2^40, (K/128)*N*2 < 2^31 (the scales are addressed with 32-bit
 *     byte offsets).  group must be 128.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every int-valued entry point. */
#define W4A16_OK              0
#define W4A16_ERR_NULL       -1   /* a required pointer is NULL */
#define W4A16_ERR_SHAPE      -2   /* M, N or K outside the valid set */
#define W4A16_ERR_GROUP      -3   /* group != 128 */
#define W4A16_ERR_ALIGN      -4   /* a device pointer is not 16-byte aligned */
#define W4A16_ERR_WORKSPACE  -5   /* the plan needs a workspace that is missing or too small */
#define W4A16_ERR_DEVICE     -6   /* no HIP device, or the current device is not gfx950 */
#define W4A16_ERR_LAUNCH     -7   /* the HIP runtime rejected a launch */
#define W4A16_ERR_PLAN       -8   /* an explicit plan names a kernel shape the library does not have */

#define W4A16_GROUP 128
#define W4A16_NVFP4_GROUP 16   /* rows per E4M3 block scale of the NVFP4 calls */
#define W4A16_MAX_M 16
#define W4A16_MAX_K (1 << 24)

/* Execution paths of the row-count dispatcher. */
#define W4A16_PATH_AUTO 0
#define W4A16_PATH_GEMV 1   /* VALU dot products, cross-lane reduction (small M) */
#define W4A16_PATH_MFMA 2   /* bf16 matrix cores, 16x16x32 tiles (larger M) */

/* Where the MFMA path takes its A operand from. */
#define W4A16_ASRC_LDS    0  /* staged once per workgroup in LDS */
#define W4A16_ASRC_GLOBAL 1  /* read per group from global memory (L1/L2) */
#define W4A16_ASRC_RING   2  /* per group through a per-wavefront LDS ring (DMA) */
#define W4A16_ASRC_SPLITN 3  /* staged once per workgroup in LDS; the wavefronts split
                                the columns instead of K (kwaves x tiles tiles share it) */

/*
 * A launch plan.  w4a16_gemm chooses one from (M, N, K); w4a16_gemm_plan
 * runs an explicit one (tests force each path with it).
 *   path    W4A16_PATH_GEMV or W4A16_PATH_MFMA
 *   tiles   16-column tiles per wavefront (1, 2 or 4)
 *   kwaves  wavefronts of one workgroup that split the workgroup's K range
 *           (with W4A16_ASRC_SPLITN: that split its columns, tiles each)
 *   splits  workgroups that split K for the same columns: 1 (none), 2, 4, 8, ...
 *           (a power of two); more than one needs a workspace (see
 *           w4a16_workspace_bytes_plan)
 *   asrc    W4A16_ASRC_LDS, W4A16_ASRC_GLOBAL, W4A16_ASRC_RING or
 *           W4A16_ASRC_SPLITN (the last three on the MFMA path only)
 *   depth   K groups each wavefront keeps in flight (0 = the default for
 *           `tiles`: 8, 4, 2 for 1, 2, 4 tiles)
 *   whole   with splits > 1: the number of leading column strips that one
 *           workgroup computes whole; only the strips after them are split
 *           `splits` ways (0: every strip is split).  A narrow matrix whose
 *           strips outnumber the CUs by a remainder gives each CU one whole
 *           strip and one piece of the remainder this way.  Ignored when
 *           splits == 1.
 */
typedef struct {
    int path;
    int tiles;
    int kwaves;
    int splits;
    int asrc;
    int depth;
    int whole;
} w4a16_plan_t;

/* Human-readable name of a status code (static storage, never NULL). */
const char *w4a16_status_string(int status);

/* Bytes of the repacked blob for a K x N matrix (= K*N/2), 0 for invalid shapes. */
size_t w4a16_repacked_bytes(int K, int N);

/*
 * One-time repack of GPTQ words into the blob layout described above, the
 * only preparation a checkpoint needs: its scales are used as they are.
 * The input is the checkpoint format of the page "Qwen3.8-27B on single DGX
 * Spark ..." (section "Quality.": symmetric GPTQ, 4-bit, group 128, no
 * act-order, no zero points); the blob order is this library's own, chosen
 * so that one wavefront loads one 16-column x 128-row piece with a single
 * 16-byte load per lane.
 *   qweight      device, uint32 [K/8][N] as in the header comment (read only)
 *   wq_repacked  device, w4a16_repacked_bytes(K, N) bytes (written)
 * A pure permutation of nibbles: every code is moved, none is changed.
 * Returns W4A16_OK, or W4A16_ERR_NULL / _SHAPE / _ALIGN / _DEVICE / _LAUNCH
 * (nothing is enqueued on an error).
 */
int w4a16_repack_weights(const void *qweight, void *wq_repacked, int K, int N, void *stream);

/*
 * The plan w4a16_gemm uses for (M, N, K): the row-count dispatch of the page
 * "Qwen3.8-27B on single DGX Spark ..." (section "How.": the matmuls are
 * kernels dispatched by row count), extended here by the column and K
 * shape.  Fills *plan and returns W4A16_OK, or returns an error status for
 * invalid shapes.  Host-only, no device work.
 */
int w4a16_get_plan(int M, int N, int K, w4a16_plan_t *plan);

/*
 * W4A16_OK if the library can run `plan` for (M, N, K) (a kernel exists and
 * its LDS fits), W4A16_ERR_PLAN if not, W4A16_ERR_SHAPE for invalid shapes.
 * A plan is one arm of the row-count dispatch (same page and section as
 * w4a16_get_plan).  Host-only, no device work.
 */
int w4a16_check_plan(int M, int N, int K, const w4a16_plan_t *plan);

/*
 * Split-K workspace layout, the same for every shape and plan:
 *   bytes [0, W4A16_SPLIT_COUNTER_BYTES)   32-bit arrival counters, one per
 *                                          column strip (strip s at index s)
 *   bytes [W4A16_SPLIT_COUNTER_BYTES, ...) fp32 partials [splits][M][N]
 * A plan with splits > 1 may have at most W4A16_SPLIT_COUNTER_BYTES / 4
 * column strips (ceil(N / 16 / tiles)).
 */
#define W4A16_SPLIT_COUNTER_BYTES 65536

/*
 * Workspace bytes that serve every call at (M, N, K) with its automatic plan
 * (w4a16_gemm, w4a16_gemm_f32, w4a16_gemm_silu_mul, w4a16_gemm_argmax): at
 * least W4A16_SPLIT_COUNTER_BYTES, plus the split-K partials
 * 4 * splits * M * N when a plan splits K.  0 for invalid shapes.
 * A workspace must be zero-filled before its first use.  Every call leaves
 * the counter region zero again and writes partials only after it, so one
 * workspace serves calls of any shape and plan issued one after another
 * (stream order); calls that share a workspace must not run concurrently.
 * Calls whose plan needs no workspace accept NULL.  No page defines a
 * workspace: it holds this library's split-K partials, which the row-count
 * dispatch (page "Qwen3.8-27B on single DGX Spark ...", section "How.")
 * uses for narrow matrices.
 */
size_t w4a16_workspace_bytes(int M, int N, int K);

/*
 * Workspace bytes one plan needs: W4A16_SPLIT_COUNTER_BYTES plus
 * 4 * splits * M * N, or 0 when splits == 1.  plan == NULL means the plan
 * w4a16_gemm would choose.  Returns 0 for invalid arguments.
 */
size_t w4a16_workspace_bytes_plan(int M, int N, int K, const w4a16_plan_t *plan);

/*
 * C = A . dequant(blob, scales), dispatched by row count: the backbone and
 * output-projection matmul of the page "Qwen3.8-27B on single DGX Spark ..."
 * (section "How.": kernels dispatched by row count; M = 1 is a decode step,
 * M > 1 the rows a speculative verify adds, page "One Config Line Made My 27B
 * Model 2.7x Faster", section "The fix: use the MTP head you already
 * downloaded"), on weights of the checkpoint contract (same first page,
 * section "Quality.").
 *   A            device bf16 [M][K]
 *   wq_repacked  device blob from w4a16_repack_weights for this K, N
 *   scales       device bf16 [K/128][N], the checkpoint's scales
 *   C            device bf16 [M][N] (written)
 *   group        must be 128
 *   workspace    device, at least w4a16_workspace_bytes(M, N, K) bytes,
 *                zero-filled before first use; may be NULL when the plan
 *                needs none (w4a16_workspace_bytes_plan(M, N, K, NULL) == 0)
 * Returns W4A16_OK or a negative status (nothing is enqueued on an error).
 * Deterministic: the same arguments give bitwise the same C.
 */
int w4a16_gemm(const void *A, const void *wq_repacked, const void *scales, void *C,
               int M, int N, int K, int group, void *workspace, size_t workspace_bytes,
               void *stream);

/*
 * As w4a16_gemm (same passages), with an explicit plan: one arm of the
 * row-count dispatch of the page "Qwen3.8-27B on single DGX Spark ..."
 * (section "How.") chosen by the caller (plan == NULL: same as w4a16_gemm).
 * Returns W4A16_ERR_PLAN when the library has no kernel for the plan.
 */
int w4a16_gemm_plan(const void *A, const void *wq_repacked, const void *scales, void *C,
                    int M, int N, int K, int group, void *workspace, size_t workspace_bytes,
                    const w4a16_plan_t *plan, void *stream);

/*
 * Allocation-free form of w4a16_gemm_plan (plan == NULL: the plan w4a16_gemm
 * chooses, or, where that plan's split-K partials would not fit the array
 * below, the same plan with every strip whole), for callers that cannot
 * allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.
 * Instead of a caller's workspace, the split-K counters and partials live in
 * a static device array of W4A16_NOALLOC_SCRATCH_BYTES that each GPU the
 * library runs on holds until the process ends.  The call allocates and
 * frees nothing.  Its first call on a GPU finds the array's address and
 * clears its counter region with a kernel on `stream`; every call leaves the
 * counters zero.  All calls on one GPU share the one array, so calls that
 * overlap in time on one GPU (different streams, concurrent graph replays)
 * race and must not be issued.  A plan whose workspace would exceed the
 * array returns W4A16_ERR_WORKSPACE; other arguments and errors as
 * w4a16_gemm_plan.
 */
#define W4A16_NOALLOC_SCRATCH_BYTES (W4A16_SPLIT_COUNTER_BYTES + (4 << 20))
int w4a16_gemm_noalloc(const void *A, const void *wq_repacked, const void *scales, void *C,
                       int M, int N, int K, int group, const w4a16_plan_t *plan, void *stream);

/*
 * Gate/up matmul with the MLP activation in its epilogue:
 *
 *     C = A . dequant(blob, scales)              (C[M][N], never stored)
 *     H[m][j] = silu(C[m][j]) * C[m][j + N/2],   0 <= j < N/2,
 *     silu(x) = x / (1 + exp(-x)),
 *
 * for a fused gate/up weight whose first N/2 columns are the gate linear and
 * last N/2 the up linear of one MLP (each layer's MLP has gate, up and down
 * linears: page "SuperQwen3.8-27b-abliterated-NVFP4-2xDGX", the structural
 * verification of its packed tensors; the pages do not name the activation,
 * and SiLU-gated is the reading taken).  H feeds the down projection.
 * silu and the product are formed in fp32 on the fp32 sums; H is rounded to
 * bf16 (nearest even) once.
 *   H            device bf16 [M][N/2] (written)
 *   N            the fused width, a multiple of 32
 *   other arguments as w4a16_gemm (blob and scales of the [K][N] fused
 *   weight; workspace at least w4a16_workspace_bytes(M, N, K)).
 * The plan w4a16_gemm would choose is used with an even tile count (gate
 * and up tiles of the same columns in one workgroup).
 */
int w4a16_gemm_silu_mul(const void *A, const void *wq_repacked, const void *scales, void *H,
                        int M, int N, int K, int group, void *workspace, size_t workspace_bytes,
                        void *stream);

/*
 * As w4a16_gemm_silu_mul (same passages) with an explicit plan of the
 * row-count dispatch, whose tile count must be even (W4A16_ERR_PLAN
 * otherwise).
 */
int w4a16_gemm_silu_mul_plan(const void *A, const void *wq_repacked, const void *scales, void *H,
                             int M, int N, int K, int group, void *workspace,
                             size_t workspace_bytes, const w4a16_plan_t *plan, void *stream);

/*
 * As w4a16_gemm, with C written as fp32 [M][N], not rounded: the partial sum
 * of one K shard when a matmul is split by rows of W across GPUs (tensor
 * parallelism, page "Qwen3.8 27B - NVFP4 for veloGB10", section "Running
 * with veloGB10": two and four nodes).  A shard holds K_i rows of W (a
 * multiple of 128: whole groups, with their scales) and the matching
 * columns of A as its own [M][K_i] matrix; the shards' fp32 outputs are
 * summed (an all-reduce) and rounded once.  Column shards need no mode of
 * their own: they are matmuls of N_i columns.
 *   C            device fp32 [M][N] (written), 16-byte aligned
 */
int w4a16_gemm_f32(const void *A, const void *wq_repacked, const void *scales, float *C, int M,
                   int N, int K, int group, void *workspace, size_t workspace_bytes, void *stream);

/* As w4a16_gemm_f32 (same passages) with an explicit plan of the row-count dispatch. */
int w4a16_gemm_f32_plan(const void *A, const void *wq_repacked, const void *scales, float *C, int M,
                        int N, int K, int group, void *workspace, size_t workspace_bytes,
                        const w4a16_plan_t *plan, void *stream);

/*
 * Output projection with the greedy pick in its epilogue: for each row m,
 *
 *     idx[m] = the column n of the largest C[m][n] = (A . dequant)[m][n]
 *              (the lowest such n among equal values; -0 equals +0),
 *     val[m] = that C[m][n] as fp32,
 *
 * the model's greedy token for each verified position.  The output
 * projection is one of the row-count dispatched kernels (page "Qwen3.8-27B
 * on single DGX Spark ...", section "How."); a drafted token is kept only if
 * the full model agrees with it (page "One Config Line Made My 27B Model
 * 2.7x Faster", section "Three caveats worth stating plainly"), which under
 * greedy decoding means it equals this argmax.  C is never stored.
 * The decision is taken on the kernel's fp32 sums.
 *   idx, val     device int32 [M] and fp32 [M] (written), 4-byte aligned
 *   workspace    device, at least W4A16_ARGMAX_WORKSPACE_BYTES, zero-filled
 *                before its first use.  The call uses only the counter region
 *                (see the split-K layout) and leaves it zero again, so one
 *                workspace serves argmax and split-K calls alike in stream
 *                order (not calls that run concurrently)
 *   other arguments as w4a16_gemm.  Plans must have splits == 1.
 * Two kernels are enqueued: the matmul, whose workgroups leave their row
 * maxima in the workspace, and a one-workgroup fold that writes idx and val.
 */
#define W4A16_ARGMAX_WORKSPACE_BYTES W4A16_SPLIT_COUNTER_BYTES   /* its counter region only */
int w4a16_gemm_argmax(const void *A, const void *wq_repacked, const void *scales, int *idx,
                      float *val, int M, int N, int K, int group, void *workspace,
                      size_t workspace_bytes, void *stream);

/* As w4a16_gemm_argmax (same passages) with an explicit plan of the row-count dispatch (splits must be 1). */
int w4a16_gemm_argmax_plan(const void *A, const void *wq_repacked, const void *scales, int *idx,
                           float *val, int M, int N, int K, int group, void *workspace,
                           size_t workspace_bytes, const w4a16_plan_t *plan, void *stream);

/*
 * Test export of the device dequantization used by both GEMM paths:
 * W[k][n] = (q - 8) * s as fp32 (exact: at most 11 significant bits),
 * device fp32 [K][N] (written); `scales` are the checkpoint's [K/128][N].
 * The dequantization whose exactness the page "Qwen3.8-27B on single DGX
 * Spark ..." (section "Quality.") gates the runtime against.
 */
int w4a16_dequant_debug(const void *wq_repacked, const void *scales, float *W, int K, int N,
                        void *stream);

/*
 * Test export of the device unpacking used by both GEMM paths:
 * codes[k][n] = q in [0, 15], device uint8 [K][N] (written): the 4-bit codes
 * of the checkpoint format (page "Qwen3.8-27B on single DGX Spark ...",
 * section "Quality.").
 */
int w4a16_unpack_debug(const void *wq_repacked, uint8_t *codes, int K, int N, void *stream);

/*
 * ---------------------------------------------------------------- NVFP4
 * The same decode/verify matmul for NVFP4 weight-only checkpoints: the
 * compressed-tensors "nvfp4-pack-quantized" format of the page "Qwen3.8 27B
 * - NVFP4 for veloGB10" (section "Specifications"), with group size 16 (page
 * "SuperQwen3.8-27b-abliterated-NVFP4-2xDGX", table "Release highlights"),
 * run with BF16 activations as the page "Qwen3.8-27B on DGX Spark (GB10):
 * vLLM 0.24 + NVFP4, the sm_121 kernel gotcha" describes (W4A16, sections
 * "What Spark-native means" and "The right stack for Spark").  The pages do
 * not define the encodings; these calls take the published ones:
 *
 *     C[m][n] = alpha * sum_k A[m][k] * e2m1(code(k, n)) * e4m3(scale(k/16, n))
 *
 *   packed   uint8 [N][K/2]: row n holds column n of W; byte j holds the
 *            FP4 E2M1 code of row k = 2j in its low nibble and of k = 2j + 1
 *            in its high nibble (bit 3 sign, bits 2..1 exponent with bias 1,
 *            bit 0 mantissa).
 *   scales   uint8 [N][K/16]: FP8 E4M3 (bias 7, OCP encoding) of rows
 *            16kb .. 16kb + 15 of column n at (n, kb).
 *   alpha    fp32 per-tensor factor applied to the fp32 sum (for a
 *            checkpoint that stores a global scale g to divide by, 1/g).
 *   blob     K*N/2 bytes: 16-byte pieces (t, g, h, c) at piece index
 *            ((t*G + g)*4 + h)*16 + c (G = K/128); byte 2b + p of a piece
 *            holds rows 128g + 16b + 4h + 2p (low nibble) and the next row
 *            (high nibble) of column n = 16t + c.
 *   repacked scales  K*N/16 bytes: the scale of block 8g + b of column
 *            n = 16t + c at byte ((t*G + g)*16 + c)*8 + b.
 * Valid shapes as for the GPTQ calls (K a multiple of 128, N of 16,
 * 1 <= M <= 16); group must be W4A16_NVFP4_GROUP.  A block scale of NaN
 * (S.1111.111) makes its outputs NaN.
 */

/* Bytes of the NVFP4 blob (= K*N/2) and of its repacked scales (= K*N/16); 0 for invalid shapes. */
size_t w4a16_nvfp4_repacked_bytes(int K, int N);
size_t w4a16_nvfp4_repacked_scale_bytes(int K, int N);

/*
 * One-time repacks into the layouts above (pure permutations of bytes) of
 * the checkpoint tensors the NVFP4 section above cites.
 *   packed / scales           device, as above (read only)
 *   wq_repacked / scales_repacked  device, the sizes above (written)
 */
int w4a16_nvfp4_repack_weights(const void *packed, void *wq_repacked, int K, int N, void *stream);
int w4a16_nvfp4_repack_scales(const void *scales, void *scales_repacked, int K, int N, void *stream);

/* Planning for the NVFP4 calls (the same row-count dispatch, page
 * "Qwen3.8-27B on single DGX Spark ...", section "How."): as w4a16_get_plan,
 * w4a16_check_plan, w4a16_workspace_bytes and w4a16_workspace_bytes_plan. */
int w4a16_nvfp4_get_plan(int M, int N, int K, w4a16_plan_t *plan);
int w4a16_nvfp4_check_plan(int M, int N, int K, const w4a16_plan_t *plan);
size_t w4a16_nvfp4_workspace_bytes(int M, int N, int K);
size_t w4a16_nvfp4_workspace_bytes_plan(int M, int N, int K, const w4a16_plan_t *plan);

/*
 * C = alpha * A . dequant(blob, scales), dispatched by row count.
 *   A            device bf16 [M][K]
 *   wq_repacked, scales   device, from the NVFP4 repacks for this K, N
 *   alpha        the per-tensor factor
 *   C            device bf16 [M][N] (written), rounded to nearest even once
 *   group        must be W4A16_NVFP4_GROUP
 *   workspace    as for w4a16_gemm, at least w4a16_nvfp4_workspace_bytes(M, N, K)
 * Every converted weight e2m1 * e4m3 is exact; each 16-row block's partial
 * sum is scaled and accumulated in fp32.  Deterministic.
 */
int w4a16_nvfp4_gemm(const void *A, const void *wq_repacked, const void *scales, float alpha, void *C,
                     int M, int N, int K, int group, void *workspace, size_t workspace_bytes,
                     void *stream);

/* As w4a16_nvfp4_gemm (same passages) with an explicit plan of the row-count dispatch. */
int w4a16_nvfp4_gemm_plan(const void *A, const void *wq_repacked, const void *scales, float alpha,
                          void *C, int M, int N, int K, int group, void *workspace,
                          size_t workspace_bytes, const w4a16_plan_t *plan, void *stream);

/*
 * The epilogue modes of the GPTQ calls for NVFP4 weights: the same contracts
 * as w4a16_gemm_silu_mul, w4a16_gemm_argmax and w4a16_gemm_f32 (and their
 * _plan forms), with C = alpha * A . dequant(blob, scales).  alpha multiplies
 * each fp32 sum before the epilogue: before SiLU(gate) * up, before the
 * argmax comparison (a negative alpha picks the smallest sum), and in the
 * fp32 output.  group must be W4A16_NVFP4_GROUP.  A checkpoint quantized to
 * NVFP4 for all its GEMMs (page "Qwen3.8 27B - NVFP4 for veloGB10", section
 * "Specifications": recipe "all") runs its gate/up, output projection and
 * tensor-parallel shards through these.
 */
int w4a16_nvfp4_gemm_silu_mul(const void *A, const void *wq_repacked, const void *scales, float alpha,
                              void *H, int M, int N, int K, int group, void *workspace,
                              size_t workspace_bytes, void *stream);
int w4a16_nvfp4_gemm_silu_mul_plan(const void *A, const void *wq_repacked, const void *scales,
                                   float alpha, void *H, int M, int N, int K, int group,
                                   void *workspace, size_t workspace_bytes, const w4a16_plan_t *plan,
                                   void *stream);
int w4a16_nvfp4_gemm_argmax(const void *A, const void *wq_repacked, const void *scales, float alpha,
                            int *idx, float *val, int M, int N, int K, int group, void *workspace,
                            size_t workspace_bytes, void *stream);
int w4a16_nvfp4_gemm_argmax_plan(const void *A, const void *wq_repacked, const void *scales,
                                 float alpha, int *idx, float *val, int M, int N, int K, int group,
                                 void *workspace, size_t workspace_bytes, const w4a16_plan_t *plan,
                                 void *stream);
int w4a16_nvfp4_gemm_f32(const void *A, const void *wq_repacked, const void *scales, float alpha,
                         float *C, int M, int N, int K, int group, void *workspace,
                         size_t workspace_bytes, void *stream);
int w4a16_nvfp4_gemm_f32_plan(const void *A, const void *wq_repacked, const void *scales, float alpha,
                              float *C, int M, int N, int K, int group, void *workspace,
                              size_t workspace_bytes, const w4a16_plan_t *plan, void *stream);

/*
 * Test export of the NVFP4 device dequantization: W[k][n] = e2m1 * e4m3 as
 * fp32 (exact; without alpha), device fp32 [K][N] (written), for the
 * format the NVFP4 section above cites (compressed-tensors
 * "nvfp4-pack-quantized", page "Qwen3.8 27B - NVFP4 for veloGB10", section
 * "Specifications").
 */
int w4a16_nvfp4_dequant(const void *wq_repacked, const void *scales, float *W, int K, int N,
                        void *stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
