/*
 * Plain CPU oracle for the NVFP4 weight-only (W4A16) variant of the matmul.
 *
 * TEST INFRASTRUCTURE ONLY, like oracle.c, and built into the same library.
 * It shares no code, header, table or constant with the HIP library.
 *
 * What is computed, and where it comes from:
 *   The pages name an NVFP4 27B checkpoint in the compressed-tensors
 *   "nvfp4-pack-quantized" layout (page "Qwen3.8 27B - NVFP4 for veloGB10",
 *   section "Specifications"), with group size 16 (page
 *   "SuperQwen3.8-27b-abliterated-NVFP4-2xDGX", table "Release
 *   highlights"), and call its weight-only use, BF16 activations, W4A16
 *   (page "Qwen3.8-27B on DGX Spark (GB10): vLLM 0.24 + NVFP4, the sm_121
 *   kernel gotcha", sections "What Spark-native means" and "The right stack
 *   for Spark").  They define neither the element nor the scale encoding;
 *   the readings taken are the published formats
 *   NVFP4 is built from:
 *     - element: FP4 E2M1 (OCP Microscaling Formats v1.0): bit 3 sign,
 *       bits 2..1 exponent with bias 1, bit 0 mantissa; exponent 0 is
 *       subnormal, value m * 2^-1; no infinities or NaN;
 *     - block scale: FP8 E4M3 (OCP 8-bit Floating Point, E4M3): bit 7 sign,
 *       bits 6..3 exponent with bias 7, bits 2..0 mantissa; exponent 0 is
 *       subnormal, value m/8 * 2^-6; S.1111.111 is NaN; no infinities;
 *       one scale per 16 consecutive k of one output column;
 *     - one fp32 per-tensor factor alpha multiplies the whole sum;
 *     - layout: packed codes uint8 [N][K/2] (row n = output column n of W,
 *       byte j holds k = 2j in its low nibble and k = 2j + 1 in its high
 *       nibble); scales uint8 [N][K/16].
 *
 *   C[m][n] = alpha * sum_k A[m][k] * e2m1(code(k, n)) * e4m3(scale(k/16, n))
 *
 * Accumulation is fp64 with k ascending.  Every product is exact in fp64
 * (a: 8 significant bits, e2m1: 2, e4m3: 4, alpha: 24), so the only
 * rounding is the running fp64 sum.
 *
 * The repack functions build the gfx950 tile-order blob and scales from
 * their written layout definitions, independently of the HIP repack kernels.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define SUPER 128   /* rows per repacked (tile, superblock) piece set */
#define BLOCK 16    /* rows per scale block */

double oracle_e2m1_to_f64(unsigned code) {
    unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
    double v = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
    return s ? -v : v;
}

double oracle_e4m3_to_f64(unsigned byte) {
    unsigned s = (byte >> 7) & 1u, e = (byte >> 3) & 15u, m = byte & 7u;
    double v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return s ? -v : v;
}

static double bf16_value(uint16_t bits) {
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Code of (k, n): nibble k % 2 of byte (n, k / 2), low nibble first. */
static unsigned nv_code(const uint8_t *packed, int K, int k, int n) {
    uint8_t b = packed[(size_t)n * (size_t)(K / 2) + (size_t)(k / 2)];
    return (k % 2 == 0) ? (unsigned)(b & 0xFu) : (unsigned)(b >> 4);
}

static double nv_scale(const uint8_t *scales, int K, int k, int n) {
    return oracle_e4m3_to_f64(scales[(size_t)n * (size_t)(K / BLOCK) + (size_t)(k / BLOCK)]);
}

/* codes[k*N + n] = code(k, n) in [0, 15]. */
void oracle_nvfp4_unpack(const uint8_t *packed, int K, int N, uint8_t *codes) {
    for (int k = 0; k < K; ++k)
        for (int n = 0; n < N; ++n) codes[(size_t)k * N + n] = (uint8_t)nv_code(packed, K, k, n);
}

/* W[k*N + n] = e2m1(code(k, n)) * e4m3(scale(k/16, n)), without alpha (exact). */
void oracle_nvfp4_dequant(const uint8_t *packed, const uint8_t *scales, int K, int N, double *W) {
    for (int k = 0; k < K; ++k)
        for (int n = 0; n < N; ++n)
            W[(size_t)k * N + n] = oracle_e2m1_to_f64(nv_code(packed, K, k, n)) * nv_scale(scales, K, k, n);
}

/*
 * C[m][j] = alpha * sum_k A[m][k] * W[k][cols[j]] and
 * D[m][j] = |alpha| * sum_k |A[m][k] * W[k][cols[j]]|, j in [0, ncols)
 * (cols NULL: all N columns).  A is bf16 [M][K]; C and D fp64 [M][ncols].
 * Parallel over columns only; each column's sum runs k ascending.
 */
void oracle_nvfp4_gemm(const uint16_t *A, const uint8_t *packed, const uint8_t *scales, double alpha,
                       int M, int N, int K, const int *cols, int ncols, int nthreads, double *C,
                       double *D) {
    double *Ad = (double *)malloc(sizeof(double) * (size_t)M * (size_t)K);
    for (size_t i = 0; i < (size_t)M * (size_t)K; ++i) Ad[i] = bf16_value(A[i]);
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
    for (int j = 0; j < ncols; ++j) {
        int n = cols ? cols[j] : j;
        double c[16], d[16];
        for (int m = 0; m < M; ++m) { c[m] = 0.0; d[m] = 0.0; }
        for (int k = 0; k < K; ++k) {
            double w = alpha * oracle_e2m1_to_f64(nv_code(packed, K, k, n)) * nv_scale(scales, K, k, n);
            for (int m = 0; m < M; ++m) {
                double p = Ad[(size_t)m * K + k] * w;
                c[m] += p;
                d[m] += fabs(p);
            }
        }
        for (int m = 0; m < M; ++m) {
            C[(size_t)m * ncols + j] = c[m];
            D[(size_t)m * ncols + j] = d[m];
        }
    }
    free(Ad);
}

/*
 * Repacked codes, written from the layout definition.
 *
 * An array of 16-byte pieces.  Piece (t, g, h, c) sits at piece index
 * ((t * G + g) * 4 + h) * 16 + c, G = K / 128, and describes column
 * n = 16 t + c.  Byte i = 2 b + p of the piece (b = 0..7, p = 0..1) holds
 * row k = 128 g + 16 b + 4 h + 2 p in its low nibble and row k + 1 in its
 * high nibble: lane group h of a wavefront owns rows 4h..4h+3 of every
 * 16-row scale block b of superblock g.  K * N / 2 bytes in all.
 */
static size_t nv_blob_byte(int K, int k, int n) {
    int G = K / SUPER;
    int t = n / 16, c = n % 16;
    int g = k / SUPER, r = k % SUPER;
    int b = r / BLOCK, h = (r % BLOCK) / 4, p = (r % 4) / 2;
    size_t piece = (((size_t)t * G + g) * 4 + h) * 16 + c;
    return piece * 16 + (size_t)(2 * b + p);
}

/* blob <- repack(packed); both K*N/2 bytes.  Requires K % 128 == 0, N % 16 == 0. */
void oracle_nvfp4_repack(const uint8_t *packed, int K, int N, uint8_t *blob) {
    memset(blob, 0, (size_t)K * (size_t)N / 2);
    for (int k = 0; k < K; ++k)
        for (int n = 0; n < N; ++n) {
            unsigned q = nv_code(packed, K, k, n);
            blob[nv_blob_byte(K, k, n)] |= (uint8_t)(q << (4u * (unsigned)(k % 2)));
        }
}

/* packed <- inverse of repack(blob). */
void oracle_nvfp4_unrepack(const uint8_t *blob, int K, int N, uint8_t *packed) {
    memset(packed, 0, (size_t)K * (size_t)N / 2);
    for (int k = 0; k < K; ++k)
        for (int n = 0; n < N; ++n) {
            unsigned q = (blob[nv_blob_byte(K, k, n)] >> (4u * (unsigned)(k % 2))) & 0xFu;
            packed[(size_t)n * (size_t)(K / 2) + (size_t)(k / 2)] |= (uint8_t)(q << (4u * (unsigned)(k % 2)));
        }
}

/*
 * Repacked scales, written from the layout definition: the scale of block
 * kb = 8 g + b (rows 16 kb .. 16 kb + 15) of column n = 16 t + c moves to
 * byte ((t * G + g) * 16 + c) * 8 + b, so one column's eight block scales of
 * a superblock are one 8-byte run.  K * N / 16 bytes in all.
 */
void oracle_nvfp4_repack_scales(const uint8_t *scales, int K, int N, uint8_t *out) {
    int G = K / SUPER;
    for (int n = 0; n < N; ++n)
        for (int kb = 0; kb < K / BLOCK; ++kb) {
            int t = n / 16, c = n % 16, g = kb / 8, b = kb % 8;
            size_t idx = (((size_t)t * G + g) * 16 + c) * 8 + (size_t)b;
            out[idx] = scales[(size_t)n * (size_t)(K / BLOCK) + (size_t)kb];
        }
}
