/*
 * Plain CPU oracle for the W4A16 decode/verify matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library.  The product path
 * (the HIP library under weight_only_int4_gptq_amd/) never calls it, and this
 * file shares no code, header, table or constant with that library.
 *
 * What is computed, and where it comes from:
 *   The checkpoint contract (page "Qwen3.8-27B on single DGX Spark ...",
 *   section "Quality."): symmetric GPTQ, 4-bit, group size 128 along K,
 *   BF16 activations, no act-order, no zero points.  The runtime there is
 *   judged against exact dequantization of its checkpoint, so the oracle is
 *   exactly that: dequantize exactly, then multiply in fp64.
 *
 *   Readings taken where the pages are silent:
 *     - qweight is uint32 [K/8][N], N contiguous; nibble j of word (kb, n)
 *       (bits 4j..4j+3, low nibble first) holds the code of k = 8*kb + j.
 *     - "symmetric, no zero points" on a 4-bit code q in [0,15] means the
 *       implicit midpoint 8:  w = (q - 8) * s.
 *     - scales are bf16 [K/128][N]; the group of row k is floor(k/128)
 *       ("no act-order" means there is no permutation of k).
 *     - every bf16 value is read exactly (bits << 16 as an IEEE float).
 *
 * Accumulation is fp64 with k ascending.  Products a*w are exact in fp64
 * (a has 8 significant bits, w at most 11), so the only rounding is the
 * running fp64 sum; its error is below K * 2^-53 * sum|a*w|.
 *
 * The repack functions build the gfx950 tile-order blob from the written
 * layout definition (see oracle_repack below), independently of the HIP
 * repack kernel.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define GROUP 128

/* bf16 bit pattern -> exact double: a bf16 is the top half of an IEEE fp32. */
static double bf16_to_f64(uint16_t bits) {
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

double oracle_bf16_to_f64(uint16_t bits) { return bf16_to_f64(bits); }

/* Code of (k, n) read from the GPTQ words: nibble k%8 of word (k/8, n),
 * low nibble first.  Unsigned shift: a word such as 0xFEDCBA98 is negative
 * when viewed as int32. */
static unsigned code_at(const uint32_t *qweight, int N, int k, int n) {
    uint32_t word = qweight[(size_t)(k / 8) * (size_t)N + (size_t)n];
    return (unsigned)((word >> (4u * (unsigned)(k % 8))) & 0xFu);
}

/* codes[k*N + n] = q(k, n) in [0, 15]. */
void oracle_unpack(const uint32_t *qweight, int K, int N, uint8_t *codes) {
    for (int k = 0; k < K; ++k)
        for (int n = 0; n < N; ++n)
            codes[(size_t)k * N + n] = (uint8_t)code_at(qweight, N, k, n);
}

/* W[k*N + n] = (q(k,n) - 8) * s[floor(k/128)][n], exact in fp64 (and also
 * exactly representable in fp32 whenever |q - 8| * s stays in fp32 range). */
void oracle_dequant(const uint32_t *qweight, const uint16_t *scales, int K, int N,
                    double *W) {
    for (int k = 0; k < K; ++k) {
        int g = k / GROUP;
        for (int n = 0; n < N; ++n) {
            double s = bf16_to_f64(scales[(size_t)g * N + n]);
            double q = (double)code_at(qweight, N, k, n);
            W[(size_t)k * N + n] = (q - 8.0) * s;
        }
    }
}

/*
 * C[m][j] = sum_k A[m][k] * W[k][cols[j]]   and   D[m][j] = sum_k |A[m][k] * W[k][cols[j]]|
 * for j in [0, ncols).  If cols is NULL the columns are 0..N-1 (ncols must be N).
 * A is bf16 [M][K] row-major.  C and D are fp64 [M][ncols].
 * nthreads <= 0 means "use the OpenMP default".  Parallel over columns only;
 * each column's sum runs k ascending in one thread, so results do not depend
 * on the thread count.
 */
void oracle_gemm(const uint16_t *A, const uint32_t *qweight, const uint16_t *scales,
                 int M, int N, int K, const int *cols, int ncols, int nthreads,
                 double *C, double *D) {
    double *Ad = (double *)malloc(sizeof(double) * (size_t)M * (size_t)K);
    for (size_t i = 0; i < (size_t)M * (size_t)K; ++i) Ad[i] = bf16_to_f64(A[i]);
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
    for (int j = 0; j < ncols; ++j) {
        int n = cols ? cols[j] : j;
        double c[16], d[16];
        for (int m = 0; m < M; ++m) { c[m] = 0.0; d[m] = 0.0; }
        for (int k = 0; k < K; ++k) {
            double s = bf16_to_f64(scales[(size_t)(k / GROUP) * N + n]);
            double w = ((double)code_at(qweight, N, k, n) - 8.0) * s;
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

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Repacked blob, written from its layout definition.
 *
 * The blob is an array of 16-byte pieces (4 little-endian uint32 words).
 * Piece (t, g, h, c) sits at piece index ((t * G + g) * 4 + h) * 16 + c, where
 *   t = column tile (16 columns), g = K group (128 rows), G = K / 128,
 *   h = quarter of the group (32 rows), c = column inside the tile.
 * It describes column n = 16 t + c and rows k = 128 g + 32 h + 8 r + e for
 * word r = 0..3 of the piece and e = 0..7 inside the word.
 * Inside a word, the code of row offset e sits at bit
 *   4 * (e / 2)        when e is even   (bits 0..15 hold e = 0, 2, 4, 6)
 *   16 + 4 * (e / 2)   when e is odd    (bits 16..31 hold e = 1, 3, 5, 7).
 * Nothing else is stored; the blob has exactly K * N / 2 bytes.
 */
static size_t blob_word_index(int K, int k, int n) {
    int G = K / GROUP;
    int t = n / 16, c = n % 16;
    int g = k / GROUP, h = (k % GROUP) / 32, r = (k % 32) / 8;
    size_t piece = (((size_t)t * G + g) * 4 + h) * 16 + c;
    return piece * 4 + (size_t)r;
}

static unsigned blob_bit(int k) {
    int e = k % 8;
    return (e % 2 == 0) ? 4u * (unsigned)(e / 2) : 16u + 4u * (unsigned)(e / 2);
}

/* blob <- repack(qweight); blob has K*N/8 words. */
void oracle_repack(const uint32_t *qweight, int K, int N, uint32_t *blob) {
    memset(blob, 0, sizeof(uint32_t) * (size_t)K * (size_t)N / 8);
    for (int k = 0; k < K; ++k)
        for (int n = 0; n < N; ++n) {
            unsigned q = code_at(qweight, N, k, n);
            blob[blob_word_index(K, k, n)] |= (uint32_t)q << blob_bit(k);
        }
}

/* qweight <- inverse of repack(blob). */
void oracle_unrepack(const uint32_t *blob, int K, int N, uint32_t *qweight) {
    memset(qweight, 0, sizeof(uint32_t) * (size_t)K * (size_t)N / 8);
    for (int k = 0; k < K; ++k)
        for (int n = 0; n < N; ++n) {
            unsigned q = (blob[blob_word_index(K, k, n)] >> blob_bit(k)) & 0xFu;
            qweight[(size_t)(k / 8) * N + n] |= (uint32_t)q << (4u * (unsigned)(k % 8));
        }
}

