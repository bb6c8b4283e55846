/*
 * Driver for an AddressSanitizer / UndefinedBehaviorSanitizer build of the
 * CPU oracle (oracle/oracle.c, oracle/nvfp4.c; test infrastructure).  It runs
 * every exported oracle function on small shapes, including odd row counts,
 * column subsets and the largest code and scale values, and checks a few
 * invariants (repack round trips, the all-codes-8 zero product) so that the
 * sanitizers see every loop and index path.  Exit status 0 means no failure;
 * the sanitizers abort on their own findings.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void oracle_unpack(const uint32_t *qweight, int K, int N, uint8_t *codes);
void oracle_dequant(const uint32_t *qweight, const uint16_t *scales, int K, int N, double *W);
void oracle_gemm(const uint16_t *A, const uint32_t *qweight, const uint16_t *scales, int M, int N, int K,
                 const int *cols, int ncols, int nthreads, double *C, double *D);
void oracle_repack(const uint32_t *qweight, int K, int N, uint32_t *blob);
void oracle_unrepack(const uint32_t *blob, int K, int N, uint32_t *qweight);
double oracle_e2m1_to_f64(unsigned code);
double oracle_e4m3_to_f64(unsigned byte);
void oracle_nvfp4_unpack(const uint8_t *packed, int K, int N, uint8_t *codes);
void oracle_nvfp4_dequant(const uint8_t *packed, const uint8_t *scales, int K, int N, double *W);
void oracle_nvfp4_gemm(const uint16_t *A, const uint8_t *packed, const uint8_t *scales, double alpha, int M,
                       int N, int K, const int *cols, int ncols, int nthreads, double *C, double *D);
void oracle_nvfp4_repack(const uint8_t *packed, int K, int N, uint8_t *blob);
void oracle_nvfp4_unrepack(const uint8_t *blob, int K, int N, uint8_t *packed);
void oracle_nvfp4_repack_scales(const uint8_t *scales, int K, int N, uint8_t *out);

static uint32_t rng = 12345u;
static uint32_t next(void) { rng = rng * 1664525u + 1013904223u; return rng; }

#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); return 1; } } while (0)

static int gptq(int M, int K, int N) {
    const size_t nw = (size_t)K / 8 * N, ns = (size_t)K / 128 * N;
    uint32_t *q = malloc(nw * 4), *blob = malloc(nw * 4), *back = malloc(nw * 4);
    uint16_t *s = malloc(ns * 2), *A = malloc((size_t)M * K * 2);
    uint8_t *codes = malloc((size_t)K * N);
    double *W = malloc(sizeof(double) * K * N), *C = malloc(sizeof(double) * M * N), *D = malloc(sizeof(double) * M * N);
    for (size_t i = 0; i < nw; ++i) q[i] = next();
    q[0] = 0xFFFFFFFFu;
    for (size_t i = 0; i < ns; ++i) s[i] = (uint16_t)(0x3C00 + (next() & 0x3FF));
    s[0] = 0x0001;                                   /* subnormal */
    for (size_t i = 0; i < (size_t)M * K; ++i) A[i] = (uint16_t)(0x3F80 ^ (next() & 0x80FF));
    oracle_unpack(q, K, N, codes);
    oracle_dequant(q, s, K, N, W);
    oracle_gemm(A, q, s, M, N, K, NULL, N, 2, C, D);
    int cols[3] = {N - 1, 0, N / 2};
    oracle_gemm(A, q, s, M, N, K, cols, 3, 1, C, D);
    oracle_repack(q, K, N, blob);
    oracle_unrepack(blob, K, N, back);
    CHECK(memcmp(q, back, nw * 4) == 0);
    for (size_t i = 0; i < nw; ++i) q[i] = 0x88888888u;  /* every code 8: exact zeros */
    oracle_gemm(A, q, s, M, N, K, NULL, N, 0, C, D);
    for (int i = 0; i < M * N; ++i) CHECK(C[i] == 0.0 && D[i] == 0.0);
    free(q); free(blob); free(back); free(s); free(A); free(codes); free(W); free(C); free(D);
    return 0;
}

static int nvfp4(int M, int K, int N) {
    const size_t np = (size_t)N * K / 2, ns = (size_t)N * K / 16;
    uint8_t *p = malloc(np), *blob = malloc(np), *back = malloc(np), *s = malloc(ns), *sr = malloc(ns);
    uint8_t *codes = malloc((size_t)K * N);
    uint16_t *A = malloc((size_t)M * K * 2);
    double *W = malloc(sizeof(double) * K * N), *C = malloc(sizeof(double) * M * N), *D = malloc(sizeof(double) * M * N);
    for (size_t i = 0; i < np; ++i) p[i] = (uint8_t)next();
    for (size_t i = 0; i < ns; ++i) s[i] = (uint8_t)(next() % 0x7F);   /* finite, subnormal included */
    for (size_t i = 0; i < (size_t)M * K; ++i) A[i] = (uint16_t)(0x3F80 ^ (next() & 0x80FF));
    for (unsigned c = 0; c < 16; ++c) (void)oracle_e2m1_to_f64(c);
    for (unsigned b = 0; b < 256; ++b) (void)oracle_e4m3_to_f64(b);
    oracle_nvfp4_unpack(p, K, N, codes);
    oracle_nvfp4_dequant(p, s, K, N, W);
    oracle_nvfp4_gemm(A, p, s, -0.5, M, N, K, NULL, N, 2, C, D);
    int cols[2] = {N - 1, 3};
    oracle_nvfp4_gemm(A, p, s, 1.0, M, N, K, cols, 2, 1, C, D);
    oracle_nvfp4_repack(p, K, N, blob);
    oracle_nvfp4_unrepack(blob, K, N, back);
    CHECK(memcmp(p, back, np) == 0);
    oracle_nvfp4_repack_scales(s, K, N, sr);
    free(p); free(blob); free(back); free(s); free(sr); free(codes); free(A); free(W); free(C); free(D);
    return 0;
}

int main(void) {
    const int shapes[][3] = {{1, 128, 16}, {3, 256, 48}, {16, 384, 32}, {5, 1024, 80}};
    for (size_t i = 0; i < sizeof(shapes) / sizeof(shapes[0]); ++i) {
        if (gptq(shapes[i][0], shapes[i][1], shapes[i][2])) return 1;
        if (nvfp4(shapes[i][0], shapes[i][1], shapes[i][2])) return 1;
    }
    printf("oracle sanitizer check: ok\n");
    return 0;
}
