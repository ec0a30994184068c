/*
 * Memory- and UB-safety driver for the fp64 oracle (test infrastructure):
 * built with AddressSanitizer and UndefinedBehaviorSanitizer together with
 * oracle/nsa_oracle.c and run on small inputs that reach every entry point:
 * padding, future, out-of-range and repeated index entries, empty rows,
 * M != N, a ragged last block, gs > 1, both element types, windows, the
 * backward with and without key-block filters and magnitudes, top-k and the
 * streaming comparison.  It checks only that results are finite where they
 * must be; the values themselves are pinned by the Python tests.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int nsa_oracle_units_t(const uint16_t *Q, const uint16_t *K, const uint16_t *V, const int32_t *idx, int64_t B,
                       int64_t M, int64_t N, int64_t H, int64_t G, int64_t D, int64_t bs, int64_t T,
                       const int64_t *units, int64_t n_units, double *O, double *LSE, int64_t *n_dup, int elem,
                       int n_threads);
int nsa_oracle_dense_units(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int64_t B, int64_t M,
                           int64_t N, int64_t H, int64_t G, int64_t D, const int64_t *units, int64_t n_units,
                           double *O, double *LSE, int n_threads);
int nsa_oracle_window_units(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int64_t B, int64_t M,
                            int64_t N, int64_t H, int64_t G, int64_t D, int64_t left, int64_t right,
                            const int64_t *units, int64_t n_units, double *O, double *LSE, int elem, int n_threads);
int nsa_oracle_bwd_units(const uint16_t *Q, const uint16_t *K, const uint16_t *V, const int32_t *idx,
                         const uint16_t *dO, int64_t B, int64_t M, int64_t N, int64_t H, int64_t G, int64_t D,
                         int64_t bs, int64_t T, const int64_t *units, int64_t n_units, const int64_t *kblocks,
                         int64_t n_kblocks, double *dQ, double *dK, double *dV, double *mQ, double *mK, double *mV,
                         int n_threads);
int nsa_oracle_topk(const float *scores, int64_t B, int64_t M, int64_t G, int64_t NB, int64_t bs, int64_t T,
                    int32_t *out);
int nsa_oracle_topk_rows(const float *scores, const int64_t *ms, int64_t R, int64_t NB, int64_t bs, int64_t T,
                         int32_t *out);
int nsa_oracle_compare(const uint16_t *Q, const uint16_t *K, const uint16_t *V, const int32_t *idx, int64_t B,
                       int64_t M, int64_t N, int64_t H, int64_t G, int64_t D, int64_t bs, int64_t T, int64_t left,
                       int64_t right, const uint16_t *Og, const float *Lg, int64_t u0, int64_t u1, int elem,
                       int n_threads, double *stats);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) { /* splitmix64 */
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
/* A value of magnitude 2^-4 .. 2 with a random sign, as a 16-bit pattern. */
static uint16_t rand_half(int bf16) {
    const uint64_t r = next_u64();
    if (bf16) return (uint16_t)(((r & 1) << 15) | ((123 + (r >> 1) % 5) << 7) | ((r >> 8) & 0x7f));
    return (uint16_t)(((r & 1) << 15) | ((11 + (r >> 1) % 5) << 10) | ((r >> 8) & 0x3ff));
}

static int failures = 0;
static void expect(int ok, const char *what) {
    if (!ok) {
        fprintf(stderr, "FAILED: %s\n", what);
        failures++;
    }
}

static void run_case(int64_t B, int64_t M, int64_t N, int64_t H, int64_t G, int64_t D, int64_t bs, int64_t T,
                     int elem, int threads) {
    const int64_t gs = H / G, NB = (N + bs - 1) / bs, U = B * M * G;
    uint16_t *Q = malloc(sizeof(uint16_t) * B * M * H * D), *K = malloc(sizeof(uint16_t) * B * N * G * D);
    uint16_t *V = malloc(sizeof(uint16_t) * B * N * G * D), *dO = malloc(sizeof(uint16_t) * B * M * H * D);
    int32_t *idx = malloc(sizeof(int32_t) * B * M * G * T);
    int64_t *units = malloc(sizeof(int64_t) * 3 * U);
    double *O = malloc(sizeof(double) * U * gs * D), *L = malloc(sizeof(double) * U * gs);
    for (int64_t i = 0; i < B * M * H * D; ++i) Q[i] = rand_half(elem), dO[i] = rand_half(0);
    for (int64_t i = 0; i < B * N * G * D; ++i) K[i] = rand_half(elem), V[i] = rand_half(elem);
    for (int64_t i = 0; i < B * M * G * T; ++i) {
        const uint64_t r = next_u64() % 8;
        /* counted, padding, future / past-the-end, repeats of entry 0 */
        idx[i] = r < 4 ? (int32_t)(next_u64() % NB) : r == 4 ? -1 : r == 5 ? (int32_t)(NB + 3)
               : r == 6 ? -7 : idx[i - i % T];
    }
    for (int64_t b = 0, u = 0; b < B; ++b)
        for (int64_t m = 0; m < M; ++m)
            for (int64_t g = 0; g < G; ++g, ++u) units[3 * u] = b, units[3 * u + 1] = m, units[3 * u + 2] = g;
    int64_t ndup = 0;
    expect(nsa_oracle_units_t(Q, K, V, idx, B, M, N, H, G, D, bs, T, units, U, O, L, &ndup, elem, threads) == 0,
           "units");
    for (int64_t i = 0; i < U * gs * D; ++i) expect(isfinite(O[i]), "O finite");
    expect(nsa_oracle_dense_units(Q, K, V, B, M, N, H, G, D, units, U, O, L, threads) == 0 || elem, "dense");
    expect(nsa_oracle_window_units(Q, K, V, B, M, N, H, G, D, 5, 2, units, U, O, L, elem, threads) == 0, "window");
    expect(nsa_oracle_window_units(Q, K, V, B, M, N, H, G, D, -1, -1, units, U, O, L, elem, threads) == 0,
           "window unbounded");
    /* streaming comparison of the oracle's own result, rounded to 16 bits */
    uint16_t *Og = malloc(sizeof(uint16_t) * B * M * H * D);
    float *Lg = malloc(sizeof(float) * B * H * M);
    for (int64_t i = 0; i < B * M * H * D; ++i) Og[i] = rand_half(elem);
    for (int64_t i = 0; i < B * H * M; ++i) Lg[i] = (i % 7 == 0) ? -INFINITY : (float)(i % 13);
    double stats[8];
    expect(nsa_oracle_compare(Q, K, V, idx, B, M, N, H, G, D, bs, T, -1, 0, Og, Lg, 0, U, elem, threads, stats) == 0,
           "compare");
    expect(nsa_oracle_compare(Q, K, V, NULL, B, M, N, H, G, D, bs, T, 3, 0, Og, Lg, U / 3, U, elem, threads,
                              stats) == 0,
           "compare window");
    expect(nsa_oracle_compare(Q, K, V, idx, B, M, N, H, G, D, bs, T, -1, 0, Og, Lg, 0, U + 1, elem, threads, stats)
               == -1,
           "compare range check");
    if (!elem) {
        double *dQ = malloc(sizeof(double) * U * gs * D), *mQ = malloc(sizeof(double) * U * gs * D);
        double *dK = calloc((size_t)(B * N * G * D), sizeof(double)), *dV = calloc((size_t)(B * N * G * D), sizeof(double));
        double *mK = calloc((size_t)(B * N * G * D), sizeof(double)), *mV = calloc((size_t)(B * N * G * D), sizeof(double));
        expect(nsa_oracle_bwd_units(Q, K, V, idx, dO, B, M, N, H, G, D, bs, T, units, U, NULL, 0, dQ, dK, dV, mQ, mK,
                                    mV, threads) == 0,
               "bwd");
        int64_t kb[6] = {0, 0, 0, B - 1, G - 1, NB - 1};
        double *fK = calloc((size_t)(2 * bs * D), sizeof(double)), *fV = calloc((size_t)(2 * bs * D), sizeof(double));
        expect(nsa_oracle_bwd_units(Q, K, V, idx, dO, B, M, N, H, G, D, bs, T, units, U, kb, 2, dQ, fK, fV, NULL, NULL,
                                    NULL, threads) == 0,
               "bwd kblocks");
        expect(nsa_oracle_bwd_units(Q, K, V, NULL, dO, B, M, N, H, G, D, bs, 1, units, U, NULL, 0, dQ, dK, dV, NULL,
                                    NULL, NULL, threads) == 0,
               "bwd dense");
        for (int64_t i = 0; i < U * gs * D; ++i) expect(isfinite(dQ[i]), "dQ finite");
        free(dQ); free(mQ); free(dK); free(dV); free(mK); free(mV); free(fK); free(fV);
    }
    free(Og); free(Lg);
    free(Q); free(K); free(V); free(dO); free(idx); free(units); free(O); free(L);
}

int main(void) {
    run_case(1, 70, 70, 4, 2, 64, 32, 5, 0, 3);     /* gs 2, ragged last block */
    run_case(2, 40, 67, 6, 2, 64, 16, 7, 0, 2);     /* M < N, B = 2, gs 3 */
    run_case(1, 90, 33, 8, 1, 128, 8, 9, 1, 4);     /* M > N, bf16, T > NB */
    run_case(1, 17, 17, 1, 1, 64, 64, 2, 0, 1);     /* one block, one thread */
    /* top-k: causal candidates, NaN scores, fewer candidates than T */
    {
        const int64_t B = 1, M = 100, G = 2, NB = 9, bs = 16, T = 4;
        float *s = malloc(sizeof(float) * B * M * G * NB);
        int32_t *out = malloc(sizeof(int32_t) * B * M * G * T);
        for (int64_t i = 0; i < B * M * G * NB; ++i) s[i] = (i % 11 == 0) ? NAN : (float)(next_u64() % 7);
        expect(nsa_oracle_topk(s, B, M, G, NB, bs, T, out) == 0, "topk");
        int64_t ms[3] = {0, 50, 99};
        expect(nsa_oracle_topk_rows(s, ms, 3, NB, bs, T, out) == 0, "topk rows");
        free(s); free(out);
    }
    if (failures) return 1;
    printf("oracle sanitizer driver: ok\n");
    return 0;
}
