/* The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host build, gcc):
 * every entry point on small seeded inputs in buffers of exactly the documented size,
 * including the edge cases (one point, fewer distinct points than centroids, empty
 * history or window, K of 1 and 256).  Any out-of-bounds access, leak or undefined
 * operation aborts the program; a few results are checked against their definition. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/oracle.c"

static uint64_t rng = 88172645463325252ull;
static double urand(void) {
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (double)(rng >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}
static float *frand(size_t n) {
    float *p = (float *)malloc(sizeof(float) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) p[i] = (float)urand();
    return p;
}
static int fails = 0;
#define CHECK(c)                                             \
    do {                                                     \
        if (!(c)) {                                          \
            fprintf(stderr, "FAIL line %d: %s\n", __LINE__, #c); \
            ++fails;                                         \
        }                                                    \
    } while (0)

static void encode_case(int64_t N, int H, int d, int dsub, int K) {
    const int M = d / dsub;
    float *x = frand((size_t)N * H * d), *cb = frand((size_t)H * K * M * dsub);
    uint8_t *codes = (uint8_t *)malloc((size_t)N * H * M + 1);
    double *d1 = (double *)malloc(sizeof(double) * (N * H * M + 1)), *d2 = (double *)malloc(sizeof(double) * (N * H * M + 1));
    double *dist = (double *)malloc(sizeof(double) * (N * H * M + 1)), *deq = (double *)malloc(sizeof(double) * (N * H * d + 1));
    CHECK(orc_encode(x, N, H, d, dsub, K, cb, codes, d1, d2) == 0);
    CHECK(orc_code_distance(x, N, H, d, dsub, K, cb, codes, dist) == 0);
    CHECK(orc_dequantize(codes, N, H, d, dsub, K, cb, deq) == 0);
    for (int64_t i = 0; i < N * H * M; ++i) {
        CHECK(codes[i] < K);
        CHECK(dist[i] == d1[i]);
        CHECK(d2[i] >= d1[i]);
    }
    free(x); free(cb); free(codes); free(d1); free(d2); free(dist); free(deq);
}

static void fit_case(int64_t N, int H, int d, int dsub, int K, int iters, int distinct) {
    const int M = d / dsub;
    float *x = frand((size_t)N * H * d);
    if (distinct > 0) /* only `distinct` different tokens */
        for (int64_t t = distinct; t < N; ++t) memcpy(x + t * H * d, x + (t % distinct) * H * d, sizeof(float) * H * d);
    int64_t *order = (int64_t *)malloc(sizeof(int64_t) * H * M * N);
    for (int64_t u = 0; u < (int64_t)H * M; ++u)
        for (int64_t i = 0; i < N; ++i) order[u * N + i] = (i * 7 + u) % N;  /* a permutation when gcd(7, N) = 1 */
    double *cb = (double *)malloc(sizeof(double) * H * K * M * dsub);
    int64_t *kept = (int64_t *)malloc(sizeof(int64_t) * H * M);
    CHECK(orc_fit_codebooks(x, N, H, d, dsub, K, iters, order, cb, kept) == 0);
    for (int u = 0; u < H * M; ++u) CHECK(kept[u] >= 1 && kept[u] <= K);
    /* Lloyd with an SSE trace */
    double *pts = (double *)malloc(sizeof(double) * N * dsub), *C = (double *)malloc(sizeof(double) * K * dsub);
    double *trace = (double *)malloc(sizeof(double) * (2 * iters + 1));
    int32_t *as = (int32_t *)malloc(sizeof(int32_t) * N);
    for (int64_t i = 0; i < N * dsub; ++i) pts[i] = urand();
    for (int64_t i = 0; i < N; ++i) order[i] = (i * 7) % N;
    CHECK(orc_kmeans(pts, N, dsub, K, iters, order, C, as, trace) >= 1);
    for (int it = 1; it < 2 * iters; ++it) CHECK(trace[it] <= trace[it - 1] * (1 + 1e-12) + 1e-300);
    free(x); free(order); free(cb); free(kept); free(pts); free(C); free(trace); free(as);
}

static void decode_case(int B, int Hq, int Hkv, int d, int dsub, int K, int64_t Tcap, int64_t Rcap,
                        const int32_t *hist, const int32_t *rec) {
    const int M = d / dsub;
    float *q = frand((size_t)B * Hq * d), *cbk = frand((size_t)Hkv * K * M * dsub), *cbv = frand((size_t)Hkv * K * M * dsub);
    uint8_t *ck = (uint8_t *)malloc((size_t)B * Hkv * Tcap * M + 1), *cv = (uint8_t *)malloc((size_t)B * Hkv * Tcap * M + 1);
    for (int64_t i = 0; i < (int64_t)B * Hkv * Tcap * M; ++i) {
        ck[i] = (uint8_t)(rng % K);
        urand();
        cv[i] = (uint8_t)(rng % K);
        urand();
    }
    float *rk = frand((size_t)B * Hkv * Rcap * d), *rv = frand((size_t)B * Hkv * Rcap * d);
    double *out = (double *)malloc(sizeof(double) * B * Hq * d), *lse = (double *)malloc(sizeof(double) * B * Hq);
    CHECK(orc_decode_exact(B, Hq, Hkv, d, dsub, K, q, cbk, cbv, ck, cv, Tcap, hist, rk, rv, Rcap, rec, 0.125, out,
                           lse) == 0);
    for (int u = 0; u < B * Hq; ++u) {
        const int b = u / Hq;
        if (hist[b] + rec[b] == 0) CHECK(isinf(lse[u]) && lse[u] < 0);
        else CHECK(isfinite(lse[u]));
    }
    free(q); free(cbk); free(cbv); free(ck); free(cv); free(rk); free(rv); free(out); free(lse);
}

int main(void) {
    orc_set_threads(2);
    CHECK(orc_version() == 1 && orc_max_threads() >= 1);
    encode_case(1, 1, 4, 2, 1);
    encode_case(37, 3, 8, 2, 5);
    encode_case(20, 2, 16, 4, 256);
    encode_case(9, 1, 64, 4, 16);
    fit_case(1, 1, 4, 2, 1, 3, 0);
    fit_case(50, 2, 8, 2, 8, 4, 0);
    fit_case(30, 1, 8, 4, 16, 2, 5);  /* fewer distinct points than centroids */
    fit_case(64, 1, 4, 2, 4, 0, 0);   /* no iterations */
    {
        const int32_t h1[2] = {5, 0}, r1[2] = {3, 0};
        decode_case(2, 4, 2, 8, 2, 16, 8, 4, h1, r1);
        const int32_t h2[3] = {0, 64, 1}, r2[3] = {2, 0, 1};
        decode_case(3, 2, 1, 16, 4, 256, 64, 2, h2, r2);
        const int32_t h3[1] = {0}, r3[1] = {0};
        decode_case(1, 1, 1, 4, 2, 2, 1, 1, h3, r3);
    }
    CHECK(orc_encode(NULL, 1, 1, 5, 2, 4, NULL, NULL, NULL, NULL) == -1);  /* d % dsub */
    printf(fails ? "oracle_sanitize: %d failures\n" : "oracle_sanitize: ok\n", fails);
    return fails != 0;
}
