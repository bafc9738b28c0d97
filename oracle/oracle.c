/*
 * Plain fp64 CPU oracle for the product-quantised KV-cache method (MILLION,
 * DAC 2025; write-up "MILLION: product-quantisation based KV-cache
 * compression and decode acceleration").
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header, table or helper with the HIP
 * library.
 *
 * Everything is computed in double precision, from exact conversions of the
 * fp32 inputs (fp16 data is widened to fp32 exactly before it gets here), with
 * plain loops: no blocking, no reordering beyond what the definitions state.
 * OpenMP only spreads independent units (heads, subspaces, sequences) over
 * threads; the arithmetic inside a unit is sequential.
 *
 * Index conventions
 *   d      head dimension, dsub subspace dimension, M = d / dsub subspaces
 *   K      centroids per subspace
 *   codebook  [H][K][M][dsub]  (centroid-major, subspace-minor)
 *   codes     logical [..][T][M] uint8, one byte per (token, subspace)
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

int orc_version(void) { return 1; }

void orc_set_threads(int n) {
    if (n > 0) omp_set_num_threads(n);
}

int orc_max_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------------------------------ */
/* Squared Euclidean distance between a point and a centroid, fp64.          */
/* The page's clustering is k-means in the fused-channel space (Fig. 4-5     */
/* paragraphs) and PQ follows nearest-neighbour search practice, so the      */
/* distance is the squared L2 norm of the difference.                        */
static double sqdist(const double *x, const double *c, int dsub) {
    double s = 0.0;
    for (int j = 0; j < dsub; ++j) {
        double t = x[j] - c[j];
        s += t * t;
    }
    return s;
}

/* Nearest centroid with lowest-index tie-break; also the runner-up distance
 * (the smallest distance over every other index, so a duplicate centroid makes
 * it equal to the best).  One pass: a strictly smaller distance takes the best
 * slot and pushes the old best to runner-up; anything else can only lower the
 * runner-up. */
static void nearest(const double *x, const double *C, int K, int dsub,
                    int32_t *code, double *d1, double *d2) {
    int best = 0;
    double bd = sqdist(x, C, dsub);
    double second = INFINITY;
    for (int c = 1; c < K; ++c) {
        const double dc = sqdist(x, C + (int64_t)c * dsub, dsub);
        if (dc < bd) {
            second = bd;
            bd = dc;
            best = c;
        } else if (dc < second) {
            second = dc;
        }
    }
    *code = best;
    *d1 = bd;
    *d2 = second;
}

/* ------------------------------------------------------------------------ */
/* O1: Lloyd k-means in one subspace (offline calibration; the MILLION      */
/* write-up, the paragraphs on Fig. 5 (fused-channel clustering) and Fig. 6  */
/* (offline codebook training)).                                             */
/* Lloyd iterations from the given centroids C (K x dsub, updated in place): */
/* assign every point to its nearest centroid (lowest index on exact ties),  */
/* then move every non-empty centroid to the mean of its members; an empty   */
/* cluster keeps its centroid.                                               */
/*   assign out: the assignment used by the last update step (n entries);    */
/*          with iters == 0 the nearest assignment of the given centroids    */
/*   trace  out (nullable): 2*iters SSE values, after each assignment step   */
/*          and after each update step                                       */
int orc_lloyd(const double *X, int64_t n, int dsub, int K, int iters, double *C,
              int32_t *assign, double *trace) {
    if (n <= 0 || K <= 0 || dsub <= 0) return -1;
    double *sum = (double *)malloc(sizeof(double) * K * dsub);
    int64_t *cnt = (int64_t *)malloc(sizeof(int64_t) * K);
    for (int it = 0; it < iters; ++it) {
        double sse = 0.0;
        for (int64_t i = 0; i < n; ++i) {
            int32_t code;
            double d1, d2;
            nearest(X + i * dsub, C, K, dsub, &code, &d1, &d2);
            assign[i] = code;
            sse += d1;
        }
        if (trace) trace[2 * it] = sse;
        memset(sum, 0, sizeof(double) * K * dsub);
        memset(cnt, 0, sizeof(int64_t) * K);
        for (int64_t i = 0; i < n; ++i) {
            cnt[assign[i]] += 1;
            for (int j = 0; j < dsub; ++j) sum[assign[i] * dsub + j] += X[i * dsub + j];
        }
        for (int c = 0; c < K; ++c)
            if (cnt[c] > 0)
                for (int j = 0; j < dsub; ++j) C[c * dsub + j] = sum[c * dsub + j] / (double)cnt[c];
        if (trace) {
            double s2 = 0.0;
            for (int64_t i = 0; i < n; ++i) s2 += sqdist(X + i * dsub, C + assign[i] * dsub, dsub);
            trace[2 * it + 1] = s2;
        }
    }
    if (iters == 0)
        for (int64_t i = 0; i < n; ++i) {
            int32_t code;
            double d1, d2;
            nearest(X + i * dsub, C, K, dsub, &code, &d1, &d2);
            assign[i] = code;
        }
    free(sum);
    free(cnt);
    return 0;
}

/* Initialisation + Lloyd.                                                   */
/*   order  a permutation of 0..n-1 (the random draw of the initialisation)  */
/* Walk `order`, keep each point not equal in value to one already kept,     */
/* until K are kept; if fewer than K distinct points exist the remaining     */
/* slots are copies of slot 0.  Returns the number of distinct points kept   */
/* (or -1 on bad arguments).                                                 */
int64_t orc_kmeans(const double *X, int64_t n, int dsub, int K, int iters,
                   const int64_t *order, double *C, int32_t *assign, double *trace) {
    if (n <= 0 || K <= 0 || dsub <= 0) return -1;
    int64_t kept = 0;
    for (int64_t i = 0; i < n && kept < K; ++i) {
        const double *p = X + order[i] * dsub;
        int dup = 0;
        for (int64_t k = 0; k < kept && !dup; ++k) {
            int same = 1;
            for (int j = 0; j < dsub; ++j)
                if (C[k * dsub + j] != p[j]) { same = 0; break; }
            dup = same;
        }
        if (!dup) {
            memcpy(C + kept * dsub, p, sizeof(double) * dsub);
            ++kept;
        }
    }
    for (int64_t k = kept; k < K; ++k) memcpy(C + k * dsub, C, sizeof(double) * dsub);
    if (orc_lloyd(X, n, dsub, K, iters, C, assign, trace) != 0) return -1;
    return kept;
}

/* Fit every (head, subspace) codebook of one tensor.
 *   X      fp32 [N][H][d] token-major values
 *   order  [H][M][N] permutations
 *   cb     out fp64 [H][K][M][dsub]
 *   kept   out [H][M] distinct points kept by the initialisation */
int orc_fit_codebooks(const float *X, int64_t N, int H, int d, int dsub, int K, int iters,
                      const int64_t *order, double *cb, int64_t *kept) {
    if (d % dsub) return -1;
    const int M = d / dsub;
    int bad = 0;
#pragma omp parallel for schedule(dynamic) reduction(| : bad)
    for (int64_t u = 0; u < (int64_t)H * M; ++u) {
        const int h = (int)(u / M), m = (int)(u % M);
        double *pts = (double *)malloc(sizeof(double) * N * dsub);
        double *C = (double *)malloc(sizeof(double) * K * dsub);
        int32_t *as = (int32_t *)malloc(sizeof(int32_t) * N);
        for (int64_t t = 0; t < N; ++t)
            for (int j = 0; j < dsub; ++j)
                pts[t * dsub + j] = (double)X[(t * H + h) * d + m * dsub + j];
        int64_t k = orc_kmeans(pts, N, dsub, K, iters, order + (int64_t)(h * M + m) * N, C, as, NULL);
        if (k < 0) bad = 1;
        kept[h * M + m] = k;
        for (int c = 0; c < K; ++c)
            for (int j = 0; j < dsub; ++j)
                cb[(((int64_t)h * K + c) * M + m) * dsub + j] = C[c * dsub + j];
        free(pts);
        free(C);
        free(as);
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* O2: brute-force encode (online prefill quantisation: the MILLION         */
/* write-up, Fig. 6 paragraph).  For every (token, head, subspace) the code is the lowest     */
/* index attaining the minimum squared distance, evaluated over all K.       */
/*   x      fp32 [N][H][d]                                                   */
/*   cb     fp32 [H][K][M][dsub]                                             */
/*   codes  out [N][H][M]                                                    */
/*   d1,d2  out [N][H][M] best and runner-up distances (may be NULL)         */
int orc_encode(const float *x, int64_t N, int H, int d, int dsub, int K, const float *cb,
               uint8_t *codes, double *d1, double *d2) {
    if (d % dsub || K < 1 || K > 256) return -1;
    const int M = d / dsub;
#pragma omp parallel for schedule(dynamic)
    for (int64_t u = 0; u < (int64_t)H * M; ++u) {
        const int h = (int)(u / M), m = (int)(u % M);
        double *C = (double *)malloc(sizeof(double) * K * dsub);
        for (int c = 0; c < K; ++c)
            for (int j = 0; j < dsub; ++j)
                C[c * dsub + j] = (double)cb[(((int64_t)h * K + c) * M + m) * dsub + j];
        double p[8];
        for (int64_t t = 0; t < N; ++t) {
            for (int j = 0; j < dsub; ++j) p[j] = (double)x[(t * H + h) * d + m * dsub + j];
            int32_t code;
            double a, b;
            nearest(p, C, K, dsub, &code, &a, &b);
            const int64_t o = (t * H + h) * M + m;
            codes[o] = (uint8_t)code;
            if (d1) d1[o] = a;
            if (d2) d2[o] = b;
        }
        free(C);
    }
    return 0;
}

/* O2 in fp32: the same nearest-centroid rule, decided in single precision.  */
/* A code is an integer that floating point decides; the page fixes no      */
/* precision, so this is the decision in the precision the GPU computes in:   */
/* the squared distance evaluated in subspace order, e_j = x_j - c_j rounded  */
/* to fp32, then d = fma(e_j, e_j, d) from d = 0 (one rounding per term).     */
/* The first centroid with a strictly smaller d than every earlier one wins   */
/* (lowest index on ties); a NaN distance never wins, and a subvector with   */
/* no distance below +inf gets code 0.                                        */
static float sqdist_f32(const float *x, const float *c, int dsub) {
    float s = 0.0f;
    for (int j = 0; j < dsub; ++j) {
        const float e = x[j] - c[j];
        s = fmaf(e, e, s);
    }
    return s;
}

float orc_sqdist_f32(const float *x, const float *c, int dsub) { return sqdist_f32(x, c, dsub); }

int orc_encode_f32(const float *x, int64_t N, int H, int d, int dsub, int K, const float *cb, uint8_t *codes) {
    if (d % dsub || K < 1 || K > 256 || dsub > 8) return -1;
    const int M = d / dsub;
#pragma omp parallel for schedule(dynamic)
    for (int64_t u = 0; u < (int64_t)H * M; ++u) {
        const int h = (int)(u / M), m = (int)(u % M);
        float *C = (float *)malloc(sizeof(float) * K * dsub);
        for (int c = 0; c < K; ++c)
            for (int j = 0; j < dsub; ++j) C[c * dsub + j] = cb[(((int64_t)h * K + c) * M + m) * dsub + j];
        float p[8];
        for (int64_t t = 0; t < N; ++t) {
            for (int j = 0; j < dsub; ++j) p[j] = x[(t * H + h) * d + m * dsub + j];
            float best = INFINITY;
            int code = 0;
            for (int c = 0; c < K; ++c) {
                const float dc = sqdist_f32(p, C + c * dsub, dsub);
                if (dc < best) {
                    best = dc;
                    code = c;
                }
            }
            codes[(t * H + h) * M + m] = (uint8_t)code;
        }
        free(C);
    }
    return 0;
}

/* Distance of given codes (e.g. another implementation's), fp64, [N][H][M]. */
int orc_code_distance(const float *x, int64_t N, int H, int d, int dsub, int K, const float *cb,
                      const uint8_t *codes, double *dist) {
    if (d % dsub) return -1;
    const int M = d / dsub;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < N; ++t)
        for (int h = 0; h < H; ++h)
            for (int m = 0; m < M; ++m) {
                const int64_t o = (t * H + h) * M + m;
                const int c = codes[o];
                double s = 0.0;
                for (int j = 0; j < dsub; ++j) {
                    double v = (double)x[(t * H + h) * d + m * dsub + j] -
                               (c < K ? (double)cb[(((int64_t)h * K + c) * M + m) * dsub + j] : NAN);
                    s += v * v;
                }
                dist[o] = s;
            }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* O3 + O4: dequantise, then exact softmax attention (the plain definition   */
/* of what the blockwise history / recent-token attention of the MILLION    */
/* write-up, Fig. 7 paragraph, computes as a whole).  The decode query attends to every       */
/* cached token: the T_b history tokens (dequantised from their codes) and   */
/* the R_b recent full-precision tokens.                                     */
/*   q        fp32 [B][Hq][d]                                                */
/*   cb_k/v   fp32 [Hkv][K][M][dsub]                                         */
/*   codes_k/v logical [B][Hkv][Tcap][M]                                     */
/*   rk/rv    fp32 [B][Hkv][Rcap][d]                                         */
/*   out      fp64 [B][Hq][d];  lse fp64 [B][Hq] (natural log)               */
/* Query head hq reads kv head hq / (Hq/Hkv).  No tokens: out = 0, lse=-inf. */
int orc_decode_exact(int B, int Hq, int Hkv, int d, int dsub, int K, const float *q,
                     const float *cb_k, const float *cb_v, const uint8_t *codes_k,
                     const uint8_t *codes_v, int64_t Tcap, const int32_t *hist_len,
                     const float *rk, const float *rv, int64_t Rcap, const int32_t *recent_len,
                     double scale, double *out, double *lse) {
    if (d % dsub || Hq % Hkv) return -1;
    const int M = d / dsub, g = Hq / Hkv;
#pragma omp parallel for schedule(dynamic)
    for (int64_t u = 0; u < (int64_t)B * Hq; ++u) {
        const int b = (int)(u / Hq), hq = (int)(u % Hq), h = hq / g;
        const int64_t T = hist_len ? hist_len[b] : 0, R = recent_len ? recent_len[b] : 0;
        const int64_t n = T + R;
        double *o = out + u * d;
        for (int e = 0; e < d; ++e) o[e] = 0.0;
        if (n == 0) {
            lse[u] = -INFINITY;
            continue;
        }
        const float *qv = q + u * d;
        double *key = (double *)malloc(sizeof(double) * d);
        double *s = (double *)malloc(sizeof(double) * n);
        const uint8_t *ck = codes_k + ((int64_t)b * Hkv + h) * Tcap * M;
        const uint8_t *cv = codes_v + ((int64_t)b * Hkv + h) * Tcap * M;
        const float *rkh = rk ? rk + ((int64_t)b * Hkv + h) * Rcap * d : NULL;
        const float *rvh = rv ? rv + ((int64_t)b * Hkv + h) * Rcap * d : NULL;
        for (int64_t i = 0; i < n; ++i) {
            if (i < T) {
                for (int m = 0; m < M; ++m)
                    for (int j = 0; j < dsub; ++j)
                        key[m * dsub + j] =
                            (double)cb_k[(((int64_t)h * K + ck[i * M + m]) * M + m) * dsub + j];
            } else {
                for (int e = 0; e < d; ++e) key[e] = (double)rkh[(i - T) * d + e];
            }
            double dot = 0.0;
            for (int e = 0; e < d; ++e) dot += (double)qv[e] * key[e];
            s[i] = scale * dot;
        }
        double mu = -INFINITY;
        for (int64_t i = 0; i < n; ++i)
            if (s[i] > mu) mu = s[i];
        double Z = 0.0;
        for (int64_t i = 0; i < n; ++i) {
            const double p = exp(s[i] - mu);
            Z += p;
            if (i < T) {
                for (int m = 0; m < M; ++m)
                    for (int j = 0; j < dsub; ++j)
                        o[m * dsub + j] +=
                            p * (double)cb_v[(((int64_t)h * K + cv[i * M + m]) * M + m) * dsub + j];
            } else {
                for (int e = 0; e < d; ++e) o[e] += p * (double)rvh[(i - T) * d + e];
            }
        }
        for (int e = 0; e < d; ++e) o[e] /= Z;
        lse[u] = mu + log(Z);
        free(key);
        free(s);
    }
    return 0;
}

/* Dequantise codes into fp64 vectors: out [N][H][d] from codes [N][H][M]. */
int orc_dequantize(const uint8_t *codes, int64_t N, int H, int d, int dsub, int K, const float *cb,
                   double *out) {
    if (d % dsub) return -1;
    const int M = d / dsub;
    for (int64_t t = 0; t < N; ++t)
        for (int h = 0; h < H; ++h)
            for (int m = 0; m < M; ++m) {
                const int c = codes[(t * H + h) * M + m];
                for (int j = 0; j < dsub; ++j)
                    out[(t * H + h) * d + m * dsub + j] =
                        c < K ? (double)cb[(((int64_t)h * K + c) * M + m) * dsub + j] : NAN;
            }
    return 0;
}
