// pq_encode on the matrix cores, for subspaces of dimension 4 and 256 centroids.
//
// MILLION write-up (DAC 2025), page "MILLION": the paragraph after Fig. 5 splits the
// head vector into subspaces of dimension 2 or 4; the Fig. 6 paragraph encodes the
// prefill KV cache with the offline-trained codebooks.  The code of a subvector is
// the index of the centroid at the smallest squared Euclidean distance, the lowest
// index winning exact ties.  The codes are those of the direct scan (nearest_codes):
// the decision is always taken on the fp32 distances sum_j (x_j - c_j)^2, and the
// matrix cores only narrow down where to look.
//
// Why the matrix cores: up to the common |x|^2, the distances of a subvector x to the
// centroids c are |c|^2 - 2 c.x, and for 16 centroids and 16 tokens the c.x part is a
// 16x16x4 product (one v_mfma_f32_16x16x4f32, K = 4 = d_sub) whose accumulator input
// is |c|^2.  At d_sub 4 the direct scan spends about 9 VALU lane-operations per
// (subvector, centroid) pair; here the products replace most of them.  (At d_sub 2 the
// direct scan needs about 5, which the products and their share of bookkeeping do not
// beat: the products and the vector work issue one after the other on a SIMD.)
//
// Pass 1 (matrix cores).  Lane l of a wave holds token j = l % 16 of a group of 16
// tokens and, of every block of 16 centroids, the 4 centroids 4g..4g+3 with
// g = l / 16 (the layout of the product's result).  For each block it takes the
// minimum over its 4 of
//     L_c = fl(|c|^2) - 2 c.x      (rounded fp32, as the product gives it)
// and keeps the smallest of those minima (its best group) and the second smallest.
// The minima are v_med3_f32 against -inf (a median that the compiler cannot turn back
// into a minimum, which would need NaN-quieting moves on every operand); NaN or
// infinite inputs make the bound below non-finite and take the direct scan.
//
// Pass 2 (exact).  Every lane computes the direct fp32 distances of its best group's
// 4 centroids; the 4 lanes of a token then keep the smallest distance, the lowest
// index on ties.  That is the direct scan's code whenever every centroid that could
// win lies in one of those groups, which the following bound establishes.
//
// The bound.  With u = 2^-24 and X = |x|^2: fl(|c|^2) (4 roundings) is within
// 4u|c|^2 of |c|^2; the product adds four terms to it, and each of its roundings (at
// most 8, however it orders them) is within u of a partial sum no larger than
// |c|^2 + 2|c||x| <= 2|c|^2 + X.  So L_c is within 20u|c|^2 + 8uX of
// E_c = |c|^2 - 2 c.x.  The direct distance d_c (6 roundings of non-negative terms)
// is within 6u |x - c|^2 <= 12u (X + |c|^2) of |x - c|^2 = X + E_c.  Let c be the
// centroid behind a lane's best value best_l, and c* the direct scan's winner
// (d_c* <= d_c).  Chaining the three estimates,
//     L_c* <= best_l + 32u |c|^2 + 32u |c*|^2 + 40u X.
// Both norms are bounded by the token itself: |c|^2 <= 2X + 2|x - c|^2, and
// |x - c|^2 = X + E_c is at most X + best_l to first order in u, so
// |c|^2 <= 4X + 2 best_l; c* is no farther from x than c, so the same holds for it.
// Hence (the u^2 terms are far inside the slack)
//     L_c* <= best_l + 296u X + 128u best_l <= best_l + 2^-15 (X + max(best_l, 0)),
// with 2^-15 = 512u leaving room for the rounding of the bound itself.  No
// centroid's norm enters it, so a codebook with far-out centroids (outlier channels)
// does not widen it.  Candidates are the groups whose value is at most
//     thr = min over the token's lanes of (best_l + 2^-15 (X + max(best_l, 0))) + 1e-30
// (the 1e-30 covers denormal operands, which the product may flush).  A lane whose
// second smallest group value is also <= thr -- a near tie, a small fraction of the
// subvectors -- a bound that is not finite (NaN or infinite inputs, overflow), or a
// subspace with a non-finite centroid sends the wave's groups to the direct scan of
// all 256 centroids, which gives the direct scan's codes by construction.
//
// Work decomposition (gfx950): one work-group of 1024 threads (16 waves, 4 per SIMD)
// per (4096 tokens, kv head, half of the subspaces, sequence).  The half's codebook
// is staged once in LDS as the product's operand rows: per (subspace, block of 16
// centroids), component k of centroid i at word 16k + i, then fl(|c|^2) of
// centroid i.  A wave takes one group of 16 tokens at a time and walks the subspaces
// for it, holding one subspace's operands (80 values a lane) at a time.

#include "nearest.h"

namespace pqkv {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMfDsub = 4;
constexpr int kMfThreads = 1024;
constexpr int kMfWaves = kMfThreads / 64;
constexpr int kMfGroups = 16;                          // groups of 16 tokens per wave
constexpr int kMfTokens = kMfWaves * kMfGroups * 16;   // tokens per work-group
constexpr int kMfBlocks = 16;                          // blocks of 16 centroids (K = 256)
constexpr int kMfWords = 16 * (kMfDsub + 1);           // operand-row words per (subspace, block)
constexpr int kMfCn = 16 * kMfDsub;                    // word of |c|^2 in a row
constexpr int kMfSlices = 4;                           // subspace quarters per kv head

// the bound's relative slack, 2^-15, and its absolute one
constexpr float kBound = 0x1p-15f;
constexpr float kBoundAbs = 1e-30f;
constexpr int kMfNg = 1;  // groups of 16 tokens a wave takes at a time

// Minimum over lanes l, l ^ 16, l ^ 32 and l ^ 48 (the 4 lanes of a token).  A
// permlane swap of a value with itself leaves each lane its own value and its
// partner's, in an order that depends on the row; the minimum of the two does not.
// The minimum is a median against `ninf` (-inf, opaque to the compiler), which takes
// no NaN-quieting moves on the swapped values.
__device__ inline float lanes_min(float v, float ninf) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __builtin_amdgcn_fmed3f(__uint_as_float(p[0]), __uint_as_float(p[1]), ninf);
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __builtin_amdgcn_fmed3f(__uint_as_float(r[0]), __uint_as_float(r[1]), ninf);
}

__device__ inline int lanes_min_int(int v) {
    const auto p = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
    v = min((int)p[0], (int)p[1]);
    const auto r = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
    return min((int)r[0], (int)r[1]);
}

// The same for (distance, index) pairs: the smaller distance, the lower index on
// equal ones (an order that does not depend on which of the two is the lane's own).
__device__ inline void lanes_argmin(float& d, int& i) {
#pragma unroll
    for (int step = 0; step < 2; ++step) {
        const auto pd = step == 0 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(d), __float_as_uint(d), false, false)
                                  : __builtin_amdgcn_permlane32_swap(__float_as_uint(d), __float_as_uint(d), false, false);
        const auto pi = step == 0 ? __builtin_amdgcn_permlane16_swap((uint32_t)i, (uint32_t)i, false, false)
                                  : __builtin_amdgcn_permlane32_swap((uint32_t)i, (uint32_t)i, false, false);
        const float d0 = __uint_as_float(pd[0]), d1 = __uint_as_float(pd[1]);
        const int i0 = (int)pi[0], i1 = (int)pi[1];
        const bool other = d1 < d0 || (d1 == d0 && i1 < i0);
        d = other ? d1 : d0;
        i = other ? i1 : i0;
    }
}

// Direct distances of one token's subvector to centroids c0 .. c0 + 3 (c0 a multiple of
// 4) of the staged rows `rows` of one subspace, strict < in ascending order: the
// running (distance, index) pair changes only for a smaller distance, so equal ones
// keep the lowest index and NaN distances never win.
__device__ inline void direct_scan_group(const float (&xs)[kMfDsub], const float* rows, int c0, float& bd, int& bi) {
    const float* r = rows + (c0 >> 4) * kMfWords + (c0 & 15);
    float cv[4][kMfDsub];
#pragma unroll
    for (int k = 0; k < kMfDsub; ++k) {  // 4 consecutive centroids: one 16-byte read per component
        const float4 v = *reinterpret_cast<const float4*>(r + 16 * k);
        cv[0][k] = v.x;
        cv[1][k] = v.y;
        cv[2][k] = v.z;
        cv[3][k] = v.w;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float dd = sq_dist<kMfDsub>(xs, cv[q]);
        const bool take = dd < bd;
        bd = take ? dd : bd;
        bi = take ? c0 + q : bi;
    }
}

template <int D, typename XT>
__global__ __launch_bounds__(kMfThreads) void encode_mfma_kernel(
    const XT* __restrict__ x, int64_t n_tokens, int64_t s_seq, int64_t s_tok, int64_t s_head,
    const float* __restrict__ cb, int Hkv, uint8_t* __restrict__ codes, int64_t t_cap, int64_t t_start) {
    constexpr int DSUB = kMfDsub;
    constexpr int M = D / DSUB;
    constexpr int MH = M / kMfSlices;  // subspaces of this work-group's quarter
    constexpr int K = kMfBlocks * 16;
    constexpr int W = kMfWords;
    __shared__ __align__(16) float rows[MH * kMfBlocks * W];  // [subspace][block][W]
    __shared__ uint32_t cnmax_bits[MH];  // per subspace: max |c|^2 (bits): below +inf iff all finite

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = blockIdx.y / kMfSlices;
    const int m0 = (blockIdx.y % kMfSlices) * MH;
    const int b = blockIdx.z;

    // ---- stage the half's codebook as operand rows.  Consecutive threads take
    // consecutive centroids of one block, so the LDS stores are conflict-free.
    for (int i = tid; i < MH; i += kMfThreads) cnmax_bits[i] = 0u;
    __syncthreads();
    const float* cbh = cb + (int64_t)h * K * M * DSUB;
    for (int e = tid; e < kMfBlocks * MH * 16; e += kMfThreads) {
        const int i = e & 15;
        const int mm = (e >> 4) % MH;
        const int bb = (e >> 4) / MH;
        const int c = bb * 16 + i;
        float v[DSUB];
        load_sub<DSUB>(cbh + ((int64_t)c * M + m0 + mm) * DSUB, v);
        float cn = v[0] * v[0];
#pragma unroll
        for (int k = 1; k < DSUB; ++k) cn = fmaf(v[k], v[k], cn);
        float* r = rows + (mm * kMfBlocks + bb) * W;
#pragma unroll
        for (int k = 0; k < DSUB; ++k) r[16 * k + i] = v[k];
        r[kMfCn + i] = cn;
        atomicMax(&cnmax_bits[mm], __float_as_uint(cn));  // non-negative: uint order
    }
    __syncthreads();

    const int j = lane & 15;  // token of the group
    const int g = lane >> 4;  // lane group: centroids 4g..4g+3 of every block; product row k = g
    uint8_t* plane = codes + ((int64_t)b * Hkv + h) * t_cap * M;
    const XT* xh = x + (int64_t)b * s_seq + (int64_t)h * s_head + m0 * DSUB;

    constexpr int NG = kMfNg;
    for (int grp = 0; grp < kMfGroups; grp += NG) {
        const int64_t t16 = (int64_t)blockIdx.x * kMfTokens + (int64_t)(grp * kMfWaves + wave) * 16;
        if (t16 >= n_tokens) break;  // the same for the whole wave
        bool live[NG];
        const XT* row[NG];
        uint8_t* dst[NG];
        int slot[NG];
        float xn[NG][DSUB];
#pragma unroll
        for (int q = 0; q < NG; ++q) {
            const int64_t tk = t16 + (int64_t)q * kMfWaves * 16 + j;
            live[q] = tk < n_tokens;
            const int64_t tl = live[q] ? tk : n_tokens - 1;  // a missing token repeats the last one
            row[q] = xh + tl * s_tok;
            dst[q] = code_slot<M>(plane, t_start + tl);
            slot[q] = (int)((t_start + tl) & (kTileTokens - 1));
            load_sub<DSUB>(row[q], xn[q]);
        }
#pragma unroll 1
        for (int mm = 0; mm < MH; ++mm) {
            const float* rm = rows + mm * kMfBlocks * W;
            const float cnsub = __uint_as_float(cnmax_bits[mm]);
            float xs[NG][DSUB], xx[NG], bv[NG];
#pragma unroll
            for (int q = 0; q < NG; ++q) {
#pragma unroll
                for (int k = 0; k < DSUB; ++k) xs[q][k] = xn[q][k];
                load_sub<DSUB>(row[q] + (mm + 1 < MH ? mm + 1 : mm) * DSUB, xn[q]);  // the next subvector
                float xg = xs[q][0];  // component g of token j: the product's row k = g
#pragma unroll
                for (int k = 1; k < DSUB; ++k) xg = g == k ? xs[q][k] : xg;
                bv[q] = -2.0f * xg;
                xx[q] = xs[q][0] * xs[q][0];
#pragma unroll
                for (int k = 1; k < DSUB; ++k) xx[q] = fmaf(xs[q][k], xs[q][k], xx[q]);
            }

            // ---- pass 1: the lane's value of every block, its best and second best.
            // med3 against -inf is the minimum; best <= second throughout, so
            // med3(best, t, second) is the new second smallest.
            float ninf = -INFINITY;
            asm volatile("" : "+v"(ninf));  // opaque: keeps each med3 a med3
            float best[NG], second[NG];
            int bidx[NG];
#pragma unroll
            for (int q = 0; q < NG; ++q) {
                best[q] = INFINITY;
                second[q] = INFINITY;
                bidx[q] = 0;
            }
#pragma unroll
            for (int bb = 0; bb < kMfBlocks; ++bb) {
                // the block's operand value (component g of centroid j) and fl(|c|^2) of
                // this lane's 4 centroids, the product's accumulator input
                const float av = rm[bb * W + lane];
                const float4 cn = *reinterpret_cast<const float4*>(rm + bb * W + kMfCn + 4 * g);
                const f32x4 c4 = {cn.x, cn.y, cn.z, cn.w};
#pragma unroll
                for (int q = 0; q < NG; ++q) {
                    const f32x4 acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv[q], c4, 0, 0, 0);
                    const float t = __builtin_amdgcn_fmed3f(__builtin_amdgcn_fmed3f(acc[0], acc[1], ninf),
                                                            __builtin_amdgcn_fmed3f(acc[2], acc[3], ninf), ninf);
                    bidx[q] = t < best[q] ? bb : bidx[q];
                    second[q] = __builtin_amdgcn_fmed3f(best[q], t, second[q]);
                    best[q] = __builtin_amdgcn_fmed3f(best[q], t, ninf);
                }
                // at most 4 blocks' products in flight: their results stay in registers
                if (bb % 4 == 3) __builtin_amdgcn_sched_barrier(0);
            }
            // ---- the bound, over the token's 4 lanes.  A candidate lane is one whose
            // best group value is within it; cbase is the first centroid of the
            // candidate group with the lowest index (every token has at least one:
            // the lane of its smallest value), and multi marks a second candidate.
            bool wide = !(cnsub < INFINITY), multi = false;
            int cbase[NG];
#pragma unroll
            for (int q = 0; q < NG; ++q) {
                const float thr = lanes_min(fmaf(kBound, xx[q] + fmaxf(best[q], 0.0f), best[q]), ninf) + kBoundAbs;
                wide = wide || !(fabsf(thr) < INFINITY) || second[q] <= thr;
                const bool cand = best[q] <= thr;
                const int key = cand ? bidx[q] * 16 + 4 * g : 0x7fffffff;
                cbase[q] = lanes_min_int(key);
                multi = multi || (cand && key != cbase[q]);
            }

            // ---- pass 2: direct distances of the candidates
            float bd[NG];
            int bi[NG];
#pragma unroll
            for (int q = 0; q < NG; ++q) {
                bd[q] = INFINITY;
                bi[q] = 0x7fffffff;
            }
            if (__any(wide)) {
                // every lane scans its 4 centroids of every block
#pragma unroll 1
                for (int bb = 0; bb < kMfBlocks; ++bb)
#pragma unroll
                    for (int q = 0; q < NG; ++q) direct_scan_group(xs[q], rm, bb * 16 + 4 * g, bd[q], bi[q]);
            } else if (__any(multi)) {
                // every lane scans its best group (those of lanes that are not
                // candidates hold no winner, and lose to one that does)
#pragma unroll
                for (int q = 0; q < NG; ++q) direct_scan_group(xs[q], rm, bidx[q] * 16 + 4 * g, bd[q], bi[q]);
            } else {
                // one candidate group per token: its 4 lanes take one centroid each
#pragma unroll
                for (int q = 0; q < NG; ++q) {
                    const int c = cbase[q] + g;
                    const float* r = rm + (c >> 4) * W + (c & 15);
                    float cv[kMfDsub];
#pragma unroll
                    for (int k = 0; k < kMfDsub; ++k) cv[k] = r[16 * k];
                    const float dd = sq_dist<kMfDsub>(xs[q], cv);
                    bd[q] = dd < INFINITY ? dd : INFINITY;  // NaN: never the winner
                    bi[q] = c;
                }
            }
#pragma unroll
            for (int q = 0; q < NG; ++q) {
                lanes_argmin(bd[q], bi[q]);
                // no distance below +inf: code 0, as the direct scan gives
                if (g == 0 && live[q]) put_code<M>(dst[q], slot[q], m0 + mm, bd[q] < INFINITY ? bi[q] : 0);
            }
        }
    }
}

template <int D, typename XT>
hipError_t launch_typed(const pqkv_dims& d, const void* x, int32_t n_seqs, int64_t n_tokens, int64_t s_seq,
                        int64_t s_tok, int64_t s_head, const float* cb, uint8_t* codes, int64_t t_cap,
                        int64_t t_start, hipStream_t stream) {
    dim3 grid((unsigned)((n_tokens + kMfTokens - 1) / kMfTokens), (unsigned)(d.n_kv_heads * kMfSlices),
              (unsigned)n_seqs);
    hipLaunchKernelGGL((encode_mfma_kernel<D, XT>), grid, dim3(kMfThreads), 0, stream, static_cast<const XT*>(x),
                       n_tokens, s_seq, s_tok, s_head, cb, d.n_kv_heads, codes, t_cap, t_start);
    return hipGetLastError();
}

template <int D>
hipError_t launch_head_dim(const pqkv_dims& d, const void* x, pqkv_dtype xt, int32_t n_seqs, int64_t n_tokens,
                           int64_t s_seq, int64_t s_tok, int64_t s_head, const float* cb, uint8_t* codes,
                           int64_t t_cap, int64_t t_start, hipStream_t stream) {
    if (xt == PQKV_F16)
        return launch_typed<D, __half>(d, x, n_seqs, n_tokens, s_seq, s_tok, s_head, cb, codes, t_cap, t_start,
                                       stream);
    return launch_typed<D, float>(d, x, n_seqs, n_tokens, s_seq, s_tok, s_head, cb, codes, t_cap, t_start, stream);
}

}  // namespace

bool encode_mfma_supported(const pqkv_dims& d) {
    return d.d_sub == kMfDsub && d.n_centroids == kMfBlocks * 16 && (d.head_dim == 128 || d.head_dim == 64);
}

hipError_t launch_encode_mfma(const pqkv_dims& d, const void* x, pqkv_dtype xt, int32_t n_seqs, int64_t n_tokens,
                              int64_t s_seq, int64_t s_tok, int64_t s_head, const float* cb, uint8_t* codes,
                              int64_t t_cap, int64_t t_start, hipStream_t stream) {
    if (d.head_dim == 128)
        return launch_head_dim<128>(d, x, xt, n_seqs, n_tokens, s_seq, s_tok, s_head, cb, codes, t_cap, t_start,
                                    stream);
    return launch_head_dim<64>(d, x, xt, n_seqs, n_tokens, s_seq, s_tok, s_head, cb, codes, t_cap, t_start, stream);
}

}  // namespace pqkv
