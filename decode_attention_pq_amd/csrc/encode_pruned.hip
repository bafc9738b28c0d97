// pq_encode at d_sub 2 by an error-bounded scan in the expanded form.
//
// MILLION write-up (DAC 2025), page "MILLION": the paragraph after Fig. 5 splits the
// head vector into subspaces of dimension 2 or 4; the Fig. 6 paragraph encodes the
// prefill KV cache with the offline-trained codebooks.  The code of a subvector is
// the index of the centroid at the smallest squared Euclidean distance, the lowest
// index winning exact ties.  The codes are those of the direct scan (nearest_codes):
// the decision is always taken on the fp32 distances sum_j (x_j - c_j)^2.
//
// Why: the direct distance costs 4 VALU instructions per (subvector, centroid) pair
// at d_sub 2 (two differences, two fused squares).  Up to the common |x|^2, the
// distance is |c|^2 - 2 c.x, which is 2 fused multiply-adds from a stored |c|^2 and
// -2x.  Its rounding error grows with |x|^2 and |c|^2 instead of with the distance,
// so this form only narrows the scan down: pass 1 finds the sub-block of 16
// centroids with the smallest value and the bound below proves that the winner lies
// in it; pass 2 rescans those 16 with the direct distance.
//
// Pass 1.  Per sub-block of 16 centroids, for each of the lane's tokens:
//     L_c = fma(c_1, -2 x_1, fma(c_0, -2 x_0, fl(|c|^2))),   fl(|c|^2) = fma(c_1, c_1, c_0 c_0)
// and the minimum of the 16 (trees of three-operand mins).  The sub-block's number
// replaces the low 4 bits of that minimum (moving it by under 16 ulp, 2^-19 of its
// magnitude), and across sub-blocks the three smallest of these tagged values are
// kept by medians: 4 instructions per sub-block and token, no index bookkeeping.
//
// The bound.  With u = 2^-24, X = |x|^2 and d = d_sub: fl(|c|^2) (d roundings) is
// within d u |c|^2 of |c|^2, and each of the d fused steps rounds within u of a
// partial sum no larger than |c|^2 + 2|c||x| <= 2|c|^2 + X, so L_c is within
// 3d u |c|^2 + d u X of E_c = |c|^2 - 2 c.x.  The direct distance (two roundings of
// each difference's square, d of the sum) is within (d + 2) u D_c of
// D_c = |x - c|^2 = X + E_c.  Let c be the centroid behind the smallest value best
// and c* the direct scan's winner (its distance is at most c's).  To first order in
// u, D_c <= X + best, D_c* <= D_c, and |c|^2, |c*|^2 <= 2X + 2 D_c <= 4X + 2 best,
// so chaining the estimates gives
//     L_c* <= best + (28d + 4) u X + (14d + 4) u best,
// at d = 2: best + 60u X + 32u best.  The tags move the best sub-block's minimum
// and the winner's sub-block minimum by at most 2^-19 = 32u of their magnitudes,
// which are at most X + |best| to first order (every L is at least -X), so with
// best now the smallest tagged value the winner's sub-block has a tagged minimum of
// at most best + 124u (X + |best|) <= best + 192u (X + |best|), with room for the
// rounding of the bound itself.  No centroid's norm enters it.  Candidates are
// therefore the sub-blocks whose tagged minimum is at most
//     thr = best + 192u (X + |best|) + 1e-30
// (the 1e-30 covers denormal operands).  Pass 2 rescans the best sub-block with the
// direct distance, and also the second best when its minimum is within thr (a near
// tie, a few in 10^4 subvectors), in ascending order with a strict <, so the lowest
// index at the smallest distance wins as in the direct scan.  When the third
// smallest minimum is within thr as well, or thr is not finite (NaN or infinite
// inputs, overflow), or the subspace has a non-finite |c|^2, the wave scans the
// subspace directly for all its tokens (a strict < scan of every centroid), which
// gives the direct scan's codes by construction.
//
// Work decomposition (gfx950): one work-group of 1024 threads (16 waves, 4 per SIMD)
// per (4096 tokens, kv head, sequence), one per CU.  The head's codebook is staged in
// LDS subspace-major -- per subspace, each sub-block's 16 centroids as (c_0, c_1)
// pairs, then 4 floats of padding (144 KiB at head_dim 128) -- so one 16-byte
// broadcast read brings two centroids to every lane, 8 bytes per centroid as in the
// direct scan.  Each lane owns 4 tokens and walks the subspaces; each centroid value
// read, and its fl(|c|^2) (computed on the fly), serves all 4.  A sub-block is taken
// in two halves of 8 centroids, which keeps a lane within the 128 registers of four
// waves per SIMD.  (Staging fl(|c|^2) in LDS instead needs half of the subspaces per
// work-group to fit, and measured slower.)

#include "nearest.h"

namespace pqkv {
namespace {

constexpr int kPrThreads = 1024;
constexpr int kPrDsub = 2;
constexpr int kPrNt = 4;    // tokens per lane
constexpr int kPrHalf = 8;  // centroids per half sub-block
constexpr int kPrSb = 16;   // centroids per sub-block
constexpr int kPrPad = 4;   // floats after every sub-block (keeps 16-byte reads aligned)
constexpr int kPrSbs = kPrSb * kPrDsub + kPrPad;  // floats per sub-block
// the bound's relative slack, 192u, and its absolute one
constexpr float kPrSlack = 192.0f * 0x1p-24f;
constexpr float kPrAbs = 1e-30f;

template <int D, typename XT>
__global__ __launch_bounds__(kPrThreads) void encode_pruned_kernel(
    const XT* __restrict__ x, int64_t n_tokens, int64_t s_seq, int64_t s_tok, int64_t s_head,
    const float* __restrict__ cb, int K, int Hkv, uint8_t* __restrict__ codes, int64_t t_cap,
    int64_t t_start) {
    constexpr int DSUB = kPrDsub;
    constexpr int M = D / DSUB;
    constexpr int SS = kLdsRows / kPrSb * kPrSbs;  // floats per subspace
    constexpr int NT = kPrNt;
    // subspace m, centroid c at rows + m * SS + (c / 16) * kPrSbs + (c % 16) * 2
    __shared__ __align__(16) float rows[M * SS];
    __shared__ uint32_t cn_bits[M];  // per subspace: max fl(|c|^2) bits, below +inf iff all finite

    const int tid = threadIdx.x;
    const int h = blockIdx.y;
    const int b = blockIdx.z;

    // ---- stage the head's codebook.  Consecutive threads take consecutive centroids
    // of one subspace: contiguous 8-byte LDS stores (the global reads are strided, and
    // served by L2 after the first work-group of the head).
    for (int i = tid; i < M; i += kPrThreads) cn_bits[i] = 0u;
    __syncthreads();
    const float* cbh = cb + (int64_t)h * K * M * DSUB;
    for (int e = tid; e < K * M; e += kPrThreads) {
        const int m = e / K;
        const int c = e - m * K;
        const float2 v = *reinterpret_cast<const float2*>(cbh + ((int64_t)c * M + m) * DSUB);
        *reinterpret_cast<float2*>(rows + m * SS + (c / kPrSb) * kPrSbs + (c % kPrSb) * DSUB) = v;
        atomicMax(&cn_bits[m], __float_as_uint(fmaf(v.y, v.y, v.x * v.x)));  // non-negative or NaN
    }
    __syncthreads();

    // tokens i, i + 1024, ... of the work-group's block
    const int64_t i = (int64_t)blockIdx.x * (NT * kPrThreads) + tid;
    if (i >= n_tokens) return;
    const XT* row[NT];
    uint8_t* dst[NT];
    int slot[NT];
    bool live[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        live[n] = i + n * kPrThreads < n_tokens;
        const int64_t in = live[n] ? i + n * kPrThreads : i;  // a missing token repeats the first
        row[n] = x + b * s_seq + in * s_tok + h * s_head;
        const int64_t t = t_start + in;
        dst[n] = code_slot<M>(codes + ((int64_t)b * Hkv + h) * t_cap * M, t);
        slot[n] = (int)(t & (kTileTokens - 1));
    }

    float nxt[NT][DSUB];
#pragma unroll
    for (int n = 0; n < NT; ++n) load_sub<DSUB>(row[n], nxt[n]);
    const int n_sb = K / kPrSb;
#pragma unroll 1
    for (int m = 0; m < M; ++m) {
        float xs[NT][DSUB];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
#pragma unroll
            for (int j = 0; j < DSUB; ++j) xs[n][j] = nxt[n][j];
            load_sub<DSUB>(row[n] + (m + 1 < M ? m + 1 : m) * DSUB, nxt[n]);
        }
        float bx0[NT], bx1[NT], xx[NT], best[NT], second[NT], third[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            bx0[n] = -2.0f * xs[n][0];
            bx1[n] = -2.0f * xs[n][1];
            xx[n] = fmaf(xs[n][1], xs[n][1], xs[n][0] * xs[n][0]);
            best[n] = INFINITY;
            second[n] = INFINITY;
            third[n] = INFINITY;
        }
        const float* base = rows + m * SS;
        float ninf = -INFINITY;
        asm volatile("" : "+v"(ninf));  // opaque: keeps each med3 a med3

        // ---- pass 1: the three smallest tagged sub-block minima of L
#pragma unroll 1
        for (int s = 0; s < n_sb; ++s) {
            const float* sp = base + s * kPrSbs;
            float hm[2][NT];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                float c0[kPrHalf], c1[kPrHalf], cn[kPrHalf];
#pragma unroll
                for (int r = 0; r < kPrHalf; r += 2) {  // one broadcast read per two centroids
                    const float4 v = *reinterpret_cast<const float4*>(sp + (hf * kPrHalf + r) * DSUB);
                    c0[r] = v.x;
                    c1[r] = v.y;
                    c0[r + 1] = v.z;
                    c1[r + 1] = v.w;
                }
#pragma unroll
                for (int r = 0; r < kPrHalf; ++r) cn[r] = fmaf(c1[r], c1[r], c0[r] * c0[r]);
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    float l[kPrHalf];
#pragma unroll
                    for (int r = 0; r < kPrHalf; ++r) l[r] = fmaf(c1[r], bx1[n], fmaf(c0[r], bx0[n], cn[r]));
                    const float t0 = fminf(fminf(l[0], l[1]), l[2]);
                    const float t1 = fminf(fminf(l[3], l[4]), l[5]);
                    hm[hf][n] = fminf(fminf(t0, t1), fminf(l[6], l[7]));
                }
            }
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                // the minimum tagged with the sub-block's number in its low 4 bits
                const float tg = __uint_as_float((__float_as_uint(fminf(hm[0][n], hm[1][n])) & ~15u) | (uint32_t)s);
                // best <= second <= third throughout: the medians keep them sorted
                third[n] = __builtin_amdgcn_fmed3f(second[n], tg, third[n]);
                second[n] = __builtin_amdgcn_fmed3f(best[n], tg, second[n]);
                best[n] = __builtin_amdgcn_fmed3f(best[n], tg, ninf);
            }
        }

        // ---- the bound: at most two candidate sub-blocks per token, for every token of the wave?
        bool wide = !(__uint_as_float(cn_bits[m]) < INFINITY);
        bool two[NT];
        int bsb[NT], ssb[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const float thr = fmaf(kPrSlack, xx[n] + fabsf(best[n]), best[n]) + kPrAbs;
            wide = wide || !(fabsf(thr) < INFINITY) || third[n] <= thr;
            two[n] = second[n] <= thr;
            bsb[n] = (int)(__float_as_uint(best[n]) & 15u);
            ssb[n] = (int)(__float_as_uint(second[n]) & 15u);
        }
        int code[NT];
        if (__any(wide)) {
            // the direct scan of every centroid, strict < upwards (the lowest index at
            // the smallest distance; NaN distances never win; none below +inf: code 0)
            float bd[NT];
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                bd[n] = INFINITY;
                code[n] = 0;
            }
#pragma unroll 2
            for (int c = 0; c < K; ++c) {
                const float2 v = *reinterpret_cast<const float2*>(base + (c / kPrSb) * kPrSbs + (c % kPrSb) * DSUB);
                const float cv[DSUB] = {v.x, v.y};
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    const float dd = sq_dist<DSUB>(xs[n], cv);
                    const bool take = dd < bd[n];
                    bd[n] = take ? dd : bd[n];
                    code[n] = take ? c : code[n];
                }
            }
        } else {
            // ---- pass 2: the direct distances of the candidate sub-blocks, in ascending
            // order, strict < (the second one only for the lanes whose token needs it)
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                const int lo = two[n] ? min(bsb[n], ssb[n]) : bsb[n];
                float bd = INFINITY;
                int bi = 0;
                auto scan = [&](int sb) {
                    const float* sp = base + sb * kPrSbs;
#pragma unroll
                    for (int r = 0; r < kPrSb; ++r) {
                        const float2 v = *reinterpret_cast<const float2*>(sp + r * DSUB);
                        const float cv[DSUB] = {v.x, v.y};
                        const float dd = sq_dist<DSUB>(xs[n], cv);
                        const bool take = dd < bd;
                        bd = take ? dd : bd;
                        bi = take ? sb * kPrSb + r : bi;
                    }
                };
                scan(lo);
                if (two[n]) scan(max(bsb[n], ssb[n]));
                // no distance below +inf: code 0, as the direct scan gives
                code[n] = bd < INFINITY ? bi : 0;
            }
        }
#pragma unroll
        for (int n = 0; n < NT; ++n)
            if (live[n]) put_code<M>(dst[n], slot[n], m, code[n]);
    }
}

template <int D, typename XT>
hipError_t launch_typed(const pqkv_dims& d, const void* x, int32_t n_seqs, int64_t n_tokens, int64_t s_seq,
                        int64_t s_tok, int64_t s_head, const float* cb, uint8_t* codes, int64_t t_cap,
                        int64_t t_start, hipStream_t stream) {
    constexpr int block = kPrNt * kPrThreads;
    dim3 grid((unsigned)((n_tokens + block - 1) / block), (unsigned)d.n_kv_heads, (unsigned)n_seqs);
    hipLaunchKernelGGL((encode_pruned_kernel<D, XT>), grid, dim3(kPrThreads), 0, stream, static_cast<const XT*>(x),
                       n_tokens, s_seq, s_tok, s_head, cb, d.n_centroids, d.n_kv_heads, codes, t_cap, t_start);
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

bool encode_pruned_supported(const pqkv_dims& d) {
    return d.d_sub == kPrDsub && d.n_centroids % 64 == 0 && d.n_centroids <= kLdsRows &&
           (d.head_dim == 128 || d.head_dim == 64);
}

hipError_t launch_encode_pruned(const pqkv_dims& d, const void* x, pqkv_dtype xt, int32_t n_seqs,
                                int64_t n_tokens, int64_t s_seq, int64_t s_tok, int64_t s_head, const float* cb,
                                uint8_t* codes, int64_t t_cap, int64_t t_start, hipStream_t stream) {
    if (d.head_dim == 128)
        return launch_head_dim<128>(d, x, xt, n_seqs, n_tokens, s_seq, s_tok, s_head, cb, codes, t_cap, t_start,
                                    stream);
    return launch_head_dim<64>(d, x, xt, n_seqs, n_tokens, s_seq, s_tok, s_head, cb, codes, t_cap, t_start, stream);
}

}  // namespace pqkv
