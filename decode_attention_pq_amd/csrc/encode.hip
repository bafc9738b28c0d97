// pq_encode: nearest-centroid codes for key/value head vectors.
//
// MILLION write-up (DAC 2025), page "MILLION": the paragraph after Fig. 5 splits
// the head vector into subspaces of dimension 2 or 4; the Fig. 6 paragraph
// encodes the prefill KV cache with the offline-trained codebooks.  The code of a
// subvector is the index of the centroid at the smallest squared Euclidean
// distance, the lowest index winning exact ties.
//
// Work decomposition (gfx950): one work-group per (token block, kv head, sequence).
// The head's codebook (K x d fp32, at most 128 KiB) is staged once into LDS; each
// lane owns one token, keeps its d-element row in registers and scans all K
// centroids of every subspace.  All lanes of a wave read the same centroid at the
// same time, so the LDS reads are broadcasts.  The scan is plain fp32 VALU work:
// (x - c)^2 summed over the subspace, strict '<' in ascending centroid order.

#include <hip/hip_fp16.h>

#include "pqkv_internal.h"

namespace pqkv {
namespace {

constexpr int kEncThreads = 512;

template <typename T>
struct Row;

template <>
struct Row<float> {
    template <int D>
    __device__ static void load(const float* __restrict__ p, float (&v)[D]) {
        const float4* p4 = reinterpret_cast<const float4*>(p);
#pragma unroll
        for (int i = 0; i < D / 4; ++i) {
            float4 t = p4[i];
            v[4 * i + 0] = t.x;
            v[4 * i + 1] = t.y;
            v[4 * i + 2] = t.z;
            v[4 * i + 3] = t.w;
        }
    }
};

template <>
struct Row<__half> {
    template <int D>
    __device__ static void load(const __half* __restrict__ p, float (&v)[D]) {
        const uint4* p4 = reinterpret_cast<const uint4*>(p);
#pragma unroll
        for (int i = 0; i < D / 8; ++i) {
            uint4 t = p4[i];
            const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                __half2 h2 = *reinterpret_cast<const __half2*>(&w[k]);
                float2 f = __half22float2(h2);
                v[8 * i + 2 * k + 0] = f.x;
                v[8 * i + 2 * k + 1] = f.y;
            }
        }
    }
};

template <int D, int DSUB, typename XT>
__global__ __launch_bounds__(kEncThreads) void encode_kernel(
    const XT* __restrict__ x, int64_t n_tokens, int64_t s_seq, int64_t s_tok, int64_t s_head,
    const float* __restrict__ cb, int K, int Hkv, uint8_t* __restrict__ codes, int64_t t_cap,
    int64_t t_start) {
    constexpr int M = D / DSUB;
    __shared__ float4 cbs4[kLdsRows * D / 4];  // [c][m][j], the global layout
    const float* cbs = reinterpret_cast<const float*>(cbs4);

    const int h = blockIdx.y;
    const int b = blockIdx.z;
    const float4* src = reinterpret_cast<const float4*>(cb + (int64_t)h * K * D);
    for (int i = threadIdx.x; i < K * D / 4; i += kEncThreads) cbs4[i] = src[i];
    __syncthreads();

    const int64_t i = (int64_t)blockIdx.x * kEncThreads + threadIdx.x;
    if (i >= n_tokens) return;

    float xv[D];
    Row<XT>::template load<D>(x + b * s_seq + i * s_tok + h * s_head, xv);

    const int64_t t = t_start + i;
    const int slot = (int)(t & (kTileTokens - 1));
    uint8_t* dst = codes + ((int64_t)b * Hkv + h) * t_cap * M + (t >> 6) * (kTileTokens * M) + slot * 16;

#pragma unroll
    for (int m = 0; m < M; ++m) {
        float best = INFINITY;
        int bi = 0;
        const float* cm = cbs + m * DSUB;
#pragma unroll 4
        for (int c = 0; c < K; ++c) {
            const float* cc = cm + c * D;
            float dd = 0.0f;
#pragma unroll
            for (int j = 0; j < DSUB; ++j) {
                const float e = xv[m * DSUB + j] - cc[j];
                dd = fmaf(e, e, dd);
            }
            if (dd < best) {
                best = dd;
                bi = c;
            }
        }
        const int p = (m - slot) & (M - 1);
        dst[(p >> 4) * (kTileTokens * 16) + (p & 15)] = (uint8_t)bi;
    }
}

template <int D, int DSUB, typename XT>
hipError_t launch_typed(const pqkv_dims& d, const void* x, int32_t n_seqs, int64_t n_tokens,
                        int64_t s_seq, int64_t s_tok, int64_t s_head, const float* cb,
                        uint8_t* codes, int64_t t_cap, int64_t t_start, hipStream_t stream) {
    dim3 grid((unsigned)((n_tokens + kEncThreads - 1) / kEncThreads), (unsigned)d.n_kv_heads,
              (unsigned)n_seqs);
    hipLaunchKernelGGL((encode_kernel<D, DSUB, XT>), grid, dim3(kEncThreads), 0, stream,
                       static_cast<const XT*>(x), n_tokens, s_seq, s_tok, s_head, cb,
                       d.n_centroids, d.n_kv_heads, codes, t_cap, t_start);
    return hipGetLastError();
}

template <int D, int DSUB>
hipError_t launch_dsub(const pqkv_dims& d, const void* x, pqkv_dtype xt, int32_t n_seqs,
                       int64_t n_tokens, int64_t s_seq, int64_t s_tok, int64_t s_head,
                       const float* cb, uint8_t* codes, int64_t t_cap, int64_t t_start,
                       hipStream_t stream) {
    if (xt == PQKV_F16)
        return launch_typed<D, DSUB, __half>(d, x, n_seqs, n_tokens, s_seq, s_tok, s_head, cb, codes,
                                             t_cap, t_start, stream);
    return launch_typed<D, DSUB, float>(d, x, n_seqs, n_tokens, s_seq, s_tok, s_head, cb, codes,
                                        t_cap, t_start, stream);
}

}  // namespace

hipError_t launch_encode(const pqkv_dims& d, const void* x, pqkv_dtype xt, int32_t n_seqs,
                         int64_t n_tokens, int64_t s_seq, int64_t s_tok, int64_t s_head,
                         const float* cb, uint8_t* codes, int64_t t_cap, int64_t t_start,
                         hipStream_t stream) {
    if (d.head_dim == 128 && d.d_sub == 2)
        return launch_dsub<128, 2>(d, x, xt, n_seqs, n_tokens, s_seq, s_tok, s_head, cb, codes, t_cap,
                                   t_start, stream);
    if (d.head_dim == 128 && d.d_sub == 4)
        return launch_dsub<128, 4>(d, x, xt, n_seqs, n_tokens, s_seq, s_tok, s_head, cb, codes, t_cap,
                                   t_start, stream);
    if (d.head_dim == 64 && d.d_sub == 2)
        return launch_dsub<64, 2>(d, x, xt, n_seqs, n_tokens, s_seq, s_tok, s_head, cb, codes, t_cap,
                                  t_start, stream);
    return launch_dsub<64, 4>(d, x, xt, n_seqs, n_tokens, s_seq, s_tok, s_head, cb, codes, t_cap,
                              t_start, stream);
}

}  // namespace pqkv
