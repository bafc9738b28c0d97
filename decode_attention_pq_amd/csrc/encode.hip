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
// lane owns one token and walks its subspaces, holding one subvector (the next
// one already requested) and scanning all K centroids for it.  All lanes of a
// wave read the same centroid at the same time, so the LDS reads are broadcasts.
// The scan is plain fp32 VALU work: (x - c)^2 summed over the subspace, strict '<'
// in ascending centroid order; with K a multiple of 64 it costs 2*d_sub + 3
// instructions per (subvector, centroid) pair (nearest_code).

#include "nearest.h"

namespace pqkv {
namespace {

constexpr int kEncThreads = 1024;

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

    // One subspace at a time: the next subvector is requested before the current
    // one is scanned, so its latency hides behind K distance evaluations.
    const XT* row = x + b * s_seq + i * s_tok + h * s_head;
    const int64_t t = t_start + i;
    uint8_t* dst = code_slot<M>(codes + ((int64_t)b * Hkv + h) * t_cap * M, t);
    const int slot = (int)(t & (kTileTokens - 1));
    float nxt[DSUB];
    load_sub<DSUB>(row, nxt);
#pragma unroll 1
    for (int m = 0; m < M; ++m) {
        float xs[DSUB];
#pragma unroll
        for (int j = 0; j < DSUB; ++j) xs[j] = nxt[j];
        load_sub<DSUB>(row + (m + 1 < M ? m + 1 : m) * DSUB, nxt);
        put_code<M>(dst, slot, m, nearest_code<DSUB, D>(xs, cbs + m * DSUB, K));
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
