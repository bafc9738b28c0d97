// pq_encode: nearest-centroid codes for key/value head vectors.
//
// MILLION write-up (DAC 2025), page "MILLION": the paragraph after Fig. 5 splits
// the head vector into subspaces of dimension 2 or 4; the Fig. 6 paragraph
// encodes the prefill KV cache with the offline-trained codebooks.  The code of a
// subvector is the index of the centroid at the smallest squared Euclidean
// distance, the lowest index winning exact ties.
//
// This is the encode for the shapes the two narrowing scans do not take: at d_sub 4
// with 256 centroids the matrix cores narrow the scan down first (encode_mfma.hip),
// and at d_sub 2 with a multiple of 64 centroids an error-bounded expanded-form scan
// does (encode_pruned.hip); the same codes come out of both.
//
// Work decomposition (gfx950): one work-group of 1024 threads per (token block,
// kv head, sequence).  The head's codebook (K x d fp32, at most 128 KiB) is staged
// once into LDS; each lane owns 4 tokens (d_sub 2) or 2 (d_sub 4) and walks their
// subspaces, holding one subvector of each (the next ones already requested) and
// scanning all K centroids for them.  All lanes of a wave read the same centroid
// at the same time, so the LDS reads are broadcasts, and each value read serves
// every token of the lane: the LDS traffic per (subvector, centroid) pair is a
// quarter or a half of one read.  The scan is plain fp32 VALU work: (x - c)^2
// summed over the subspace, then, for K a multiple of 64, a minimum per 16
// centroids and a rescan of the winning 16 (nearest_codes).

#include "nearest.h"

namespace pqkv {
namespace {

constexpr int kEncThreads = 1024;
// tokens per lane (every centroid value read from LDS serves all of them): as many
// as the registers of four waves per SIMD hold
template <int DSUB>
constexpr int enc_tokens_per_lane() { return DSUB == 2 ? 4 : 2; }
// floats between sub-blocks of 16 centroid rows in LDS, so that the sub-blocks the
// lanes of a half-wave rescan sit on different banks: the codebook rows are a
// multiple of 32 banks long, so sub-block b starts on bank PAD*b mod 32 -- with 2
// floats (d_sub 2, 8-byte reads) the 16 sub-blocks of 256 centroids tile the 32
// banks; 16-byte reads (d_sub 4) need 4
template <int DSUB>
constexpr int enc_pad() { return DSUB == 2 ? 2 : 4; }

template <int D, int DSUB, typename XT>
__global__ __launch_bounds__(kEncThreads) void encode_kernel(
    const XT* __restrict__ x, int64_t n_tokens, int64_t s_seq, int64_t s_tok, int64_t s_head,
    const float* __restrict__ cb, int K, int Hkv, uint8_t* __restrict__ codes, int64_t t_cap,
    int64_t t_start) {
    constexpr int M = D / DSUB;
    constexpr int PAD = enc_pad<DSUB>();
    // [c][m][j], the global layout, with PAD floats after every 16 centroid rows
    __shared__ float2 cbs2[(kLdsRows * D + kLdsRows / 16 * PAD) / 2];
    const float* cbs = reinterpret_cast<const float*>(cbs2);

    const int h = blockIdx.y;
    const int b = blockIdx.z;
    const float2* src = reinterpret_cast<const float2*>(cb + (int64_t)h * K * D);
    for (int i = threadIdx.x; i < K * D / 2; i += kEncThreads) cbs2[i + i / (8 * D) * (PAD / 2)] = src[i];
    __syncthreads();

    // tokens i, i + kEncThreads, ... of the work-group's block
    constexpr int NT = enc_tokens_per_lane<DSUB>();
    const int64_t i = (int64_t)blockIdx.x * (NT * kEncThreads) + threadIdx.x;
    if (i >= n_tokens) return;
    const XT* row[NT];
    uint8_t* dst[NT];
    int slot[NT];
    bool live[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        live[n] = i + n * kEncThreads < n_tokens;
        const int64_t in = live[n] ? i + n * kEncThreads : i;  // a missing token repeats the first
        row[n] = x + b * s_seq + in * s_tok + h * s_head;
        const int64_t t = t_start + in;
        dst[n] = code_slot<M>(codes + ((int64_t)b * Hkv + h) * t_cap * M, t);
        slot[n] = (int)(t & (kTileTokens - 1));
    }

    // One subspace at a time: the next subvectors are requested before the current
    // ones are scanned, so their latency hides behind K distance evaluations.
    float nxt[NT][DSUB];
#pragma unroll
    for (int n = 0; n < NT; ++n) load_sub<DSUB>(row[n], nxt[n]);
#pragma unroll 1
    for (int m = 0; m < M; ++m) {
        float xs[NT][DSUB];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
#pragma unroll
            for (int j = 0; j < DSUB; ++j) xs[n][j] = nxt[n][j];
            load_sub<DSUB>(row[n] + (m + 1 < M ? m + 1 : m) * DSUB, nxt[n]);
        }
        int code[NT];
        nearest_codes<DSUB, D, PAD, NT>(xs, cbs + m * DSUB, K, code);
#pragma unroll
        for (int n = 0; n < NT; ++n)
            if (live[n]) put_code<M>(dst[n], slot[n], m, code[n]);
    }
}

template <int D, int DSUB, typename XT>
hipError_t launch_typed(const pqkv_dims& d, const void* x, int32_t n_seqs, int64_t n_tokens,
                        int64_t s_seq, int64_t s_tok, int64_t s_head, const float* cb,
                        uint8_t* codes, int64_t t_cap, int64_t t_start, hipStream_t stream) {
    constexpr int block = enc_tokens_per_lane<DSUB>() * kEncThreads;
    dim3 grid((unsigned)((n_tokens + block - 1) / block), (unsigned)d.n_kv_heads,
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
    if (encode_mfma_supported(d))  // the same codes from the matrix cores (encode_mfma.hip)
        return launch_encode_mfma(d, x, xt, n_seqs, n_tokens, s_seq, s_tok, s_head, cb, codes, t_cap, t_start,
                                  stream);
    if (encode_pruned_supported(d))  // the same codes from a bounded expanded-form scan (encode_pruned.hip)
        return launch_encode_pruned(d, x, xt, n_seqs, n_tokens, s_seq, s_tok, s_head, cb, codes, t_cap, t_start,
                                    stream);
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
