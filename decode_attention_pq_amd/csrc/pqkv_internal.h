// Internal declarations shared by the libpqkv translation units (host side).
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime.h>

#include "../../include/pqkv.h"
#include "decode_plan.h"

namespace pqkv {

hipError_t launch_encode(const pqkv_dims& d, const void* x, pqkv_dtype xt, int32_t n_seqs,
                         int64_t n_tokens, int64_t s_seq, int64_t s_tok, int64_t s_head,
                         const float* cb, uint8_t* codes, int64_t t_cap, int64_t t_start,
                         hipStream_t stream);

// The matrix-core form of pq_encode (same arguments, same codes), for the shapes
// encode_mfma_supported accepts (d_sub 4, 256 centroids).
bool encode_mfma_supported(const pqkv_dims& d);
hipError_t launch_encode_mfma(const pqkv_dims& d, const void* x, pqkv_dtype xt, int32_t n_seqs,
                              int64_t n_tokens, int64_t s_seq, int64_t s_tok, int64_t s_head,
                              const float* cb, uint8_t* codes, int64_t t_cap, int64_t t_start,
                              hipStream_t stream);

// The error-bounded expanded-form scan (same arguments, same codes), for the shapes
// encode_pruned_supported accepts (d_sub 2, a multiple of 64 centroids).
bool encode_pruned_supported(const pqkv_dims& d);
hipError_t launch_encode_pruned(const pqkv_dims& d, const void* x, pqkv_dtype xt, int32_t n_seqs,
                                int64_t n_tokens, int64_t s_seq, int64_t s_tok, int64_t s_head,
                                const float* cb, uint8_t* codes, int64_t t_cap, int64_t t_start,
                                hipStream_t stream);

hipError_t launch_build_lut(const pqkv_dims& d, int32_t batch, const void* q, pqkv_dtype qt,
                            const float* cb, float* lut, hipStream_t stream);

hipError_t launch_append(const pqkv_dims& d, int32_t batch, const void* new_k, const void* new_v,
                         void* recent_k, void* recent_v, pqkv_dtype rt, int64_t r_cap,
                         const int32_t* hist_in, const int32_t* recent_in, int32_t* hist_out,
                         int32_t* recent_out, int32_t n_roll, const float* cb_k, const float* cb_v,
                         uint8_t* codes_k, uint8_t* codes_v, int64_t t_cap, hipStream_t stream);

hipError_t launch_kmeans(const pqkv_dims& d, const void* x, pqkv_dtype xt, int64_t n, int64_t s_tok,
                         int64_t s_head, const int32_t* order, int32_t iters, float* cb, int32_t* kept,
                         hipStream_t stream);

// Dense fp16 decode attention (the full-precision baseline).
constexpr int kFp16Threads = 256;  // 4 waves per work-group

struct Fp16Plan {
    int n_split;           // token splits per (sequence, kv head)
    int64_t split_tokens;  // tokens per split (a multiple of 128)
    int partial_stride;    // floats per partial record: d outputs + max + sum, padded
    size_t partials_offset;
    size_t workspace_bytes;
};

struct Fp16Call {
    int head_dim, n_q_heads, n_kv_heads;
    const void* q;  // fp16 [B][Hq][d]
    const void* k;  // fp16 [B][Hkv][t_cap][d]
    const void* v;
    int64_t t_cap;
    const int32_t* seq_len;  // device [B]
    int64_t max_len;
    float scale;
    float* out;
    float* lse;
    float* partials;
    uint32_t* counters;
};

Fp16Plan plan_fp16_decode(int head_dim, int n_q_heads, int n_kv_heads, int32_t batch, int64_t max_len);

hipError_t launch_fp16_decode(const Fp16Plan& p, int32_t batch, const Fp16Call& c, hipStream_t stream);

hipError_t launch_merge_states(int64_t n_rows, int32_t head_dim, const float* out_a,
                               const float* lse_a, const float* out_b, const float* lse_b,
                               float* out, float* lse, hipStream_t stream);

}  // namespace pqkv
