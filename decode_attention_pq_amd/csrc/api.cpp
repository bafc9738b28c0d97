// libpqkv C interface: argument validation, split planning and dispatch.
//
// Every entry point validates its arguments on the host and returns a status
// before anything is enqueued; kernels are launched asynchronously on the
// caller's stream.  No exception crosses the interface.

#include <cstdint>
#include <cstring>

#include "pqkv_internal.h"

namespace pqkv {
namespace {

bool dims_ok(const pqkv_dims* d) {
    if (!d) return false;
    if (d->head_dim != 64 && d->head_dim != 128) return false;
    if (d->d_sub != 2 && d->d_sub != 4) return false;
    if (d->n_centroids < 2 || d->n_centroids > 256) return false;
    if (d->n_q_heads < 1 || d->n_kv_heads < 1) return false;
    if (d->n_q_heads % d->n_kv_heads) return false;
    if (d->n_kv_heads > 65535) return false;
    return true;
}

bool dtype_ok(pqkv_dtype t) { return t == PQKV_F16 || t == PQKV_F32; }

size_t dtype_bytes(pqkv_dtype t) { return t == PQKV_F16 ? 2 : 4; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Distinguish "bad argument" from "well-formed but not supported".
pqkv_status check_dims(const pqkv_dims* d) {
    if (!d) return PQKV_ERR_INVALID;
    if (d->n_q_heads < 1 || d->n_kv_heads < 1 || d->head_dim < 1 || d->d_sub < 1 || d->n_centroids < 1)
        return PQKV_ERR_INVALID;
    if (d->n_q_heads % d->n_kv_heads || d->head_dim % d->d_sub) return PQKV_ERR_INVALID;
    return dims_ok(d) ? PQKV_OK : PQKV_ERR_UNSUPPORTED;
}

pqkv_status hip_status(hipError_t e) { return e == hipSuccess ? PQKV_OK : PQKV_ERR_HIP; }

// Byte ranges [a, a + n) and [b, b + n) overlap.
bool overlap(const void* a, const void* b, size_t n) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + n && y < x + n;
}

}  // namespace

DecodePlan plan_decode(const pqkv_dims& d, int32_t batch, int64_t max_hist_len) {
    DecodePlan p{};
    const int M = d.head_dim / d.d_sub;
    const int g = d.n_q_heads / d.n_kv_heads;
    // query heads per work-group: as many as share an LDS row, dividing the group size
    int qh = 1;
    for (int c : {4, 2}) {
        if (c * M <= 64 && g % c == 0) {
            qh = c;
            break;
        }
    }
    p.qh = qh;
    p.n_groups = g / qh;
    p.partial_stride = d.head_dim + 4;
    p.units = (int64_t)batch * d.n_kv_heads * p.n_groups;
    if (max_hist_len <= 0) {
        // recent window only: one work-group per unit
        p.rounds = 0;
        p.n_split = 1;
        p.split_tokens = 0;
    } else {
        // Every candidate tiles-per-wave count r gives the fewest splits of at most r
        // rounds, cut evenly, run in the smallest kernel build that holds them.  Its
        // cost is modelled as the work-group waves the CUs run one after another, each
        // paying a work-group's fixed costs (codebooks, LUT, epilogue, merge; about 2.4
        // rounds of streaming), its rounds, and 0.15 round per unused step of the build.
        // The cheapest wins, fewer work-groups on a tie.
        const int64_t per_tok = kTokensPerRound;
        int64_t n_split = 0, rounds = 0, best_cost = 0, best_items = 0;
        for (int r = 1; r <= decode_max_rounds(M, qh); ++r) {
            const int64_t ns = (max_hist_len + r * per_tok - 1) / (r * per_tok);
            const int64_t rr = (max_hist_len + ns * per_tok - 1) / (ns * per_tok);
            // past the merge's split limit only the longest candidate is kept (and refused)
            if (ns > kMaxSplits && (n_split != 0 || r < decode_max_rounds(M, qh))) continue;
            const int64_t items = p.units * ns;
            const int64_t waves = (items + kPlanCUs - 1) / kPlanCUs;
            const int64_t cost =
                waves * (kPlanFixed + kPlanRound * rr + kPlanUnused * (decode_kernel_rounds(M, qh, (int)rr) - rr));
            if (n_split == 0 || cost < best_cost || (cost == best_cost && items < best_items)) {
                n_split = ns;
                rounds = rr;
                best_cost = cost;
                best_items = items;
            }
        }
        p.rounds = (int)rounds;
        p.n_split = (int)n_split;
        p.split_tokens = rounds * kTokensPerRound;
    }
    const size_t part = (size_t)batch * d.n_q_heads * p.n_split * p.partial_stride * sizeof(float);
    p.partials_offset = decode_counter_bytes(batch, d.n_q_heads);
    p.workspace_bytes = p.partials_offset + (part + 255) / 256 * 256;
    return p;
}

pqkv_status check_decode_args(const pqkv_dims* dims, int32_t batch, const void* q, pqkv_dtype q_dtype,
                              const float* lut, const float* codebook_k, const float* codebook_v,
                              const uint8_t* codes_k, const uint8_t* codes_v, int64_t t_cap,
                              const int32_t* hist_len, int64_t max_hist_len, const void* recent_k,
                              const void* recent_v, pqkv_dtype recent_dtype, int64_t r_cap,
                              const int32_t* recent_len, float softmax_scale, const float* out,
                              const float* lse, DecodePlan* plan) {
    const pqkv_status ds = check_dims(dims);
    if (ds != PQKV_OK) return ds;
    if (!dtype_ok(q_dtype) || !dtype_ok(recent_dtype)) return PQKV_ERR_INVALID;
    if (batch < 0 || max_hist_len < 0 || r_cap < 0 || t_cap < 0) return PQKV_ERR_INVALID;
    if (max_hist_len > 0 && (t_cap % kTileTokens || max_hist_len > t_cap)) return PQKV_ERR_INVALID;
    if (r_cap > PQKV_MAX_RECENT) return PQKV_ERR_UNSUPPORTED;
    // the table is read four centroids at a time
    if (lut && dims->n_centroids % 4) return PQKV_ERR_UNSUPPORTED;
    if (batch == 0) return PQKV_OK;
    // q and the table are read with 8- or 16-byte loads, codebook and recent rows with
    // 16-byte loads (some straight into LDS)
    if (!q || !out || !lse || !aligned(q, 16)) return PQKV_ERR_INVALID;
    if (max_hist_len > 0) {
        if ((!lut && !codebook_k) || !codebook_v || !codes_k || !codes_v || !hist_len) return PQKV_ERR_INVALID;
        if (!aligned(codes_k, 16) || !aligned(codes_v, 16) || !aligned(codebook_v, 16)) return PQKV_ERR_INVALID;
        if ((codebook_k && !aligned(codebook_k, 16)) || (lut && !aligned(lut, 16))) return PQKV_ERR_INVALID;
    }
    if (r_cap > 0) {
        if (!recent_k || !recent_v || !recent_len) return PQKV_ERR_INVALID;
        if (!aligned(recent_k, 16) || !aligned(recent_v, 16)) return PQKV_ERR_INVALID;
    }
    if (!(softmax_scale == softmax_scale)) return PQKV_ERR_INVALID;  // NaN
    if ((int64_t)batch * dims->n_q_heads > 0x7fffffffLL) return PQKV_ERR_UNSUPPORTED;
    *plan = plan_decode(*dims, batch, max_hist_len);
    if (plan->n_split > kMaxSplits || plan->units * plan->n_split > 0x7fffffffLL - 8) return PQKV_ERR_UNSUPPORTED;
    return PQKV_OK;
}

// Kernel arguments of a checked call.
DecodeArgs decode_args(const void* q, const float* lut, const float* codebook_k, const float* codebook_v,
                       const uint8_t* codes_k, const uint8_t* codes_v, int64_t t_cap, const int32_t* hist_len,
                       int64_t max_hist_len, const void* recent_k, const void* recent_v, int64_t r_cap,
                       const int32_t* recent_len, float softmax_scale, float* out, float* lse,
                       uint32_t* counters, float* partials) {
    DecodeArgs a;
    a.q = q;
    a.lut = max_hist_len > 0 ? lut : nullptr;
    a.cb_k = a.lut ? nullptr : codebook_k;
    a.cb_v = codebook_v;
    a.codes_k = codes_k;
    a.codes_v = codes_v;
    a.t_cap = t_cap;
    a.hist_len = max_hist_len > 0 ? hist_len : nullptr;  // no history: the kernel takes 0
    a.max_hist = max_hist_len;
    a.rk = r_cap > 0 ? recent_k : nullptr;
    a.rv = r_cap > 0 ? recent_v : nullptr;
    a.r_cap = r_cap;
    a.recent_len = r_cap > 0 ? recent_len : nullptr;
    a.scale_log2 = softmax_scale * 1.4426950408889634f;
    a.out = out;
    a.lse = lse;
    a.counters = counters;
    a.partials = partials;
    return a;
}

Fp16Plan plan_fp16_decode(int head_dim, int n_q_heads, int n_kv_heads, int32_t batch, int64_t max_len) {
    // About two work-groups per CU (each holds 16 KiB of loads in flight per wave),
    // splits of a multiple of 128 tokens (a round of the 4 waves at d = 128), at most 64.
    Fp16Plan p{};
    const int64_t units = (int64_t)batch * n_kv_heads;
    const int64_t want = units > 0 ? (2 * kPlanCUs + units - 1) / units : 1;
    int64_t ns = want < 1 ? 1 : (want > 64 ? 64 : want);
    if (max_len <= 0) {
        ns = 1;
        p.split_tokens = 128;
    } else {
        const int64_t most = (max_len + 511) / 512;  // splits of at least 512 tokens
        ns = ns > most ? most : ns;
        p.split_tokens = ((max_len + ns - 1) / ns + 127) / 128 * 128;
        ns = (max_len + p.split_tokens - 1) / p.split_tokens;
    }
    p.n_split = (int)ns;
    p.partial_stride = head_dim + 4;
    p.partials_offset = decode_counter_bytes(batch, n_q_heads);
    const size_t part = (size_t)batch * n_q_heads * p.n_split * p.partial_stride * sizeof(float);
    p.workspace_bytes = p.partials_offset + (part + 255) / 256 * 256;
    return p;
}

namespace {

pqkv_status check_fp16_dims(const pqkv_dims* d) {
    if (!d || d->n_q_heads < 1 || d->n_kv_heads < 1 || d->head_dim < 1) return PQKV_ERR_INVALID;
    if (d->n_q_heads % d->n_kv_heads) return PQKV_ERR_INVALID;
    const int g = d->n_q_heads / d->n_kv_heads;
    if ((d->head_dim != 64 && d->head_dim != 128) || (g != 1 && g != 2 && g != 4 && g != 8)) return PQKV_ERR_UNSUPPORTED;
    if (d->n_kv_heads > 65535) return PQKV_ERR_UNSUPPORTED;
    return PQKV_OK;
}

}  // namespace

}  // namespace pqkv

using namespace pqkv;

extern "C" {

const char* pqkv_status_str(pqkv_status s) {
    switch (s) {
        case PQKV_OK: return "ok";
        case PQKV_ERR_INVALID: return "invalid argument";
        case PQKV_ERR_UNSUPPORTED: return "unsupported shape";
        case PQKV_ERR_WORKSPACE: return "workspace missing or too small";
        case PQKV_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

pqkv_status pqkv_encode(const pqkv_dims* dims, const void* x, pqkv_dtype x_dtype, int32_t n_seqs,
                        int64_t n_tokens, int64_t x_seq_stride, int64_t x_tok_stride,
                        int64_t x_head_stride, const float* codebook, uint8_t* codes, int64_t t_cap,
                        int64_t t_start, hipStream_t stream) {
    const pqkv_status ds = check_dims(dims);
    if (ds != PQKV_OK) return ds;
    if (!dtype_ok(x_dtype)) return PQKV_ERR_INVALID;
    if (n_seqs < 0 || n_tokens < 0 || t_start < 0 || t_cap <= 0 || t_cap % kTileTokens) return PQKV_ERR_INVALID;
    if (x_seq_stride < 0 || x_tok_stride < 0 || x_head_stride < 0) return PQKV_ERR_INVALID;
    if (t_start + n_tokens > t_cap) return PQKV_ERR_INVALID;
    if (n_seqs > 65535) return PQKV_ERR_UNSUPPORTED;
    if (n_seqs == 0 || n_tokens == 0) return PQKV_OK;
    if (!x || !codebook || !codes) return PQKV_ERR_INVALID;
    // every row is read with 16-byte loads
    const int64_t row_align = 16 / (int64_t)dtype_bytes(x_dtype);
    if (!aligned(x, 16) || x_seq_stride % row_align || x_tok_stride % row_align || x_head_stride % row_align)
        return PQKV_ERR_INVALID;
    if (!aligned(codebook, 16)) return PQKV_ERR_INVALID;
    if ((n_tokens + 2047) / 2048 > 0x7fffffffLL) return PQKV_ERR_UNSUPPORTED;  // grid x: blocks of >= 2048 tokens
    return hip_status(launch_encode(*dims, x, x_dtype, n_seqs, n_tokens, x_seq_stride, x_tok_stride,
                                    x_head_stride, codebook, codes, t_cap, t_start, stream));
}

pqkv_status pqkv_build_lut(const pqkv_dims* dims, int32_t batch, const void* q, pqkv_dtype q_dtype,
                           const float* codebook_k, float* lut, hipStream_t stream) {
    const pqkv_status ds = check_dims(dims);
    if (ds != PQKV_OK) return ds;
    if (!dtype_ok(q_dtype) || batch < 0) return PQKV_ERR_INVALID;
    if (batch == 0) return PQKV_OK;
    if (!q || !codebook_k || !lut) return PQKV_ERR_INVALID;
    if ((int64_t)batch * dims->n_q_heads > 0x7fffffffLL) return PQKV_ERR_UNSUPPORTED;
    return hip_status(launch_build_lut(*dims, batch, q, q_dtype, codebook_k, lut, stream));
}

size_t pqkv_decode_workspace_bytes(const pqkv_dims* dims, int32_t batch, int64_t max_hist_len) {
    if (check_dims(dims) != PQKV_OK || batch <= 0 || max_hist_len < 0) return 0;
    return plan_decode(*dims, batch, max_hist_len).workspace_bytes;
}

pqkv_status pqkv_decode_plan(const pqkv_dims* dims, int32_t batch, int64_t max_hist_len,
                             pqkv_decode_plan_info* info) {
    if (!dims || !info || batch <= 0 || max_hist_len < 0) return PQKV_ERR_INVALID;
    const pqkv_status ds = check_dims(dims);
    if (ds != PQKV_OK) return ds;
    if ((int64_t)batch * dims->n_q_heads > 0x7fffffffLL) return PQKV_ERR_UNSUPPORTED;
    const DecodePlan p = plan_decode(*dims, batch, max_hist_len);
    if (p.n_split > kMaxSplits || p.units * p.n_split > 0x7fffffffLL - 8) return PQKV_ERR_UNSUPPORTED;
    const int M = dims->head_dim / dims->d_sub;
    info->q_heads_per_group = p.qh;
    info->splits = p.n_split;
    info->split_tokens = p.split_tokens;
    info->rounds = p.rounds;
    info->build_rounds = decode_kernel_rounds(M, p.qh, p.rounds);
    info->work_groups = p.units * p.n_split;
    info->device_plan = batch >= 2 && batch <= kDevicePlanMaxBatch && max_hist_len > 0 ? 1 : 0;
    info->workspace_bytes = p.workspace_bytes;
    return PQKV_OK;
}

pqkv_status pqkv_decode_attention(const pqkv_dims* dims, int32_t batch, const void* q,
                                  pqkv_dtype q_dtype, const float* lut, const float* codebook_k,
                                  const float* codebook_v, const uint8_t* codes_k,
                                  const uint8_t* codes_v, int64_t t_cap, const int32_t* hist_len,
                                  int64_t max_hist_len, const void* recent_k, const void* recent_v,
                                  pqkv_dtype recent_dtype, int64_t r_cap,
                                  const int32_t* recent_len, float softmax_scale, float* out,
                                  float* lse, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
    DecodePlan plan{};
    const pqkv_status st =
        check_decode_args(dims, batch, q, q_dtype, lut, codebook_k, codebook_v, codes_k, codes_v, t_cap, hist_len,
                          max_hist_len, recent_k, recent_v, recent_dtype, r_cap, recent_len, softmax_scale, out,
                          lse, &plan);
    if (st != PQKV_OK || batch == 0) return st;
    if (!workspace || workspace_bytes < plan.workspace_bytes || !aligned(workspace, 256)) return PQKV_ERR_WORKSPACE;
    // the workspace holds the counters at byte 0 and the partials after them
    const DecodeArgs a = decode_args(q, lut, codebook_k, codebook_v, codes_k, codes_v, t_cap, hist_len,
                                     max_hist_len, recent_k, recent_v, r_cap, recent_len, softmax_scale, out, lse,
                                     static_cast<uint32_t*>(workspace),
                                     reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.partials_offset));
    return hip_status(launch_decode(*dims, batch, q_dtype, recent_dtype, plan, a, stream));
}

size_t pqkv_fp16_decode_workspace_bytes(const pqkv_dims* dims, int32_t batch, int64_t max_len) {
    if (check_fp16_dims(dims) != PQKV_OK || batch <= 0 || max_len < 0) return 0;
    return plan_fp16_decode(dims->head_dim, dims->n_q_heads, dims->n_kv_heads, batch, max_len).workspace_bytes;
}

pqkv_status pqkv_fp16_decode_attention(const pqkv_dims* dims, int32_t batch, const void* q, const void* k_cache,
                                       const void* v_cache, int64_t t_cap, const int32_t* seq_len, int64_t max_len,
                                       float softmax_scale, float* out, float* lse, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
    const pqkv_status ds = check_fp16_dims(dims);
    if (ds != PQKV_OK) return ds;
    if (batch < 0 || max_len < 0 || t_cap < 0 || max_len > t_cap) return PQKV_ERR_INVALID;
    if (batch == 0) return PQKV_OK;
    if (!q || !k_cache || !v_cache || !seq_len || !out || !lse) return PQKV_ERR_INVALID;
    // rows are read 16 bytes per lane
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16)) return PQKV_ERR_INVALID;
    if (!(softmax_scale == softmax_scale)) return PQKV_ERR_INVALID;
    if ((int64_t)batch * dims->n_kv_heads * 64 > 0x7fffffffLL) return PQKV_ERR_UNSUPPORTED;
    const Fp16Plan plan = plan_fp16_decode(dims->head_dim, dims->n_q_heads, dims->n_kv_heads, batch, max_len);
    if (!workspace || workspace_bytes < plan.workspace_bytes || !aligned(workspace, 256)) return PQKV_ERR_WORKSPACE;
    Fp16Call c;
    c.head_dim = dims->head_dim;
    c.n_q_heads = dims->n_q_heads;
    c.n_kv_heads = dims->n_kv_heads;
    c.q = q;
    c.k = k_cache;
    c.v = v_cache;
    c.t_cap = t_cap;
    c.seq_len = seq_len;
    c.max_len = max_len;
    c.scale = softmax_scale;
    c.out = out;
    c.lse = lse;
    c.counters = static_cast<uint32_t*>(workspace);
    c.partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.partials_offset);
    return hip_status(launch_fp16_decode(plan, batch, c, stream));
}

pqkv_status pqkv_merge(int64_t n_rows, int32_t head_dim, const float* out_a, const float* lse_a,
                       const float* out_b, const float* lse_b, float* out, float* lse,
                       hipStream_t stream) {
    if (n_rows < 0 || head_dim < 1) return PQKV_ERR_INVALID;
    if (head_dim > 1024) return PQKV_ERR_UNSUPPORTED;
    if (n_rows == 0) return PQKV_OK;
    if (!out_a || !lse_a || !out_b || !lse_b || !out || !lse) return PQKV_ERR_INVALID;
    if ((n_rows + 3) / 4 > 0x7fffffffLL) return PQKV_ERR_UNSUPPORTED;
    return hip_status(launch_merge_states(n_rows, head_dim, out_a, lse_a, out_b, lse_b, out, lse, stream));
}

pqkv_status pqkv_append_kv(const pqkv_dims* dims, int32_t batch, const void* new_k, const void* new_v,
                           void* recent_k, void* recent_v, pqkv_dtype recent_dtype, int64_t r_cap,
                           const int32_t* hist_len_in, const int32_t* recent_len_in, int32_t* hist_len_out,
                           int32_t* recent_len_out, int32_t n_roll, const float* codebook_k,
                           const float* codebook_v, uint8_t* codes_k, uint8_t* codes_v, int64_t t_cap,
                           int64_t max_hist_len, hipStream_t stream) {
    const pqkv_status ds = check_dims(dims);
    if (ds != PQKV_OK) return ds;
    if (!dtype_ok(recent_dtype)) return PQKV_ERR_INVALID;
    if (batch < 0 || r_cap < 1 || n_roll < 1 || n_roll > r_cap || max_hist_len < 0) return PQKV_ERR_INVALID;
    if (t_cap <= 0 || t_cap % kTileTokens || max_hist_len + n_roll > t_cap) return PQKV_ERR_INVALID;
    if (r_cap > PQKV_MAX_RECENT || n_roll > 512 || batch > 32767) return PQKV_ERR_UNSUPPORTED;
    if (batch == 0) return PQKV_OK;
    if (!new_k || !new_v || !recent_k || !recent_v || !hist_len_in || !recent_len_in || !hist_len_out ||
        !recent_len_out || !codebook_k || !codebook_v || !codes_k || !codes_v)
        return PQKV_ERR_INVALID;
    // rows move with 16-byte loads and stores
    if (!aligned(new_k, 16) || !aligned(new_v, 16) || !aligned(recent_k, 16) || !aligned(recent_v, 16) ||
        !aligned(codebook_k, 16) || !aligned(codebook_v, 16))
        return PQKV_ERR_INVALID;
    // every work-group reads the old lengths while one per sequence writes the new ones
    const size_t lb = (size_t)batch * sizeof(int32_t);
    const void* ins[2] = {hist_len_in, recent_len_in};
    const void* outs[2] = {hist_len_out, recent_len_out};
    for (const void* o : outs)
        for (const void* i : ins)
            if (overlap(o, i, lb)) return PQKV_ERR_INVALID;
    if (overlap(hist_len_out, recent_len_out, lb)) return PQKV_ERR_INVALID;
    return hip_status(launch_append(*dims, batch, new_k, new_v, recent_k, recent_v, recent_dtype, r_cap,
                                    hist_len_in, recent_len_in, hist_len_out, recent_len_out, n_roll,
                                    codebook_k, codebook_v, codes_k, codes_v, t_cap, stream));
}

pqkv_status pqkv_fit_codebooks(const pqkv_dims* dims, const void* x, pqkv_dtype x_dtype, int64_t n_points,
                               int64_t x_tok_stride, int64_t x_head_stride, const int32_t* order,
                               int32_t iters, float* codebook, int32_t* kept, hipStream_t stream) {
    const pqkv_status ds = check_dims(dims);
    if (ds != PQKV_OK) return ds;
    if (!dtype_ok(x_dtype) || n_points < 1 || iters < 0 || x_tok_stride < 0 || x_head_stride < 0)
        return PQKV_ERR_INVALID;
    if (n_points > PQKV_MAX_FIT_POINTS || iters > 100000) return PQKV_ERR_UNSUPPORTED;
    if (!x || !order || !codebook) return PQKV_ERR_INVALID;
    return hip_status(launch_kmeans(*dims, x, x_dtype, n_points, x_tok_stride, x_head_stride, order, iters,
                                    codebook, kept, stream));
}

}  // extern "C"
