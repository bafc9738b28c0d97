/*
 * libpqkv -- product-quantised KV cache: encode and decode attention on MI355X (gfx950).
 *
 * The method is MILLION (DAC 2025), as described in its write-up ("MILLION:
 * product-quantisation based KV-cache compression and decode acceleration"):
 * every key/value head vector is split into subspaces of dimension 2 or 4
 * (the paragraph after Fig. 5), each subspace is replaced by the uint8 index of
 * its nearest codebook centroid when the prefill cache is written (Fig. 6
 * paragraph), and decode attention scores the compressed history through an
 * asymmetric-distance lookup table of query x codebook, computed apart from the
 * attention over recent full-precision tokens and merged with it (Fig. 7
 * paragraph), on a split-over-tokens flash-decoding base (Fig. 8 paragraph).
 *
 * Conventions shared by every entry point
 *   - Every data pointer is a DEVICE pointer owned by the caller.  The library
 *     allocates nothing and keeps no pointer after the enqueued work finishes.
 *   - Work is enqueued asynchronously on `stream` (NULL = the null stream); no
 *     entry point synchronises the host.
 *   - Arguments are validated on the host before anything is enqueued.  A
 *     violation returns PQKV_ERR_INVALID / PQKV_ERR_UNSUPPORTED /
 *     PQKV_ERR_WORKSPACE and enqueues nothing.  A failed launch returns
 *     PQKV_ERR_HIP.  A device-side fault shows up at the caller's next
 *     synchronisation.  No C++ exception crosses this interface.
 *   - The library keeps no mutable global state and its calls are thread-safe,
 *     except pqkv_decode_attention_noalloc (a static device array per GPU).
 *
 * Shapes and symbols
 *   d = head_dim in {64, 128};  d_sub in {2, 4};  M = d / d_sub subspaces;
 *   K = n_centroids in [2, 256];  Hq query heads, Hkv kv heads, Hq % Hkv == 0;
 *   query head hq reads kv head hq / (Hq / Hkv).
 *
 * Codebook layout (fp32, one per (layer, kv head, tensor K or V)):
 *   codebook[h][c][m][j]  = [Hkv][K][M][d_sub]   (centroid-major, subspace-minor)
 *   Centroid c of subspace m of head h is the d_sub floats at ((h*K + c)*M + m)*d_sub.
 *
 * Code-cache layout (uint8, one byte per (token, subspace)):
 *   codes[b][h] is a plane of t_cap*M bytes (t_cap a multiple of 64); planes are
 *   dense: plane (b, h) starts at byte (b*Hkv + h) * t_cap * M.
 *   Inside a plane, token t and subspace m sit at byte
 *       tile  = t / 64,  l = t % 64,  p = (m - l) mod M,
 *       off   = tile*64*M + (p / 16)*1024 + l*16 + (p % 16).
 *   So a tile of 64 tokens is 64*M contiguous bytes; the 16-byte chunk i of the
 *   64 tokens of a tile is one contiguous 1 KiB run (one token per 16 bytes),
 *   and byte p of token slot l holds subspace (p + l) mod M.  Reading a tile
 *   with one 16-byte load per lane is fully coalesced, and lanes that consume
 *   byte p at the same time touch 64 different subspaces, which keeps the
 *   on-chip table accesses free of bank conflicts.
 */
#ifndef PQKV_H
#define PQKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PQKV_OK = 0,
    PQKV_ERR_INVALID = 1,     /* a bad argument: null pointer, negative size, bad stride, bad enum */
    PQKV_ERR_UNSUPPORTED = 2, /* a valid but unsupported shape (head_dim, d_sub, K, r_cap ...) */
    PQKV_ERR_WORKSPACE = 3,   /* workspace missing or smaller than pqkv_decode_workspace_bytes */
    PQKV_ERR_HIP = 4          /* the HIP runtime refused a launch */
} pqkv_status;

typedef enum { PQKV_F16 = 0, PQKV_F32 = 1 } pqkv_dtype;

typedef struct {
    int32_t head_dim;    /* d: 64 or 128 */
    int32_t d_sub;       /* subspace dimension: 2 or 4 */
    int32_t n_centroids; /* K: 2..256 */
    int32_t n_q_heads;   /* Hq >= 1 */
    int32_t n_kv_heads;  /* Hkv >= 1, divides Hq */
} pqkv_dims;

/* Largest recent window (r_cap) pqkv_decode_attention accepts. */
#define PQKV_MAX_RECENT 1024

/* Most calibration points per (kv head, subspace) pqkv_fit_codebooks takes. */
#define PQKV_MAX_FIT_POINTS 8192

/*
 * pqkv_encode -- nearest-centroid codes for a block of tokens (the online
 * prefill quantisation of the Fig. 6 paragraph; the subspace split of the
 * paragraph after Fig. 5).
 *
 * For every sequence b < n_seqs, token i < n_tokens, kv head h and subspace m:
 *     code = argmin_c sum_j (x[b][i][h][m*d_sub + j] - codebook[h][c][m][j])^2,
 * lowest c on exact ties, distances evaluated in fp32 as the sum of squared
 * differences (no expanded |x|^2 - 2x.c + |c|^2 form).  The code is written to
 * token position t_start + i of plane (b, h) of `codes`.
 *
 *   x            device, x_dtype (F16 or F32); element (b, i, h, e) at
 *                x + b*x_seq_stride + i*x_tok_stride + h*x_head_stride + e (in elements);
 *                strides >= 0, rows of d contiguous elements.
 *   codebook     device fp32 [Hkv][K][M][d_sub] (layout above).
 *   codes        device uint8, n_seqs consecutive sequences of Hkv planes of t_cap*M bytes.
 *   t_cap        plane capacity in tokens, multiple of 64, t_start + n_tokens <= t_cap.
 *   n_seqs, n_tokens may be 0 (nothing is enqueued).
 * Only the bytes of the encoded tokens are written.  Errors: INVALID for null
 * pointers with work to do, negative sizes, t_start + n_tokens > t_cap, t_cap
 * not a multiple of 64, bad dtype; UNSUPPORTED for dims outside the ranges above.
 */
pqkv_status pqkv_encode(const pqkv_dims* dims, const void* x, pqkv_dtype x_dtype, int32_t n_seqs,
                        int64_t n_tokens, int64_t x_seq_stride, int64_t x_tok_stride,
                        int64_t x_head_stride, const float* codebook, uint8_t* codes, int64_t t_cap,
                        int64_t t_start, hipStream_t stream);

/*
 * pqkv_build_lut -- the asymmetric-distance lookup table of the Fig. 7
 * paragraph, materialised:
 *     lut[b][hq][m][c] = sum_j q[b][hq][m*d_sub + j] * codebook_k[hq / g][c][m][j]
 * in fp32, unscaled (no softmax scale).
 *   q           device [batch][Hq][d] in q_dtype (F16 or F32), dense.
 *   codebook_k  device fp32 [Hkv][K][M][d_sub].
 *   lut         device fp32 [batch][Hq][M][K], dense, written whole.
 * pqkv_decode_attention takes this table through its `lut` argument; given NULL
 * there, it builds the same table itself in on-chip memory.  Errors as for
 * pqkv_encode.
 */
pqkv_status pqkv_build_lut(const pqkv_dims* dims, int32_t batch, const void* q, pqkv_dtype q_dtype,
                           const float* codebook_k, float* lut, hipStream_t stream);

/*
 * Workspace bytes pqkv_decode_attention needs for these sizes.  Depends only on
 * its arguments.  Returns 0 for invalid dims, batch <= 0 or max_hist_len < 0.
 */
size_t pqkv_decode_workspace_bytes(const pqkv_dims* dims, int32_t batch, int64_t max_hist_len);

/*
 * The preset pqkv_decode_attention runs for these sizes: the kernel parameters that the
 * Fig. 8 paragraph tunes per context length, here chosen at run time by a cost model over
 * the split length and the kernel builds.  Host only: it reads no device memory and
 * enqueues nothing.  For 2..16 sequences with a history the kernel re-plans the splits on
 * the device from the actual lengths when they differ (device_plan = 1); the figures below
 * are then the launched grid, which bounds that plan.
 */
typedef struct {
    int32_t q_heads_per_group; /* query heads of one kv head per work-group: 1, 2 or 4 */
    int32_t splits;            /* history splits per (sequence, kv head, head group); 1 without history */
    int64_t split_tokens;      /* tokens per split, a multiple of 512; 0 without history */
    int32_t rounds;            /* 512-token rounds per split: tiles per wave */
    int32_t build_rounds;      /* tiles per wave of the kernel build that runs them */
    int64_t work_groups;       /* work-groups launched, one per CU at a time */
    int32_t device_plan;       /* 1: the kernel reads the lengths first and re-plans the splits
                                  on the device when they differ */
    size_t workspace_bytes;    /* pqkv_decode_workspace_bytes of the same sizes */
} pqkv_decode_plan_info;

/* Errors: INVALID for a null pointer, batch <= 0 or max_hist_len < 0; UNSUPPORTED for
 * dims outside the ranges above or a history beyond what the merge's 512 splits cover. */
pqkv_status pqkv_decode_plan(const pqkv_dims* dims, int32_t batch, int64_t max_hist_len,
                             pqkv_decode_plan_info* info);

/*
 * pqkv_decode_attention -- one decode step of attention for `batch` sequences
 * over a PQ-compressed history plus a recent full-precision window (Fig. 7
 * paragraph: history attention apart from new-token attention, ad-LUT scoring
 * of the history; Fig. 8 paragraph: flash-decoding split over tokens).
 *
 * For query row (b, hq), h = hq / g, the result is ordinary softmax attention of
 * q[b][hq] over the hist_len[b] history tokens of planes (b, h) -- key and value
 * of token t being the centroids its K and V codes select -- followed by the
 * recent_len[b] recent tokens of recent_k/v[b][h]:
 *     s_i  = softmax_scale * q . key_i,
 *     out  = sum_i exp(s_i - mu) value_i / sum_i exp(s_i - mu),   mu = max_i s_i,
 *     lse  = mu + ln sum_i exp(s_i - mu).
 * A row with no tokens gets out = 0 and lse = -inf.
 *
 *   q             device [batch][Hq][d], q_dtype, dense, 16-byte aligned.
 *   lut           NULL: the kernel builds the ad-LUT from q and codebook_k in on-chip
 *                 memory.  Otherwise device fp32 [batch][Hq][M][K], 16-byte aligned: the
 *                 unscaled table pqkv_build_lut writes (entry (b, hq, m, c) = q_m . centroid c
 *                 of subspace m of kv head hq / g), read in place of building it; the
 *                 history scores are then softmax_scale times sums of its entries, and
 *                 codebook_k is not read (it may be NULL).  Needs K % 4 == 0.
 *   codebook_k/v  device fp32 [Hkv][K][M][d_sub], 16-byte aligned.
 *   codes_k/v     device uint8 cache planes (layout above), batch*Hkv planes of t_cap*M
 *                 bytes, 16-byte aligned; only tokens < hist_len[b] are read.
 *   hist_len      device int32 [batch], each in [0, max_hist_len]; may be NULL if
 *                 max_hist_len == 0 (every history is then empty).
 *   max_hist_len  host bound on hist_len, <= t_cap; sizes the split-over-tokens grid.
 *   recent_k/v    device [batch][Hkv][r_cap][d] in recent_dtype, dense, 16-byte aligned;
 *                 may be NULL if r_cap == 0.
 *   recent_len    device int32 [batch], each in [0, r_cap]; may be NULL if r_cap == 0.
 *   r_cap         0..PQKV_MAX_RECENT.
 *   out           device fp32 [batch][Hq][d];  lse device fp32 [batch][Hq] (natural log).
 *   workspace     device, >= pqkv_decode_workspace_bytes(dims, batch, max_hist_len) bytes,
 *                 256-byte aligned.  It starts with completion counters (4 bytes per
 *                 (sequence, query head), rounded up to 256 bytes), followed by per-split
 *                 partial results.  The counters must be zero before the first call that
 *                 uses the workspace (e.g. one hipMemset of the whole buffer); every call
 *                 returns them to zero.  Their size depends only on batch and n_q_heads, so
 *                 one zeroed workspace serves every later call whose batch * n_q_heads is
 *                 at most that of the first, whatever its max_hist_len, as long as it is
 *                 large enough; zero it again before a call with a larger batch * n_q_heads.
 *                 Calls sharing one workspace must be ordered on one stream.
 * The call allocates nothing, records no memset and never waits on the host, so
 * it may be captured in a HIP graph and replayed with new device-side q and
 * lengths (max_hist_len, fixed at capture, must still bound them).
 * Device-side lengths outside their bounds are clamped to them.  Errors: INVALID
 * for null pointers, misaligned pointers, negative sizes, max_hist_len > t_cap, bad
 * dtype; UNSUPPORTED for dims outside the ranges above, r_cap > PQKV_MAX_RECENT, a
 * lut with K % 4 != 0, or a max_hist_len that needs more than 512 splits per (sequence,
 * kv head, query-head group): above 4,194,304 tokens, or 2,097,152 where four query
 * heads share a work-group (n_q_heads / n_kv_heads a multiple of 4 with head_dim / d_sub
 * <= 16); WORKSPACE for a missing, short or misaligned workspace.
 */
pqkv_status pqkv_decode_attention(const pqkv_dims* dims, int32_t batch, const void* q,
                                  pqkv_dtype q_dtype, const float* lut, const float* codebook_k,
                                  const float* codebook_v, const uint8_t* codes_k,
                                  const uint8_t* codes_v, int64_t t_cap, const int32_t* hist_len,
                                  int64_t max_hist_len, const void* recent_k, const void* recent_v,
                                  pqkv_dtype recent_dtype, int64_t r_cap,
                                  const int32_t* recent_len, float softmax_scale, float* out,
                                  float* lse, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/*
 * pqkv_decode_attention_noalloc -- pqkv_decode_attention for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, same kernels and the same
 * result, without the workspace: the per-split partials and completion counters
 * live in a static device array of PQKV_NOALLOC_SCRATCH_BYTES that the library
 * holds on every GPU it runs on until the process ends.  The first call on a device
 * looks the array up and clears its counters on `stream` (a small kernel); later
 * calls allocate nothing and launch only the decode kernel.
 *
 * Every call on one GPU shares that GPU's array: calls that overlap in time on one
 * GPU (different streams, or host threads) race and give wrong results.  Order them
 * on one stream.  This entry point keeps global state, unlike the rest of the library.
 * Errors as for pqkv_decode_attention, and WORKSPACE when batch * n_q_heads exceeds
 * PQKV_NOALLOC_MAX_ROWS or the partials exceed the array (about 15,000 (sequence,
 * query head, split) records at head_dim 128).
 */
#define PQKV_NOALLOC_SCRATCH_BYTES (8u << 20)
#define PQKV_NOALLOC_MAX_ROWS 16384
pqkv_status pqkv_decode_attention_noalloc(const pqkv_dims* dims, int32_t batch, const void* q,
                                          pqkv_dtype q_dtype, const float* lut, const float* codebook_k,
                                          const float* codebook_v, const uint8_t* codes_k,
                                          const uint8_t* codes_v, int64_t t_cap, const int32_t* hist_len,
                                          int64_t max_hist_len, const void* recent_k, const void* recent_v,
                                          pqkv_dtype recent_dtype, int64_t r_cap,
                                          const int32_t* recent_len, float softmax_scale, float* out,
                                          float* lse, hipStream_t stream);

/*
 * pqkv_fp16_decode_attention -- dense fp16 decode attention over a full-precision
 * K/V cache: the baseline the page compares MILLION's decode speed with (Fig. 12
 * paragraph: time per output token against an FP16 KV cache).  It computes the
 * same softmax attention as pqkv_decode_attention's definition, with every cached
 * token's key and value read from the fp16 cache:
 *     s_i = softmax_scale * q . k_i,  out = sum_i exp(s_i - mu) v_i / sum_i exp(s_i - mu),
 *     lse = mu + ln sum_i exp(s_i - mu),   i < seq_len[b];  no tokens: out = 0, lse = -inf.
 * Split-K over tokens (flash decoding) with fp32 accumulation.
 *
 *   dims          head_dim (64 or 128), n_q_heads, n_kv_heads (Hq / Hkv in {1, 2, 4, 8});
 *                 d_sub and n_centroids are not read.
 *   q             device fp16 [batch][Hq][d], 16-byte aligned.
 *   k_cache/v_cache  device fp16 [batch][Hkv][t_cap][d], 16-byte aligned.
 *   seq_len       device int32 [batch], each in [0, max_len] (clamped to it).
 *   max_len       host bound on seq_len, <= t_cap.
 *   out, lse      device fp32 [batch][Hq][d] and [batch][Hq].
 *   workspace     as for pqkv_decode_attention (counters first, zeroed before first use),
 *                 >= pqkv_fp16_decode_workspace_bytes(dims, batch, max_len) bytes.
 * Errors: INVALID for null or misaligned pointers, negative sizes, max_len > t_cap;
 * UNSUPPORTED for other head sizes or group sizes; WORKSPACE for a short workspace.
 */
size_t pqkv_fp16_decode_workspace_bytes(const pqkv_dims* dims, int32_t batch, int64_t max_len);
pqkv_status pqkv_fp16_decode_attention(const pqkv_dims* dims, int32_t batch, const void* q, const void* k_cache,
                                       const void* v_cache, int64_t t_cap, const int32_t* seq_len, int64_t max_len,
                                       float softmax_scale, float* out, float* lse, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream);

/*
 * pqkv_append_kv -- one decode step of the live cache: each sequence's new key
 * and value enter its recent full-precision window, and a window that is full
 * first rolls its oldest n_roll tokens into the PQ history.  This is the batched,
 * delayed quantisation of the Fig. 7 paragraph: generated tokens are kept in full
 * precision, apart from the quantised history, and quantised later in batches.
 *
 * For every sequence b, with T = hist_len_in[b] and R = recent_len_in[b]:
 *   1. if R == r_cap: for every kv head h, rows 0..n_roll-1 of recent_k/v[b][h] are
 *      encoded exactly as pqkv_encode would (same codes, same tie rule) into history
 *      positions T..T+n_roll-1 of planes (b, h) of codes_k/v; rows n_roll..R-1 move
 *      down to rows 0..R-n_roll-1; T += n_roll; R -= n_roll;
 *   2. new_k/v[b][h] is written to recent row R of every head, and R += 1;
 *   3. hist_len_out[b] = T, recent_len_out[b] = R.
 * So hist_len + recent_len grows by exactly one per call, and the recent window
 * always holds the newest tokens in order.  Rows and code bytes of other
 * positions are left untouched.
 *
 *   new_k/new_v     device [batch][Hkv][d] in recent_dtype, dense, 16-byte aligned.
 *   recent_k/v      device [batch][Hkv][r_cap][d] in recent_dtype, dense, 16-byte aligned;
 *                   updated in place.
 *   r_cap           1..PQKV_MAX_RECENT;  n_roll in 1..min(r_cap, 512).
 *   hist_len_in, recent_len_in    device int32 [batch]: 0 <= hist_len_in[b] <= max_hist_len,
 *                   0 <= recent_len_in[b] <= r_cap.
 *   hist_len_out, recent_len_out  device int32 [batch]; must not overlap each other or the
 *                   _in arrays (every work-group reads the old lengths while one per
 *                   sequence writes the new ones); swap in and out between steps.
 *   codebook_k/v    device fp32 [Hkv][K][M][d_sub], 16-byte aligned.
 *   codes_k/v       device uint8 cache planes (layout above), updated in place.
 *   t_cap           plane capacity in tokens, multiple of 64, max_hist_len + n_roll <= t_cap.
 *   max_hist_len    host bound on hist_len_in (as for pqkv_decode_attention).
 * A sequence whose device lengths break these bounds is left unchanged and its
 * out lengths repeat the in lengths.  Errors: INVALID for null pointers, bad
 * sizes or alignment, overlapping length arrays, bad dtype; UNSUPPORTED for dims
 * outside the ranges above, r_cap > PQKV_MAX_RECENT, n_roll > 512 or batch > 32767.
 */
pqkv_status pqkv_append_kv(const pqkv_dims* dims, int32_t batch, const void* new_k, const void* new_v,
                           void* recent_k, void* recent_v, pqkv_dtype recent_dtype, int64_t r_cap,
                           const int32_t* hist_len_in, const int32_t* recent_len_in, int32_t* hist_len_out,
                           int32_t* recent_len_out, int32_t n_roll, const float* codebook_k,
                           const float* codebook_v, uint8_t* codes_k, uint8_t* codes_v, int64_t t_cap,
                           int64_t max_hist_len, hipStream_t stream);

/*
 * pqkv_fit_codebooks -- offline codebook training: Lloyd k-means of every
 * (kv head, subspace) codebook of one tensor on calibration vectors (the Fig. 5
 * paragraph clusters with k-means; the paragraph after it trains one codebook
 * per subspace of dimension d_sub; the Fig. 6 paragraph does it offline).
 *
 * For every kv head h and subspace m, with the n_points subvectors
 *     p_i = x[i][h][m*d_sub .. m*d_sub + d_sub - 1]:
 *   1. initialisation: walk order[h][m][0..n_points-1] and keep each p_order[i] that is not
 *      equal (all d_sub values) to one already kept, until K are kept; entries outside
 *      [0, n_points) are skipped; if fewer than K distinct points exist, the remaining
 *      centroids copy centroid 0;
 *   2. `iters` Lloyd iterations: every point takes its nearest centroid by squared distance
 *      (lowest index on exact ties), then every centroid with members moves to their mean;
 *      an empty cluster keeps its centroid.
 * All arithmetic is fp64 with every product, sum and quotient rounded on its own and member
 * sums taken in point order, so the result is the exact IEEE evaluation of this definition
 * (independent of the launch shape).  The fp64 centroids are rounded to fp32 at the end.
 *
 *   x            device, x_dtype (F16 or F32); element (i, h, e) at
 *                x + i*x_tok_stride + h*x_head_stride + e (in elements), strides >= 0.
 *   n_points     1..PQKV_MAX_FIT_POINTS.
 *   order        device int32 [Hkv][M][n_points] (a permutation per problem: the random draw
 *                of the initialisation, supplied by the caller).
 *   iters        >= 0.
 *   codebook     device fp32 out [Hkv][K][M][d_sub] (layout above), written whole.
 *   kept         device int32 out [Hkv][M]: distinct points kept by the initialisation; may be NULL.
 * Errors: INVALID for null pointers, n_points < 1, iters < 0, negative strides, bad dtype;
 * UNSUPPORTED for dims outside the ranges above or n_points > PQKV_MAX_FIT_POINTS.
 */
pqkv_status pqkv_fit_codebooks(const pqkv_dims* dims, const void* x, pqkv_dtype x_dtype, int64_t n_points,
                               int64_t x_tok_stride, int64_t x_head_stride, const int32_t* order,
                               int32_t iters, float* codebook, int32_t* kept, hipStream_t stream);

/*
 * pqkv_merge -- log-sum-exp merge of two normalised attention states over
 * disjoint token sets (the combination step of the Fig. 7 paragraph):
 *     mu = max(lse_a, lse_b),  wa = exp(lse_a - mu),  wb = exp(lse_b - mu),
 *     out = (wa*out_a + wb*out_b) / (wa + wb),  lse = mu + ln(wa + wb),
 * row by row; a side with lse = -inf has weight 0; two such sides give out = 0,
 * lse = -inf.
 *   out_a/out_b/out  device fp32 [n_rows][head_dim];  lse_a/lse_b/lse device fp32 [n_rows].
 *   out may alias out_a or out_b and lse may alias lse_a or lse_b (element-wise in place).
 *   head_dim in 1..1024.
 */
pqkv_status pqkv_merge(int64_t n_rows, int32_t head_dim, const float* out_a, const float* lse_a,
                       const float* out_b, const float* lse_b, float* out, float* lse,
                       hipStream_t stream);

/* Static description of a status code. */
const char* pqkv_status_str(pqkv_status status);

#ifdef __cplusplus
}
#endif

#endif /* PQKV_H */
