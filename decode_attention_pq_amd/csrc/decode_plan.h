// The decode path's constants, split plan and kernel arguments (host side).
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime.h>

#include "../../include/pqkv.h"

namespace pqkv {

constexpr int kTileTokens = 64;      // tokens per code tile (one per lane)
constexpr int kDecodeThreads = 512;  // decode work-group: 8 wave64s
constexpr int kDecodeWaves = kDecodeThreads / 64;
constexpr int kTokensPerRound = kDecodeWaves * kTileTokens;  // one tile per wave per round
constexpr int kPlanCUs = 256;         // MI355X compute units the split plan fills
constexpr int kLdsRows = 256;         // LDS table rows (any uint8 code stays in bounds)

// Tiles per wave in one decode split: each tile's scores stay in registers until
// the split's softmax max is known, and the fully unrolled tile loop fits the
// register budget.
constexpr int decode_max_rounds(int n_sub, int qh) { return qh == 4 ? 8 : 16; }
// Tiles per wave of the kernel build that runs a split of `rounds` tiles per wave:
// the smallest build that holds them.  Steps past the plan's rounds still issue
// their (dummy) loads, so the 64-subspace kernel comes in 2-, 4-, 8-, 12- and
// 16-round builds, and the narrower ones in a 4-round build beside the longest.
constexpr int decode_kernel_rounds(int n_sub, int qh, int rounds) {
    return n_sub == 64 ? (rounds <= 2 ? 2 : rounds <= 4 ? 4 : rounds <= 8 ? 8 : rounds <= 12 ? 12 : 16)
                       : (rounds <= 4 ? 4 : decode_max_rounds(n_sub, qh));
}
// Work-group id -> work item of a grid of n items: ids that share an XCD (id mod 8,
// the order in which the hardware deals work-groups out to the 8 XCDs) take contiguous
// items, XCD x holding ceil((n - x) / 8) of them, so the splits of one kv head meet in
// one L2.  Ids below n map one to one onto [0, n).
constexpr int xcd_item(int id, int n) {
    const int x = id & 7;
    return x * (n >> 3) + (x < (n & 7) ? x : (n & 7)) + (id >> 3);
}
// Whether work-group `id` has an item when only the first `used` of the grid's items
// exist (the device-side plan may need fewer than the host launched).
constexpr bool xcd_has_item(int id, int used) { return (id >> 3) < (used - (id & 7) + 7) / 8; }

// Splits per unit the merge can take (its split maxima and sums live in LDS).
constexpr int kMaxSplits = 512;

// The split plan's cost model, in units of about a twentieth of a round of streaming:
// a work-group's fixed costs (codebooks, LUT, epilogue, merge), one round of its split,
// one unused step of its kernel build.  The host plan and the device-side plan of
// ragged batches price candidates with the same constants.
constexpr int kPlanFixed = 48;
constexpr int kPlanRound = 20;
constexpr int kPlanUnused = 3;
// Batches of 2 to this many sequences plan their splits on the device, from the
// actual lengths: every work-group reads them all and prices each round count.
constexpr int kDevicePlanMaxBatch = 16;

// How a decode call is cut into work-groups.
struct DecodePlan {
    int qh;              // query heads per work-group (share one kv head)
    int n_groups;        // query-head groups per kv head (= g / qh)
    int rounds;          // tiles per wave (tokens per split = rounds * 512)
    int n_split;         // splits over the history per (sequence, kv head, group)
    int64_t split_tokens;
    int partial_stride;  // floats per partial record: d outputs + max + sum, padded
    int64_t units;       // (sequence, kv head, group) units, one completion counter each
    size_t partials_offset;  // byte offset of the partials (the counters sit at byte 0)
    size_t workspace_bytes;
};

DecodePlan plan_decode(const pqkv_dims& d, int32_t batch, int64_t max_hist_len);

// Completion counters at the start of a workspace: one u32 slot per (sequence,
// query head), which bounds the units of every plan, rounded up to 256 bytes.  The
// offset of the partials after them depends only on batch and n_q_heads, so a
// workspace zeroed once serves every later call whatever its max_hist_len.
inline size_t decode_counter_bytes(int32_t batch, int32_t n_q_heads) {
    return ((size_t)batch * (size_t)n_q_heads * sizeof(uint32_t) + 255) / 256 * 256;
}

struct DecodeArgs {
    const void* q;
    const float* lut;  // nullable: the materialised table [B][Hq][M][K], unscaled
    const float* cb_k;
    const float* cb_v;
    const uint8_t* codes_k;
    const uint8_t* codes_v;
    int64_t t_cap;
    const int32_t* hist_len;
    int64_t max_hist;
    const void* rk;
    const void* rv;
    int64_t r_cap;
    const int32_t* recent_len;
    float scale_log2;  // softmax scale * log2(e)
    float* out;
    float* lse;
    float* partials;
    uint32_t* counters;
};

hipError_t launch_decode(const pqkv_dims& d, int32_t batch, pqkv_dtype qt, pqkv_dtype rt,
                         const DecodePlan& plan, const DecodeArgs& a, hipStream_t stream);

// Host-side validation shared by the decode entry points: the status the call
// returns before any launch (PQKV_OK if it may go ahead), with the plan filled in.
pqkv_status check_decode_args(const pqkv_dims* dims, int32_t batch, const void* q, pqkv_dtype q_dtype,
                              const float* lut, const float* codebook_k, const float* codebook_v,
                              const uint8_t* codes_k, const uint8_t* codes_v, int64_t t_cap,
                              const int32_t* hist_len, int64_t max_hist_len, const void* recent_k,
                              const void* recent_v, pqkv_dtype recent_dtype, int64_t r_cap,
                              const int32_t* recent_len, float softmax_scale, const float* out,
                              const float* lse, DecodePlan* plan);

// Kernel arguments of a call that check_decode_args accepted: the completion counters
// (one u32 per (sequence, query head), zero between calls) and the partials.
DecodeArgs decode_args(const void* q, const float* lut, const float* codebook_k, const float* codebook_v,
                       const uint8_t* codes_k, const uint8_t* codes_v, int64_t t_cap, const int32_t* hist_len,
                       int64_t max_hist_len, const void* recent_k, const void* recent_v, int64_t r_cap,
                       const int32_t* recent_len, float softmax_scale, float* out, float* lse,
                       uint32_t* counters, float* partials);

}  // namespace pqkv
