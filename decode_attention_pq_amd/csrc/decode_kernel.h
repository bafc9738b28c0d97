// PQ decode attention in one kernel (included by the decode_m*.hip translation
// units, each of which instantiates one family of builds): ad-LUT scoring of the compressed history,
// split-over-tokens softmax with a per-subspace histogram value side, exact
// attention over the recent full-precision window, and the log-sum-exp merge.
//
// MILLION write-up (DAC 2025), page "MILLION":
//   - Fig. 7 paragraph: history attention and new-token attention are computed
//     apart and combined; because the history is much longer than the codebook,
//     the query x codebook asymmetric-distance table (ad-LUT) is built first and
//     replaces per-token inner products.
//   - Fig. 8 paragraph: a flash-decoding base (the history is split across
//     work-groups and their partial softmax states are reduced) with packed codes
//     loaded as wide words.
//
// gfx950 design (not the page's GPU design):
//   - One work-group of 512 threads per (sequence, kv head, query-head group,
//     history split).  Work-group ids are remapped so that all splits of one kv
//     head run on the same XCD and share its L2 copy of the codebooks.
//   - Every wave owns whole 64-token tiles; a lane holds one token's M codes,
//     read with M/16 16-byte loads that are contiguous across the wave.  A wave
//     walks one stream of tiles -- its K tiles, then the V tiles of the same
//     tokens -- keeping three tiles in flight ahead of the one in use.  The
//     codebook values for the LUT are requested before the first tiles, because
//     vector-memory loads of a wave retire in issue order.
//   - LDS holds a u32 histogram (bytes 0..64K) and the ad-LUT of the
//     work-group's QH query heads (bytes 64K..128K), both with row c = centroid
//     c and entry m*QH + j = (subspace m, query head j): the heads of a subspace
//     are adjacent, so with QH >= 2 one 8-byte read gathers two heads' table
//     entries and one 8-byte atomic adds two heads' weights (the LDS pays about
//     1.1x and 1.45x the time of the 4-byte forms for them).  The code-cache layout
//     rotates each token's bytes by its slot, so at every step the 64 lanes
//     address 64 different subspaces and the LDS accesses never conflict; one
//     v_perm_b32 per code forms the byte address (code << 8) | (4*QH*m),
//     plus 0x10000 for the LUT.
//   - A wave's tiles per split (RW: 2 to 16) are a template parameter: their
//     scores stay in registers until the work-group max is known.
//   - Two-phase softmax inside the work-group: scores stay in registers, the
//     work-group max is taken once, then p = exp2(s - max) is added into the
//     histogram.  The adds are u32 fixed point (round(p * 2^S)): on gfx950 an
//     fp32 LDS add serialises the wave (~190 clk per instruction) while the u32
//     add takes ~4 clk.  S comes from a bound on the split's weight sum (taken
//     with the max), as large as keeps every cell inside u32, so the rounding is
//     relative to the sum of the weights.
//   - Each work-group also takes a slice of the recent window (exact fp32 dot
//     products), writes its partial (max, sum, unnormalised output), and the
//     last work-group of a (sequence, kv head, group) to finish merges all
//     partials into out and lse (completion counter in the workspace).  A unit
//     whose history fits one split writes out and lse directly.

#pragma once

#include <hip/hip_fp16.h>

#include "pqkv_internal.h"

namespace pqkv {
namespace {

constexpr float kLn2 = 0.6931471805599453f;
constexpr int kThreads = kDecodeThreads;
constexpr int kWaves = kDecodeWaves;
constexpr int kRow = 64;  // floats per LDS table row
constexpr int kPrefetch = 3;  // code tiles a wave keeps in flight ahead of use
constexpr int kRecentPre = 4; // recent rows per wave requested before the first tiles

__device__ inline float to_f32(float v) { return v; }
__device__ inline float to_f32(__half v) { return __half2float(v); }

// Wave-wide reductions on DPP lane moves (no LDS round trips): pairs, quads,
// half rows and rows of 16 by quad permutes and mirrors, then rows 0+1 and 2+3
// by row_bcast:15 and the whole wave by row_bcast:31; lane 63 ends with the
// total, which readlane makes uniform.  Lanes a row-masked move does not write
// take `id`, the operation's identity.
template <int CTRL, int ROWS>
__device__ inline uint32_t dpp_move(uint32_t v, uint32_t id) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, CTRL, ROWS, 0xF, false);
}

template <typename Op>
__device__ inline uint32_t wave_reduce(uint32_t v, uint32_t id, Op op) {
    v = op(v, dpp_move<0xB1, 0xF>(v, id));   // quad_perm [1,0,3,2]
    v = op(v, dpp_move<0x4E, 0xF>(v, id));   // quad_perm [2,3,0,1]
    v = op(v, dpp_move<0x141, 0xF>(v, id));  // row_half_mirror
    v = op(v, dpp_move<0x140, 0xF>(v, id));  // row_mirror
    v = op(v, dpp_move<0x142, 0xA>(v, id));  // row_bcast:15 into rows 1 and 3
    v = op(v, dpp_move<0x143, 0xC>(v, id));  // row_bcast:31 into rows 2 and 3
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ inline float wave_max(float v) {
    return __uint_as_float(wave_reduce(__float_as_uint(v), 0xff800000u, [](uint32_t x, uint32_t y) {
        return __float_as_uint(fmaxf(__uint_as_float(x), __uint_as_float(y)));
    }));
}

__device__ inline float wave_sum(float v) {
    return __uint_as_float(wave_reduce(__float_as_uint(v), 0u, [](uint32_t x, uint32_t y) {
        return __float_as_uint(__uint_as_float(x) + __uint_as_float(y));
    }));
}

__device__ inline uint32_t wave_sum_u32(uint32_t v) {
    return wave_reduce(v, 0u, [](uint32_t x, uint32_t y) { return x + y; });
}

__device__ inline uint32_t wave_min_u32(uint32_t v) {
    return wave_reduce(v, 0xffffffffu, [](uint32_t x, uint32_t y) { return x < y ? x : y; });
}

__device__ inline uint32_t wave_max_u32(uint32_t v) {
    return wave_reduce(v, 0u, [](uint32_t x, uint32_t y) { return x > y ? x : y; });
}

// ceil(x / y) for x, y < 2^22 (x a count of 512-token rounds): a float quotient,
// corrected to the exact one.
__device__ inline uint32_t ceil_div_small(uint32_t x, uint32_t y) {
    uint32_t q = (uint32_t)((float)x / (float)y);
    q += q * y < x ? 1u : 0u;
    q += q * y < x ? 1u : 0u;
    q -= (q > 0u && (q - 1u) * y >= x) ? 1u : 0u;
    return q;
}

// LDS byte offset of a pointer into a __shared__ array.
__device__ inline uint32_t lds_offset(const float* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) float*)p;
}

// Direct-to-LDS 16-byte load: lane l's 16 bytes from `src` land at LDS byte
// `lds_base + 16*l` (lds_base wave-uniform).  Issued from inline assembly so
// the compiler does not make every later LDS access wait for all outstanding
// loads; the reader must wait (vmcnt 0) before touching the destination.  M0,
// which holds the LDS base for the instruction, is restored afterwards.
__device__ inline void lds_dma16(const void* src, uint32_t lds_base) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
        : "memory");
}

// N consecutive floats (N = 2 or 4, 8- or 16-byte aligned) in one load.
template <int N>
__device__ inline void load_f32x(const float* p, float (&v)[N]) {
    if constexpr (N == 4) {
        const float4 t = *reinterpret_cast<const float4*>(p);
        v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    } else if constexpr (N == 2) {
        const float2 t = *reinterpret_cast<const float2*>(p);
        v[0] = t.x; v[1] = t.y;
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = p[i];
    }
}

// Histogram byte address of byte s of code word `cw`, with byte s of offset word
// `mw`: (code << 8) | (4*QH*m).  v_perm_b32 selector: result byte 0 = source-1 byte
// s, byte 1 = source-0 byte s, bytes 2 and 3 = 0.
template <int S>
__device__ inline uint32_t hist_addr(uint32_t cw, uint32_t mw) {
    constexpr uint32_t sel = 0x0c0c0000u | ((4u + S) << 8) | (uint32_t)S;
    return __builtin_amdgcn_perm(cw, mw, sel);
}

// Same for the LUT at LDS byte 65536: `ml` holds the offsets of two steps in
// bytes 0-1 and the constant 1 in byte 2, giving 0x10000 | (code << 8) | (4*QH*m).
template <int S>
__device__ inline uint32_t lut_addr(uint32_t cw, uint32_t ml) {
    constexpr uint32_t sel = 0x0c000000u | (2u << 16) | ((4u + S) << 8) | (uint32_t)(S & 1);
    return __builtin_amdgcn_perm(cw, ml, sel);
}

__device__ inline float lds_f32(const float* base, uint32_t byte_off) {
    return *reinterpret_cast<const float*>(reinterpret_cast<const char*>(base) + byte_off);
}

__device__ inline void lds_add_u32(float* base, uint32_t byte_off, uint32_t v) {
    __hip_atomic_fetch_add(reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(base) + byte_off), v,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Two adjacent table entries (two query heads of one subspace) in one 8-byte read.
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ inline f32x2 lds_f32x2(const float* base, uint32_t byte_off) {
    const void* p = __builtin_assume_aligned(reinterpret_cast<const char*>(base) + byte_off, 8);
    return *static_cast<const f32x2*>(p);
}

// Two adjacent u32 histogram cells (two query heads of one subspace) in one 8-byte
// add: the low word never carries into the high one, every cell staying below 2^32.
__device__ inline void lds_add_u32x2(float* base, uint32_t byte_off, uint32_t lo, uint32_t hi) {
    __hip_atomic_fetch_add(reinterpret_cast<unsigned long long*>(reinterpret_cast<char*>(base) + byte_off),
                           ((unsigned long long)hi << 32) | lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Read by loads whose slot is unused (a tile past the history, a missing
// codebook): every prefetch is issued unconditionally, which lets the compiler
// count outstanding loads exactly instead of waiting for all of them.
__device__ uint4 g_zero_block[kTileTokens * 4];

// Cross-work-group partial results: device-coherent store and load.
__device__ inline void publish(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ inline float collect(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Code tiles are read once per call: non-temporal loads keep them from evicting
// the codebooks and the kernel's own code from the caches.
template <int NCH>
__device__ inline void load_tile(u32x4 (&cw)[NCH], const uint8_t* __restrict__ plane, int64_t tile, int lane,
                                 bool ok) {
    const uint8_t* p = ok ? plane + tile * (kTileTokens * NCH * 16) : reinterpret_cast<const uint8_t*>(g_zero_block);
    p += ok ? lane * 16 : 0;  // an unused slot reads one 16-byte line
#pragma unroll
    for (int c = 0; c < NCH; ++c)
        cw[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + c * (kTileTokens * 16)));
}

__device__ inline void load4(const float* p, float (&v)[4]) {
    const float4 t = *reinterpret_cast<const float4*>(p);
    v[0] = t.x;
    v[1] = t.y;
    v[2] = t.z;
    v[3] = t.w;
}

__device__ inline void load4(const __half* p, float (&v)[4]) {
    const uint2 t = *reinterpret_cast<const uint2*>(p);
    const float2 a = __half22float2(*reinterpret_cast<const __half2*>(&t.x));
    const float2 b = __half22float2(*reinterpret_cast<const __half2*>(&t.y));
    v[0] = a.x;
    v[1] = a.y;
    v[2] = b.x;
    v[3] = b.y;
}

#ifdef PQKV_TIMELINE
// Probe builds only (tests/probes/decode_timeline.py): lane 0 of every wave writes
// s_memrealtime stamps to g_timeline[(work-group * 8 + wave) * 48 + k]: k < 14 at the
// phase boundaries, 14 and 15 the work-group's XCC_ID and HW_ID registers, 16 + s when
// step s's code tile is in registers (s < 32; the stamp first waits for the whole
// tile).  libpqkv itself is built without it, and stamp() and tile_ready() are empty.
__device__ unsigned long long* g_timeline;
#endif

// Issue priority of this wave on its SIMD (0-3).  The two waves of a SIMD would
// otherwise be served oldest first, so the younger one falls behind in each phase and
// the work-group then waits for it at the next barrier; a wave that is ahead by a
// quarter of the phase's tiles drops a level below the other.
__device__ inline void set_prio(int p) {
    if (p <= 0) __builtin_amdgcn_s_setprio(0);
    else if (p == 1) __builtin_amdgcn_s_setprio(1);
    else if (p == 2) __builtin_amdgcn_s_setprio(2);
    else __builtin_amdgcn_s_setprio(3);
}

struct DecArgs {
    // first 64 bytes: everything the work mapping and the first loads need, so one
    // scalar load brings it in
    int K, Hq, Hkv, n_groups, n_split, rounds, n_items;
    int len_first;  // 0: lengths read after the first loads (one sequence); 1: before them;
                    // 2: all of them before anything else, for the device-side split plan
    int64_t split_tokens;
    const int32_t* hist_len;
    const int32_t* recent_len;
    const void* q;
    const float* lut;   // the materialised ad-LUT [B][Hq][M][K] (EXT builds), unscaled
    const float* cb_k;
    const float* cb_v;
    const uint8_t* codes_k;
    const uint8_t* codes_v;
    int64_t t_cap;
    int64_t max_hist;
    const void* rk;
    const void* rv;
    int64_t r_cap;
    float scale_log2;
    int pstride;
    float* partials;
    uint32_t* counters;
    float* out;
    float* lse;
};

// EXT: the ad-LUT comes from memory (pqkv_build_lut's table) instead of being built
// from q and the key codebook.
template <int M, int DSUB, int QH, int RW, bool EXT, typename QT, typename RT>
__global__ __launch_bounds__(kThreads) void pq_decode_kernel(DecArgs a) {
    constexpr int D = M * DSUB;
    constexpr int NCH = M / 16;
    static_assert(RW >= 1 && RW <= decode_max_rounds(M, QH), "tiles per wave beyond the register budget");
    constexpr int RS = PQKV_MAX_RECENT;
    constexpr int P = kPrefetch;          // tiles in flight ahead of the one being used
    constexpr int NSLOT = P + 1;
    constexpr int CPL = D / 64;                // epilogue: output components per lane
    constexpr int CPER = kLdsRows / kWaves;    // epilogue: centroids per wave
    constexpr int CHALF = CPER / 2;            // of which staged through LDS
    static_assert(kWaves * CHALF * D <= kLdsRows * kRow, "staged value rows must fit the LUT region");
    static_assert(QH * M <= kRow, "query-head group must fit one LDS row");
    // LDS table columns: subspace m, query head j at column m*QH + j, so the QH heads of a
    // subspace sit side by side and a pair of them is one 8-byte access
    constexpr int CS = 4 * QH;  // bytes per subspace in a row
    static_assert(CS * (M - 1) <= 255, "subspace offsets must fit one address byte");

    // LDS: histogram (u32) at byte 0, LUT at byte 65536, then the small buffers.
    __shared__ float lds[2 * kLdsRows * kRow];
    __shared__ float ored[kWaves * QH * D];     // per-wave output partials
    __shared__ float rs[QH * RS];               // recent scores, then weights * 2^S
    __shared__ float red[kWaves * QH];   // per-wave maxima
    __shared__ float redl[kWaves * QH];  // per-wave bounds on the history weight sums
    __shared__ float redr[kWaves * QH];  // per-wave recent weight sums
    __shared__ uint32_t redu[kWaves * QH];
    __shared__ float lfin[QH];           // single-split units: the weight sums
    __shared__ int last_flag;
    uint32_t* hist = reinterpret_cast<uint32_t*>(lds);
    float* table = lds + kLdsRows * kRow;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
#ifdef PQKV_TIMELINE
    unsigned long long* tl = g_timeline ? g_timeline + ((size_t)blockIdx.x * kWaves + wave) * 48 : nullptr;
    auto stamp = [&](int k) {
        if (tl && lane == 0 && k < 48) tl[k] = __builtin_amdgcn_s_memrealtime();
    };
    auto tile_ready = [&](int s, const u32x4(&cw)[NCH]) {
        asm volatile("" ::"v"(cw[0].x), "v"(cw[NCH - 1].w));
        stamp(16 + s);
    };
    stamp(0);
    if (tl && lane == 0) {
        tl[14] = (unsigned)__builtin_amdgcn_s_getreg((20 << 0) | (0 << 6) | (31 << 11));  // XCC_ID
        tl[15] = (unsigned)__builtin_amdgcn_s_getreg((4 << 0) | (0 << 6) | (31 << 11));   // HW_ID
    }
#else
    auto stamp = [](int) {};
    auto tile_ready = [](int, const u32x4(&)[NCH]) {};
#endif

    // XCD-aware work mapping: work-group ids that share an XCD (id mod 8) take
    // contiguous items, so all splits of one kv head meet in one L2.  The grid has
    // exactly n_items work-groups; XCD x holds ceil((n_items - x) / 8) of them.
    // Items run head-major (all sequences of kv head 0, then of head 1, ...), so
    // every XCD gets a share of every sequence even when their lengths differ.
    const int L = blockIdx.x;
    int item = xcd_item(L, a.n_items);
    const int batch = a.n_items / (a.Hkv * a.n_groups * a.n_split);
    // This work-group's piece: sequence b, kv head h, query-head group grp, split
    // `split` of the sequence's ns_dev splits (device plan) starting at token t0 and at
    // most tspan long; its partial record is item item_first + split.
    int b, h, grp, split, item_first, ns_dev = 0, T_dev = 0;
    int64_t t0, tspan;
    int mode = a.len_first;
    int Tl = 0;
    if (mode == 2) {
        // lane l holds sequence l's length; equal lengths keep the host's plan
        int li = lane < batch ? lane : 0;
        asm volatile("" : "+v"(li));
        Tl = a.hist_len[li];
        Tl = lane < batch ? (Tl < 0 ? 0 : (Tl > (int)a.max_hist ? (int)a.max_hist : Tl)) : 0;
        const uint32_t lo = wave_min_u32(lane < batch ? (uint32_t)Tl : 0xffffffffu);
        if (lo == wave_max_u32((uint32_t)Tl)) mode = 1;
    }
    if (mode == 2) {
        // ---- the device-side split plan (2 <= batch <= 16): lane l holds sequence l's
        // length; lane r - 1 prices splits of at most r rounds (r <= RW, this build) with
        // the host plan's cost model, over the grid the host launched; the cheapest wins,
        // fewer work-groups on a tie.  Every wave computes the same plan.
        const uint32_t u = ((uint32_t)Tl + kTokensPerRound - 1u) / kTokensPerRound;  // rounds of the sequence
        const uint32_t r = (uint32_t)lane + 1u;
        uint32_t S = 0u, RRm = 0u;
        for (int q = 0; q < batch; ++q) {
            const uint32_t uq = (uint32_t)__builtin_amdgcn_readlane((int)u, q);
            const uint32_t nb = uq ? ceil_div_small(uq, r) : 1u;
            const uint32_t rr = uq ? ceil_div_small(uq, nb) : 0u;
            S += nb;
            RRm = rr > RRm ? rr : RRm;
        }
        const uint64_t items_r = (uint64_t)(a.Hkv * a.n_groups) * S;
        const uint64_t waves_r = (items_r + kPlanCUs - 1) / kPlanCUs;
        const uint64_t cost_r = waves_r * (uint64_t)(kPlanFixed + kPlanRound * RRm + kPlanUnused * (RW - RRm));
        const bool cand = r <= (uint32_t)RW && items_r <= (uint64_t)a.n_items;
        const uint32_t cost = cand ? (uint32_t)(cost_r < 0xfffffffeull ? cost_r : 0xfffffffeull) : 0xffffffffu;
        const uint32_t best = wave_min_u32(cost);
        const uint32_t rbest = wave_max_u32(cost == best ? r : 0u);  // the longest splits among the cheapest
        const uint32_t nbl = lane < batch ? (u ? ceil_div_small(u, rbest) : 1u) : 0u;
        const uint32_t Sb = wave_sum_u32(nbl);
        // the plan's items spread over every XCD the same way, contiguous within one:
        // XCD x takes ceil((used - x) / 8) of them; the grid's other work-groups exit
        // (nothing issued yet but the lengths, which have landed)
        const int used = a.Hkv * a.n_groups * (int)Sb;
        if (!xcd_has_item(L, used)) return;
        item = xcd_item(L, used);
        const int hg = item / (int)Sb;
        const int kk = item - hg * (int)Sb;
        int acc = 0, bq = 0;
        for (int q = 0; q < batch; ++q) {
            const int n = __builtin_amdgcn_readlane((int)nbl, q);
            if (kk < acc + n) {
                bq = q;
                break;
            }
            acc += n;
        }
        b = bq;
        split = kk - acc;
        ns_dev = __builtin_amdgcn_readlane((int)nbl, b);
        T_dev = __builtin_amdgcn_readlane(Tl, b);
        // even splits of the sequence, whole 64-token tiles each
        tspan = T_dev > 0 ? ((int64_t)(((uint32_t)T_dev + (uint32_t)ns_dev - 1u) / (uint32_t)ns_dev) + kTileTokens - 1) /
                                kTileTokens * kTileTokens
                          : kTileTokens;
        t0 = (int64_t)split * tspan;
        grp = hg % a.n_groups;
        h = hg / a.n_groups;
        item_first = hg * (int)Sb + acc;
    } else {
        const int unit0 = item / a.n_split;
        split = item - unit0 * a.n_split;
        grp = unit0 % a.n_groups;
        const int hb = unit0 / a.n_groups;
        b = hb % batch;
        h = hb / batch;
        item_first = unit0 * a.n_split;
        t0 = (int64_t)split * a.split_tokens;
        tspan = a.split_tokens;
    }
    const int unit = (h * batch + b) * a.n_groups + grp;  // its completion counter
    const int hq0 = h * (a.Hq / a.Hkv) + grp * QH;
    const int K = a.K;

    // The lengths come through the vector memory path: scalar loads return out of
    // order, so waiting for one would also wait for every later scalar load.  They
    // are used only after the length-independent loads below have been issued.
    int len_idx = b;
    asm volatile("" : "+v"(len_idx));  // a per-lane index makes these vector loads
    // (the device plan has read every length already)
    const int T_in = mode == 2 ? T_dev : (a.hist_len ? a.hist_len[len_idx] : 0);  // no history: no lengths
    const int R_in = a.recent_len ? a.recent_len[len_idx] : 0;
    // A sequence uses the splits that hold its history (at least one, which also
    // takes the recent window or gives the empty result); work-groups of the other
    // splits have nothing to do.  When lengths may differ, they learn it before
    // issuing any load.
    auto splits_used = [&](int64_t Tc) -> int {  // lengths are int32 and split_tokens <= 2^13
        const uint32_t st = (uint32_t)a.split_tokens;
        return Tc > 0 ? (int)(((uint32_t)Tc + st - 1u) / st) : 1;
    };
    auto clamp_hist = [&](int64_t Tr) -> int64_t { return Tr < 0 ? 0 : (Tr > a.max_hist ? a.max_hist : Tr); };
    if (mode == 1) {
        int T_early = T_in;
        asm volatile("" : "+v"(T_early));
        if (split >= splits_used(clamp_hist(T_early))) {
            __builtin_amdgcn_s_waitcnt(0);
            return;
        }
    }
    __builtin_amdgcn_sched_barrier(0);  // nothing below moves above the check
    const int64_t tile0 = t0 / kTileTokens;
    const int rounds = mode == 2 ? RW : a.rounds;  // a device plan's splits end at t1, within RW rounds

    // ---- 1. loads in the order they are needed (a wave's loads retire in issue
    //         order): this thread's query values, the codebook values of this
    //         thread's LUT entries, the first recent rows, the first tiles.
    //         LUT entries: thread t builds subspaces [mg*EPL, mg*EPL + EPL) of
    //         centroids c = (t + k*512) / (M/EPL), from one 16-byte load each.
    constexpr int EPL = 4 / DSUB;
    constexpr int LUT_LOADS = kLdsRows * M / EPL / kThreads;
    static_assert(LUT_LOADS * kThreads == kLdsRows * (M / EPL), "the LUT loads cover the table rows exactly");
    const int mg = tid % (M / EPL);
    const QT* qrow = static_cast<const QT*>(a.q) + (int64_t)(b * a.Hq + hq0) * D;
    float ql[QH][4];       // q elements [4*mg, 4*mg + 4) of each head, for the LUT
    float qr[QH][D / 64];  // q elements lane + 64k of each head, for the recent scores
#pragma unroll
    for (int j = 0; j < QH; ++j) {
        load4(qrow + j * D + 4 * mg, ql[j]);
#pragma unroll
        for (int k = 0; k < D / 64; ++k) qr[j][k] = to_f32(qrow[j * D + lane + 64 * k]);
    }
    // The splits of one head share an L2: each starts on a different block of
    // centroids, so the first requests of all of them together cover the
    // codebook once and the later ones find it in L2.
    const int lut_rot = split * LUT_LOADS / (a.n_split < LUT_LOADS ? a.n_split : LUT_LOADS);
    auto lut_block = [&](int k) { return (k + lut_rot) % LUT_LOADS; };
    // A materialised table: thread t takes column col = t % COLS (query head col / M,
    // subspace col % M) and blocks of 4 centroids t / COLS + k * (512 / COLS), one
    // 16-byte load each (the table holds K consecutive centroids per (head, subspace)).
    // A wave's lanes take distinct columns, so the LDS stores do not conflict.
    constexpr int COLS = QH * M;
    constexpr int XLOADS = EXT ? kLdsRows * COLS / 4 / kThreads : 0;
    const int xcol = tid % COLS;
    auto xblock = [&](int k) { return tid / COLS + k * (kThreads / COLS); };
    float4 xlut[XLOADS > 0 ? XLOADS : 1];
    if constexpr (EXT) {
        const float* lc = a.lut + ((int64_t)(b * a.Hq + hq0) * M + xcol) * K;
#pragma unroll
        for (int k = 0; k < XLOADS; ++k) {
            const int c0 = 4 * xblock(k) < K - 4 ? 4 * xblock(k) : K - 4;  // rows past K copy the last four
            xlut[k] = *reinterpret_cast<const float4*>(lc + c0);
        }
    }
    float4 cbq[EXT ? 1 : LUT_LOADS];
    if constexpr (!EXT) {
        const float* cbh = a.cb_k ? a.cb_k + (int64_t)h * K * M * DSUB + mg * 4
                                  : reinterpret_cast<const float*>(g_zero_block);
        const int cstride = a.cb_k ? M * DSUB : 0;
#pragma unroll
        for (int k = 0; k < LUT_LOADS; ++k) {
            int c = (tid + lut_block(k) * kThreads) / (M / EPL);
            c = c < K ? c : K - 1;
            cbq[k] = *reinterpret_cast<const float4*>(cbh + (int64_t)c * cstride);
        }
    }
    // Keep the scheduler from hoisting later loads above the codebook loads (the LUT
    // would then wait for them too); the loads below also depend on the sequence
    // lengths, whose fetch the codebook loads overlap.
    __builtin_amdgcn_sched_barrier(0);
    stamp(1);  // codebook requests issued
    int T_v = T_in, R_v = R_in;
    asm volatile("" : "+v"(T_v), "+v"(R_v));  // first use of the lengths: here, not earlier
    const int64_t T = clamp_hist(T_v);
    const int ns = mode == 2 ? ns_dev : splits_used(T);
    if (split >= ns) {  // loads are in flight: let them land before the work-group ends
        __builtin_amdgcn_s_waitcnt(0);
        return;
    }
    const int64_t t1 = T < t0 + tspan ? T : t0 + tspan;
    int R = R_v;
    R = R < 0 ? 0 : (R > a.r_cap ? (int)a.r_cap : R);
    const int rs_per = (R + ns - 1) / ns;
    const int r0 = split * rs_per;
    const int n_rec = R - r0 < rs_per ? (R - r0 > 0 ? R - r0 : 0) : rs_per;
    const bool has_hist = t0 < t1;

    const int64_t plane_off = ((int64_t)b * a.Hkv + h) * a.t_cap * M;
    const uint8_t* plane_k = a.codes_k + plane_off;
    const uint8_t* plane_v = a.codes_v + plane_off;

    // Step s < RW scores K tile s of this wave; step RW + s adds V tile s into the
    // histogram.  Tile of round r: tile0 + r*8 + wave.
    auto step_tile = [&](int s) -> int64_t { return tile0 + (int64_t)(s < RW ? s : s - RW) * kWaves + wave; };
    auto step_ok = [&](int s) -> bool {
        const int r = s < RW ? s : s - RW;
        return r < rounds && step_tile(s) * kTileTokens < t1;
    };
    auto issue = [&](u32x4 (&slot)[NCH], int s) {
        load_tile<NCH>(slot, s < RW ? plane_k : plane_v, step_tile(s), lane, step_ok(s));
    };
    const RT* rk = static_cast<const RT*>(a.rk) + (((int64_t)b * a.Hkv + h) * a.r_cap + r0) * D;
    const RT* rv = static_cast<const RT*>(a.rv) + (((int64_t)b * a.Hkv + h) * a.r_cap + r0) * D;
    const RT* rzero = reinterpret_cast<const RT*>(g_zero_block);
    float kpre[kRecentPre][D / 64];
#pragma unroll
    for (int p = 0; p < kRecentPre; ++p) {
        const int i = wave + p * kWaves;
        const RT* row = i < n_rec ? rk + (int64_t)i * D + lane : rzero;
#pragma unroll
        for (int k = 0; k < D / 64; ++k) kpre[p][k] = to_f32(row[i < n_rec ? 64 * k : 0]);
    }
    u32x4 ring[NSLOT][NCH];
#pragma unroll
    for (int s = 0; s < P; ++s) issue(ring[s], s);

    // zero the histogram now, while the codebook is on its way (phase 1 reads only the
    // LUT region; the barrier before phase 1 orders these stores before any atomic).
    // All rows: those past K stay 0, so the epilogue reads them without a check.
    if (has_hist)
        for (int e = tid; e < kLdsRows * kRow / 4; e += kThreads)
            reinterpret_cast<uint4*>(hist)[e] = make_uint4(0u, 0u, 0u, 0u);

    // ---- 2. ad-LUT in LDS, recent-window scores, per-lane subspace offsets
#pragma unroll
    for (int j = 0; j < QH; ++j) {
#pragma unroll
        for (int i = 0; i < 4; ++i) ql[j][i] *= a.scale_log2;
#pragma unroll
        for (int k = 0; k < D / 64; ++k) qr[j][k] *= a.scale_log2;
    }
    if constexpr (EXT) {
        if (has_hist) {
#pragma unroll
            for (int k = 0; k < XLOADS; ++k) {
                const float v[4] = {xlut[k].x, xlut[k].y, xlut[k].z, xlut[k].w};
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    table[(4 * xblock(k) + i) * kRow + (xcol % M) * QH + xcol / M] = v[i] * a.scale_log2;
            }
        }
    } else if (has_hist) {
#pragma unroll
        for (int k = 0; k < LUT_LOADS; ++k) {
            // c < kLdsRows always; rows past K hold copies of row K-1 that no code reads
            const int c = (tid + lut_block(k) * kThreads) / (M / EPL);
            const float cv[4] = {cbq[k].x, cbq[k].y, cbq[k].z, cbq[k].w};
#pragma unroll
            for (int j = 0; j < QH; ++j) {
#pragma unroll
                for (int t = 0; t < EPL; ++t) {
                    float s = 0.0f;
#pragma unroll
                    for (int i = 0; i < DSUB; ++i) s = fmaf(ql[j][t * DSUB + i], cv[t * DSUB + i], s);
                    table[c * kRow + (mg * EPL + t) * QH + j] = s;
                }
            }
        }
    }
    for (int i = wave, p = 0; i < n_rec; i += kWaves, ++p) {
        float kv[D / 64];
        if (p < kRecentPre) {  // prefetched above
#pragma unroll
            for (int q = 0; q < kRecentPre; ++q)
                if (q == p)
#pragma unroll
                    for (int k = 0; k < D / 64; ++k) kv[k] = kpre[q][k];
        } else {
#pragma unroll
            for (int k = 0; k < D / 64; ++k) kv[k] = to_f32(rk[(int64_t)i * D + lane + 64 * k]);
        }
#pragma unroll
        for (int j = 0; j < QH; ++j) {
            float s = 0.0f;
#pragma unroll
            for (int k = 0; k < D / 64; ++k) s = fmaf(qr[j][k], kv[k], s);
            s = wave_sum(s);
            if (lane == 0) rs[j * RS + i] = s;
        }
    }
    // ml[k]: subspace byte offsets CS*((2k + slot) mod M) and CS*((2k + 1 + slot) mod M)
    // in bytes 0-1 and the LUT's 64 KiB base in byte 2
    uint32_t ml[M / 2];
#pragma unroll
    for (int k = 0; k < M / 2; ++k)
        ml[k] = 0x10000u | (uint32_t)(((2 * k + lane) & (M - 1)) * CS) |
                ((uint32_t)(((2 * k + 1 + lane) & (M - 1)) * CS) << 8);
    stamp(2);  // this wave's part of the LUT built
    __syncthreads();
    stamp(3);  // phase 1 starts

    // ---- 3. phase 1: K codes -> scores (log2 domain)
    float sc[RW][QH];
#pragma unroll
    for (int s = 0; s < RW; ++s) {
        set_prio(3 - (4 * s) / RW);
        if (s == RW / 2) stamp(12);  // half of phase 1
        issue(ring[(s + P) % NSLOT], s + P);
#pragma unroll
        for (int j = 0; j < QH; ++j) sc[s][j] = -INFINITY;
        if (step_ok(s)) {
            const u32x4(&cw)[NCH] = ring[s % NSLOT];
            tile_ready(s, cw);
            float acc[QH][4];
#pragma unroll
            for (int j = 0; j < QH; ++j)
#pragma unroll
                for (int t = 0; t < 4; ++t) acc[j][t] = 0.0f;
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const uint32_t words[4] = {cw[c].x, cw[c].y, cw[c].z, cw[c].w};
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t a0 = lut_addr<0>(words[w], ml[c * 8 + 2 * w]);
                    const uint32_t a1 = lut_addr<1>(words[w], ml[c * 8 + 2 * w]);
                    const uint32_t a2 = lut_addr<2>(words[w], ml[c * 8 + 2 * w + 1]);
                    const uint32_t a3 = lut_addr<3>(words[w], ml[c * 8 + 2 * w + 1]);
                    if constexpr (QH == 1) {  // addresses carry the 65536 base
                        acc[0][0] += lds_f32(lds, a0);
                        acc[0][1] += lds_f32(lds, a1);
                        acc[0][2] += lds_f32(lds, a2);
                        acc[0][3] += lds_f32(lds, a3);
                    } else {
#pragma unroll
                        for (int jp = 0; jp < QH; jp += 2) {  // two heads per read
                            const f32x2 v0 = lds_f32x2(lds + jp, a0), v1 = lds_f32x2(lds + jp, a1);
                            const f32x2 v2 = lds_f32x2(lds + jp, a2), v3 = lds_f32x2(lds + jp, a3);
                            acc[jp][0] += v0.x;
                            acc[jp + 1][0] += v0.y;
                            acc[jp][1] += v1.x;
                            acc[jp + 1][1] += v1.y;
                            acc[jp][2] += v2.x;
                            acc[jp + 1][2] += v2.y;
                            acc[jp][3] += v3.x;
                            acc[jp + 1][3] += v3.y;
                        }
                    }
                }
            }
            const bool tok_ok = step_tile(s) * kTileTokens + lane < t1;
#pragma unroll
            for (int j = 0; j < QH; ++j)
                sc[s][j] = tok_ok ? (acc[j][0] + acc[j][1]) + (acc[j][2] + acc[j][3]) : -INFINITY;
        }
    }

    stamp(4);  // phase 1 ends
    set_prio(0);
    // ---- 4. work-group max over history and recent scores, and a bound on the
    //         history's weight sum, which sets the histogram's fixed-point scale: a
    //         lane's RW weights sum to at most RW times its largest.  Each wave takes
    //         the bound against its own max; the waves' bounds meet after the barrier.
#pragma unroll
    for (int j = 0; j < QH; ++j) {
        float vl = -INFINITY;
#pragma unroll
        for (int s = 0; s < RW; ++s) vl = fmaxf(vl, sc[s][j]);
        float v = vl;
        for (int i = tid; i < n_rec; i += kThreads) v = fmaxf(v, rs[j * RS + i]);
        v = wave_max(v);
        float l = vl != -INFINITY ? (float)RW * exp2f(vl - v) : 0.0f;
        l = wave_sum(l);
        if (lane == 0) {
            red[wave * QH + j] = v;
            redl[wave * QH + j] = l;
        }
    }
    __syncthreads();
    stamp(5);  // the maxima have met
    // Fixed point: the history weights p = 2^(s - max) are added to the histogram as
    // round(p * 2^S), S the largest with L * 2^S < 2^31 for the bound L on the split's
    // weight sum (capped at 64).  A cell, and the split's sum, then stay below 2^31
    // plus half a unit per token, inside u32, and each weight is exact to 2^-(S+1),
    // i.e. to L * 2^-32 with L at most RW times the true sum: the rounding is
    // relative to the sum of the weights, not to the largest one.
    float mx[QH], fs[QH], fi[QH];
#pragma unroll
    for (int j = 0; j < QH; ++j) {
        float mw[kWaves], lw[kWaves];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            mw[w] = red[w * QH + j];
            lw[w] = redl[w * QH + j];
        }
        float v = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) v = fmaxf(v, mw[w]);
        // a wave without tokens has max -inf and adds 2^-inf = 0 (its bound is finite)
        float L = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) L = fmaf(lw[w], exp2f(mw[w] - v), L);
        if (v == -INFINITY) L = 0.0f;
        mx[j] = v;
        // L = f * 2^e with f in [0.5, 1): S = 31 - e (normal L; 64 for zero or tiny L)
        const int e = (int)((__float_as_uint(L) >> 23) & 0xffu) - 126;
        int S = L >= 1.0e-30f ? 31 - e : 64;
        S = S < 0 ? 0 : (S > 64 ? 64 : S);
        fs[j] = __uint_as_float((uint32_t)(127 + S) << 23);
        fi[j] = __uint_as_float((uint32_t)(127 - S) << 23);
    }
    const bool any = mx[0] != -INFINITY;  // the split holds at least one token (all heads alike)

    // ---- 5. phase 2: add round(p * 2^S) into histogram[code][m].
    // First request this thread's value-codebook entries for the epilogue: lane
    // (cg, m) of wave w covers subspace m, components [cg*CPL, cg*CPL + CPL) and
    // centroids [w*CPER, w*CPER + CPER).  The first half of those centroid rows
    // go straight into this wave's block of the LUT region (unused from here on)
    // by direct-to-LDS loads; the second half come to registers.
    const int em = lane % M;
    const int ecomp = (lane / M) * CPL;
    const int ec0 = wave * CPER;
    const float* cv_lds = lds + kLdsRows * kRow + wave * (CHALF * D);
    {
        const float* head = a.cb_v ? a.cb_v + (int64_t)h * K * D : nullptr;
        const uint32_t dst = lds_offset(cv_lds);
#pragma unroll
        for (int i = 0; i < CHALF * D / 256; ++i) {  // 1 KiB (64 lanes x 16 bytes) per load
            const int foff = ec0 * D + i * 256 + lane * 4;
            const float* src = (head && foff / D < K) ? head + foff
                                                      : reinterpret_cast<const float*>(g_zero_block) + lane * 4;
            lds_dma16(src, dst + i * 1024);
        }
    }
    const float* cbv = a.cb_v ? a.cb_v + (int64_t)h * K * M * DSUB + em * DSUB + ecomp
                              : reinterpret_cast<const float*>(g_zero_block);
    const int vstride = a.cb_v ? M * DSUB : 0;
    float cvr[CPER - CHALF][CPL];
#pragma unroll
    for (int k = 0; k < CPER - CHALF; ++k) {
        const int c = ec0 + CHALF + k < K ? ec0 + CHALF + k : K - 1;
        load_f32x<CPL>(cbv + (int64_t)c * vstride, cvr[k]);
    }
    float vpre[kRecentPre][CPL];  // recent value rows of this wave's first recent tokens
#pragma unroll
    for (int p = 0; p < kRecentPre; ++p) {
        const int i = wave + p * kWaves;
        const RT* row = i < n_rec ? rv + (int64_t)i * D + em * DSUB + ecomp : rzero;
#pragma unroll
        for (int t = 0; t < CPL; ++t) vpre[p][t] = to_f32(row[i < n_rec ? t : 0]);
    }
    // byte s of mw[k] = CS * ((4k + s + slot) mod M): subspace byte offsets
    uint32_t mw[M / 4];
#pragma unroll
    for (int k = 0; k < M / 4; ++k) {
        uint32_t w = 0;
#pragma unroll
        for (int s = 0; s < 4; ++s) w |= (uint32_t)(((4 * k + s + lane) & (M - 1)) * CS) << (8 * s);
        mw[k] = w;
    }
    uint32_t lsum[QH];
#pragma unroll
    for (int j = 0; j < QH; ++j) lsum[j] = 0u;
#pragma unroll
    for (int s = RW; s < 2 * RW; ++s) {
        set_prio(3 - (4 * (s - RW)) / RW);
        if (s == RW + RW / 2) stamp(13);  // half of phase 2
        if (s + P < 2 * RW) issue(ring[(s + P) % NSLOT], s + P);  // nothing is left to request at the end
        if (step_ok(s) && step_tile(s) * kTileTokens + lane < t1) {
            const u32x4(&cw)[NCH] = ring[s % NSLOT];
            tile_ready(s, cw);
            uint32_t p[QH];
#pragma unroll
            for (int j = 0; j < QH; ++j) {
                p[j] = __float2uint_rn(exp2f(sc[s - RW][j] - mx[j]) * fs[j]);
                lsum[j] += p[j];
            }
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const uint32_t words[4] = {cw[c].x, cw[c].y, cw[c].z, cw[c].w};
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t mwv = mw[c * 4 + w];
                    const uint32_t a0 = hist_addr<0>(words[w], mwv);
                    const uint32_t a1 = hist_addr<1>(words[w], mwv);
                    const uint32_t a2 = hist_addr<2>(words[w], mwv);
                    const uint32_t a3 = hist_addr<3>(words[w], mwv);
                    if constexpr (QH == 1) {
                        lds_add_u32(lds, a0, p[0]);
                        lds_add_u32(lds, a1, p[0]);
                        lds_add_u32(lds, a2, p[0]);
                        lds_add_u32(lds, a3, p[0]);
                    } else {
#pragma unroll
                        for (int jp = 0; jp < QH; jp += 2) {  // two heads per add
                            lds_add_u32x2(lds + jp, a0, p[jp], p[jp + 1]);
                            lds_add_u32x2(lds + jp, a1, p[jp], p[jp + 1]);
                            lds_add_u32x2(lds + jp, a2, p[jp], p[jp + 1]);
                            lds_add_u32x2(lds + jp, a3, p[jp], p[jp + 1]);
                        }
                    }
                }
            }
        }
    }
    stamp(6);  // phase 2 ends
    set_prio(0);
    // recent weights, scaled by 2^S like the histogram
#pragma unroll
    for (int j = 0; j < QH; ++j) {
        float l = 0.0f;
        for (int i = tid; i < n_rec; i += kThreads) {
            const float p = exp2f(rs[j * RS + i] - mx[j]) * fs[j];
            rs[j * RS + i] = p;
            l += p;
        }
        l = wave_sum(l);
        const uint32_t lh = wave_sum_u32(lsum[j]);
        if (lane == 0) {
            redr[wave * QH + j] = l;
            redu[wave * QH + j] = lh;
        }
    }
    __syncthreads();
    stamp(7);  // the histogram is complete

    // ---- 6. output partial: histogram x value codebook + recent weights x values
    // partial records: one per (item, query head of the group), item = item_first + split
    float* part = a.partials + ((int64_t)(item_first + split) * QH) * a.pstride;
    const int64_t head_step = a.pstride;
    {
        float acc[QH][CPL];
#pragma unroll
        for (int j = 0; j < QH; ++j)
#pragma unroll
            for (int i = 0; i < CPL; ++i) acc[j][i] = 0.0f;
        if (any) {
            if (has_hist) {
                // the staged value-codebook rows must have landed in LDS (the
                // direct-to-LDS loads are not tracked by the compiler's waits)
                __builtin_amdgcn_s_waitcnt(0);
                __builtin_amdgcn_sched_barrier(0);
                // histogram reads in groups of 8, so the LDS latency is paid once per group
                // (rows past K hold 0 and meet zero or finite value rows)
#pragma unroll
                for (int k0 = 0; k0 < CPER; k0 += 8) {
                    uint32_t hv[8][QH];
                    float cv[8][CPL];
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        const int c = ec0 + k0 + k;
#pragma unroll
                        for (int j = 0; j < QH; ++j) hv[k][j] = hist[c * kRow + em * QH + j];
#pragma unroll
                        for (int i = 0; i < CPL; ++i)
                            cv[k][i] = k0 + k < CHALF ? cv_lds[(k0 + k) * D + em * DSUB + ecomp + i]
                                                      : cvr[k0 + k - CHALF < 0 ? 0 : k0 + k - CHALF][i];
                    }
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
#pragma unroll
                        for (int j = 0; j < QH; ++j) {
                            const float w = (float)hv[k][j];
#pragma unroll
                            for (int i = 0; i < CPL; ++i) acc[j][i] = fmaf(w, cv[k][i], acc[j][i]);
                        }
                    }
                }
            }
            for (int i = wave, pidx = 0; i < n_rec; i += kWaves, ++pidx) {
                float v[CPL];
                if (pidx < kRecentPre) {
#pragma unroll
                    for (int q = 0; q < kRecentPre; ++q)
                        if (q == pidx)
#pragma unroll
                            for (int t = 0; t < CPL; ++t) v[t] = vpre[q][t];
                } else {
                    const RT* vr = rv + (int64_t)i * D + em * DSUB + ecomp;
#pragma unroll
                    for (int t = 0; t < CPL; ++t) v[t] = to_f32(vr[t]);
                }
#pragma unroll
                for (int j = 0; j < QH; ++j) {
                    const float p = rs[j * RS + i];
#pragma unroll
                    for (int t = 0; t < CPL; ++t) acc[j][t] = fmaf(p, v[t], acc[j][t]);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < QH; ++j)
#pragma unroll
            for (int i = 0; i < CPL; ++i) ored[(wave * QH + j) * D + em * DSUB + ecomp + i] = acc[j][i];
    }
    stamp(8);  // epilogue done
    __syncthreads();
    if (ns == 1) {
        // The unit's only split: it normalises its own output, with no partial
        // round trip.  The result is the one the merge gives for a single split
        // (the fixed-point scale cancels exactly, being a power of two).
        if (tid < QH) {
            uint32_t lh = 0u;
            float lr = 0.0f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                lh += redu[w * QH + tid];
                lr += redr[w * QH + tid];
            }
            lfin[tid] = (float)lh + lr;
        }
        __syncthreads();
        for (int e = tid; e < QH * D; e += kThreads) {
            float s = 0.0f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) s += ored[w * QH * D + e];
            const int j = e / D;
            const int el = e - j * D;
            float m = mx[0], inv = fi[0];
#pragma unroll
            for (int q = 1; q < QH; ++q) {
                m = j == q ? mx[q] : m;
                inv = j == q ? fi[q] : inv;
            }
            const int64_t orow = (int64_t)(b * a.Hq + hq0 + j);
            a.out[orow * D + el] = any ? (s * inv) / (lfin[j] * inv) : 0.0f;
            if (el == 0) a.lse[orow] = any ? (m + log2f(lfin[j] * inv)) * kLn2 : -INFINITY;
        }
        return;
    }
    // Partials are published with agent-scope stores, which write through the
    // XCD-private L2, so the merging work-group on another XCD reads them from memory.
    for (int e = tid; e < QH * D; e += kThreads) {
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) s += ored[w * QH * D + e];
        const int j = e / D;
        float inv = fi[0];
#pragma unroll
        for (int q = 1; q < QH; ++q) inv = j == q ? fi[q] : inv;
        publish(part + j * head_step + (e - j * D), s * inv);
    }
    if (tid < QH) {
        uint32_t lh = 0u;
        float lr = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            lh += redu[w * QH + tid];
            lr += redr[w * QH + tid];
        }
        float m = mx[0], inv = fi[0];
#pragma unroll
        for (int q = 1; q < QH; ++q) {
            m = tid == q ? mx[q] : m;
            inv = tid == q ? fi[q] : inv;
        }
        publish(part + tid * head_step + D, any ? m : -INFINITY);
        publish(part + tid * head_step + D + 1, ((float)lh + lr) * inv);
    }

    // ---- 7. the last work-group of this unit merges every split's partial.
    // Every wave waits for its stores to complete before the barrier; the counter
    // increment that follows is therefore ordered after all of them.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    stamp(9);  // partial published
    if (tid == 0) {
        const uint32_t done = __hip_atomic_fetch_add(a.counters + unit, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last_flag = (done == (uint32_t)(ns - 1));
    }
    __syncthreads();
    stamp(10);  // counter returned
    if (!last_flag) return;
    // Every output element reads (max, sum, value) of eight splits at a time --
    // all loads in flight together -- and folds them in with a running max.
    const float* prow0 = a.partials + (int64_t)item_first * QH * a.pstride;
    for (int e = tid; e < QH * D; e += kThreads) {
        const int j = e / D;
        const int el = e - j * D;
        const float* prow = prow0 + j * head_step;
        float mall = -INFINITY, l = 0.0f, o = 0.0f;
        for (int s0 = 0; s0 < ns; s0 += 8) {
            float pm[8], pl[8], po[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int sp = s0 + u < ns ? s0 + u : ns - 1;
                const float* ps = prow + (int64_t)sp * QH * a.pstride;
                pm[u] = collect(ps + D);
                pl[u] = collect(ps + D + 1);
                po[u] = collect(ps + el);
            }
            float cm = -INFINITY;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (s0 + u < ns) cm = fmaxf(cm, pm[u]);
            if (cm == -INFINITY) continue;
            const float mnew = fmaxf(mall, cm);
            const float r = exp2f(mall - mnew);  // 0 while nothing has been folded in
            l *= r;
            o *= r;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (s0 + u < ns && pm[u] != -INFINITY) {
                    const float wgt = exp2f(pm[u] - mnew);
                    l = fmaf(wgt, pl[u], l);
                    o = fmaf(wgt, po[u], o);
                }
            }
            mall = mnew;
        }
        const int64_t orow = (int64_t)(b * a.Hq + hq0 + j);
        if (mall == -INFINITY) {
            a.out[orow * D + el] = 0.0f;
            if (el == 0) a.lse[orow] = -INFINITY;
            continue;
        }
        a.out[orow * D + el] = o / l;
        if (el == 0) a.lse[orow] = (mall + log2f(l)) * kLn2;
    }
    if (tid == 0) __hip_atomic_store(a.counters + unit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    stamp(11);  // merge done
}

template <int M, int DSUB, int QH, int RW, bool EXT, typename QT, typename RT>
hipError_t launch_typed(const pqkv_dims& d, int32_t batch, const DecodePlan& plan, const DecodeArgs& in,
                        hipStream_t stream) {
    if (plan.rounds > RW) return hipErrorInvalidValue;  // the build must unroll every round
    DecArgs k;
    k.q = in.q;
    k.lut = in.lut;
    k.cb_k = in.cb_k;
    k.cb_v = in.cb_v;
    k.codes_k = in.codes_k;
    k.codes_v = in.codes_v;
    k.t_cap = in.t_cap;
    k.hist_len = in.hist_len;
    k.max_hist = in.max_hist;
    k.rk = in.rk;
    k.rv = in.rv;
    k.r_cap = in.r_cap;
    k.recent_len = in.recent_len;
    k.scale_log2 = in.scale_log2;
    k.partials = in.partials;
    k.counters = in.counters;
    k.out = in.out;
    k.lse = in.lse;
    k.K = d.n_centroids;
    k.Hq = d.n_q_heads;
    k.Hkv = d.n_kv_heads;
    k.n_groups = plan.n_groups;
    k.n_split = plan.n_split;
    k.len_first = batch == 1 ? 0 : (batch <= kDevicePlanMaxBatch && in.max_hist > 0 ? 2 : 1);
    k.rounds = plan.rounds;
    k.pstride = plan.partial_stride;
    k.split_tokens = plan.split_tokens;
    const int64_t items = (int64_t)batch * d.n_kv_heads * plan.n_groups * plan.n_split;
    k.n_items = (int)items;
    hipLaunchKernelGGL((pq_decode_kernel<M, DSUB, QH, RW, EXT, QT, RT>), dim3((unsigned)items), dim3(kThreads), 0,
                       stream, k);
    return hipGetLastError();
}

// The build that holds the plan's rounds (decode_kernel_rounds).
template <int M, int DSUB, int QH, bool EXT, typename QT, typename RT>
hipError_t launch_rw(const pqkv_dims& d, int32_t batch, const DecodePlan& plan, const DecodeArgs& a,
                     hipStream_t stream) {
    const int rw = decode_kernel_rounds(M, QH, plan.rounds);
    if constexpr (M == 64) {
        if (rw == 2) return launch_typed<M, DSUB, QH, 2, EXT, QT, RT>(d, batch, plan, a, stream);
        if (rw == 8) return launch_typed<M, DSUB, QH, 8, EXT, QT, RT>(d, batch, plan, a, stream);
        if (rw == 12) return launch_typed<M, DSUB, QH, 12, EXT, QT, RT>(d, batch, plan, a, stream);
    }
    if (rw == 4) return launch_typed<M, DSUB, QH, 4, EXT, QT, RT>(d, batch, plan, a, stream);
    return launch_typed<M, DSUB, QH, decode_max_rounds(M, QH), EXT, QT, RT>(d, batch, plan, a, stream);
}

// Every kernel build of one (subspace count, subspace dimension, table source):
// query-head groups, round counts and the q / recent-window element types.
template <int M, int DSUB, bool EXT>
hipError_t launch_family(const pqkv_dims& d, int32_t batch, pqkv_dtype qt, pqkv_dtype rt, const DecodePlan& plan,
                         const DecodeArgs& a, hipStream_t stream) {
    auto qh = [&](auto q_tag, auto r_tag) -> hipError_t {
        using QT = decltype(q_tag);
        using RT = decltype(r_tag);
        if constexpr (M <= 16) {
            if (plan.qh == 4) return launch_rw<M, DSUB, 4, EXT, QT, RT>(d, batch, plan, a, stream);
        }
        if constexpr (M <= 32) {
            if (plan.qh == 2) return launch_rw<M, DSUB, 2, EXT, QT, RT>(d, batch, plan, a, stream);
        }
        return launch_rw<M, DSUB, 1, EXT, QT, RT>(d, batch, plan, a, stream);
    };
    if (qt == PQKV_F16) return rt == PQKV_F16 ? qh(__half(), __half()) : qh(__half(), 0.0f);
    return rt == PQKV_F16 ? qh(0.0f, __half()) : qh(0.0f, 0.0f);
}

}  // namespace
}  // namespace pqkv
