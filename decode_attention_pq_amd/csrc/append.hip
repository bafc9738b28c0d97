// pqkv_append_kv: a decode step's new key/value enters the full-precision recent
// window; a window that is full first rolls its oldest tokens into the PQ history.
//
// MILLION write-up (DAC 2025), page "MILLION", Fig. 7 paragraph: the tokens a
// decode generates are kept apart from the quantised history, in full precision,
// and are quantised later in batches, so quantisation stays off the per-token
// path.  Rolling n_roll tokens at once is that batched, delayed quantisation; the
// codes are the nearest-centroid codes of pqkv_encode.
//
// Work decomposition: two kernels on the caller's stream.
//   roll_kernel    one work-group of 8 waves per (64 rolled rows, kv head, sequence and
//                  tensor): work-groups of sequences whose window is not full return at
//                  once; the others stage the head's codebook in LDS and encode, wave w
//                  taking subspaces [w*M/8, (w+1)*M/8) of the 64 rows (one row per lane).
//   append_kernel  one work-group per (kv head, sequence, tensor): after the encode
//                  has read them (stream order), the remaining rows of a full window
//                  move down in chunks of at most n_roll rows with a barrier after each
//                  chunk (a chunk writes only rows that earlier chunks have finished
//                  reading), then the new row is written.  The (h = 0, K) work-group of a
//                  sequence writes its new lengths to separate arrays, so no work-group
//                  can see a length that another has already advanced.

#include "nearest.h"

namespace pqkv {
namespace {

constexpr int kAppThreads = 512;
constexpr int kAppWaves = kAppThreads / 64;
constexpr int kRollSubspaces = 16;  // subspaces one roll work-group encodes (2 per wave)

__device__ inline float to_float(float v) { return v; }
__device__ inline float to_float(__half v) { return __half2float(v); }

struct AppendArgs {
    const void* new_k;
    const void* new_v;
    void* rk;
    void* rv;
    int64_t r_cap;
    const int32_t* hist_in;
    const int32_t* recent_in;
    int32_t* hist_out;
    int32_t* recent_out;
    int32_t n_roll;
    const float* cb_k;
    const float* cb_v;
    uint8_t* codes_k;
    uint8_t* codes_v;
    int64_t t_cap;
    int K, Hkv;
};

// The window of sequence b rolls in this call, and where its history goes.
__device__ inline bool roll_ok(const AppendArgs& a, int64_t T, int64_t R, bool& rolls) {
    const bool ok = T >= 0 && R >= 0 && R <= a.r_cap && (R < a.r_cap || T + a.n_roll <= a.t_cap);
    rolls = ok && R == a.r_cap;
    return ok;
}

template <int D, int DSUB, typename RT>
__global__ __launch_bounds__(kAppThreads) void roll_kernel(AppendArgs a) {
    constexpr int M = D / DSUB;
    constexpr int SW = kRollSubspaces;       // subspaces per work-group
    constexpr int MW = SW / kAppWaves;       // subspaces per wave
    constexpr int CS = SW * DSUB;            // floats per staged centroid row
    static_assert(M % SW == 0 && SW % kAppWaves == 0, "roll subspace split");
    // floats after every 16 centroid rows: sub-block b of the rescan starts on bank
    // PAD*b mod 32, which tiles the 32 banks with the 8-byte reads of d_sub 2 at 2
    constexpr int PAD = DSUB == 2 ? 2 : 4;
    __shared__ __align__(16) float cbs[kLdsRows * CS + kLdsRows / 16 * PAD];
    const int g = blockIdx.x % (M / SW);     // subspace group
    const int rb = blockIdx.x / (M / SW);    // block of 64 rolled rows
    const int h = blockIdx.y;
    const int b = blockIdx.z >> 1;
    const int tensor = blockIdx.z & 1;       // 0 = K, 1 = V
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int64_t T = a.hist_in[b];
    const int64_t R = a.recent_in[b];
    bool rolls;
    if (!roll_ok(a, T, R, rolls) || !rolls) return;

    // stage subspaces [g*SW, g*SW + SW) of every centroid: CS contiguous floats per row
    const float* cb = (tensor ? a.cb_v : a.cb_k) + (int64_t)h * a.K * D + g * CS;
    for (int i = tid; i < a.K * CS; i += kAppThreads) cbs[i + i / (16 * CS) * PAD] = cb[(i / CS) * D + i % CS];
    __syncthreads();
    const int row = rb * 64 + lane;
    if (row < a.n_roll) {
        const RT* rows = static_cast<const RT*>(tensor ? a.rv : a.rk) + ((int64_t)b * a.Hkv + h) * a.r_cap * D;
        const int m0 = g * SW + wave * MW;
        float xv[MW * DSUB];
#pragma unroll
        for (int j = 0; j < MW * DSUB; ++j) xv[j] = to_float(rows[(int64_t)row * D + m0 * DSUB + j]);
        uint8_t* plane = (tensor ? a.codes_v : a.codes_k) + ((int64_t)b * a.Hkv + h) * a.t_cap * M;
        const int64_t t = T + row;
        write_nearest_codes_slice<D, DSUB, MW, CS, PAD>(xv, cbs + wave * MW * DSUB, a.K, code_slot<M>(plane, t),
                                                   (int)(t & (kTileTokens - 1)), m0);
    }
}

template <int D, typename RT>
__global__ __launch_bounds__(kAppThreads) void append_kernel(AppendArgs a) {
    constexpr int U = D * (int)sizeof(RT) / 16;  // 16-byte units per row
    const int h = blockIdx.x;
    const int b = blockIdx.y;
    const int tensor = blockIdx.z;  // 0 = K, 1 = V
    const int tid = threadIdx.x;
    int64_t T = a.hist_in[b];
    int64_t R = a.recent_in[b];
    const int n_roll = a.n_roll;
    bool rolls;
    if (!roll_ok(a, T, R, rolls)) {
        if (h == 0 && tensor == 0 && tid == 0) {
            a.hist_out[b] = (int32_t)T;
            a.recent_out[b] = (int32_t)R;
        }
        return;
    }
    RT* rows = static_cast<RT*>(tensor ? a.rv : a.rk) + ((int64_t)b * a.Hkv + h) * a.r_cap * D;
    if (rolls) {
        // move rows n_roll..R-1 down to 0..R-n_roll-1 (the roll kernel, earlier on the
        // stream, has read rows 0..n_roll-1)
        uint4* r4 = reinterpret_cast<uint4*>(rows);
        const int64_t left = R - n_roll;
        const int chunk = n_roll < kAppThreads / U ? n_roll : kAppThreads / U;
        for (int64_t base = 0; base < left; base += chunk) {
            const int64_t rows_here = left - base < chunk ? left - base : chunk;
            uint4 v;
            const bool mine = tid < rows_here * U;
            if (mine) v = r4[(base + n_roll) * U + tid];
            if (mine) r4[base * U + tid] = v;
            __syncthreads();
        }
        T += n_roll;
        R -= n_roll;
    }
    // append the new row at R
    const RT* nr = static_cast<const RT*>(tensor ? a.new_v : a.new_k) + ((int64_t)b * a.Hkv + h) * D;
    if (tid < U)
        reinterpret_cast<uint4*>(rows + R * D)[tid] = reinterpret_cast<const uint4*>(nr)[tid];
    if (h == 0 && tensor == 0 && tid == 0) {
        a.hist_out[b] = (int32_t)T;
        a.recent_out[b] = (int32_t)(R + 1);
    }
}

template <int D, int DSUB, typename RT>
hipError_t launch_typed(int32_t batch, const AppendArgs& a, hipStream_t stream) {
    dim3 rgrid((unsigned)((a.n_roll + 63) / 64 * (D / DSUB / kRollSubspaces)), (unsigned)a.Hkv,
               (unsigned)batch * 2u);
    hipLaunchKernelGGL((roll_kernel<D, DSUB, RT>), rgrid, dim3(kAppThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid((unsigned)a.Hkv, (unsigned)batch, 2u);
    hipLaunchKernelGGL((append_kernel<D, RT>), grid, dim3(kAppThreads), 0, stream, a);
    return hipGetLastError();
}

template <int D, int DSUB>
hipError_t launch_dsub(int32_t batch, pqkv_dtype rt, const AppendArgs& a, hipStream_t stream) {
    if (rt == PQKV_F16) return launch_typed<D, DSUB, __half>(batch, a, stream);
    return launch_typed<D, DSUB, float>(batch, a, stream);
}

}  // namespace

hipError_t launch_append(const pqkv_dims& d, int32_t batch, const void* new_k, const void* new_v,
                         void* recent_k, void* recent_v, pqkv_dtype rt, int64_t r_cap,
                         const int32_t* hist_in, const int32_t* recent_in, int32_t* hist_out,
                         int32_t* recent_out, int32_t n_roll, const float* cb_k, const float* cb_v,
                         uint8_t* codes_k, uint8_t* codes_v, int64_t t_cap, hipStream_t stream) {
    AppendArgs a{new_k,   new_v,      recent_k, recent_v, r_cap, hist_in, recent_in,
                 hist_out, recent_out, n_roll,   cb_k,     cb_v,  codes_k, codes_v,
                 t_cap,   d.n_centroids, d.n_kv_heads};
    if (d.head_dim == 128 && d.d_sub == 2) return launch_dsub<128, 2>(batch, rt, a, stream);
    if (d.head_dim == 128 && d.d_sub == 4) return launch_dsub<128, 4>(batch, rt, a, stream);
    if (d.head_dim == 64 && d.d_sub == 2) return launch_dsub<64, 2>(batch, rt, a, stream);
    return launch_dsub<64, 4>(batch, rt, a, stream);
}

}  // namespace pqkv
