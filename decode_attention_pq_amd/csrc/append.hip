// pqkv_append_kv: a decode step's new key/value enters the full-precision recent
// window; a window that is full first rolls its oldest tokens into the PQ history.
//
// MILLION write-up (DAC 2025), page "MILLION", Fig. 7 paragraph: the tokens a
// decode generates are kept apart from the quantised history, in full precision,
// and are quantised later in batches, so quantisation stays off the per-token
// path.  Rolling n_roll tokens at once is that batched, delayed quantisation; the
// codes are the nearest-centroid codes of pqkv_encode.
//
// Work decomposition: one work-group per (kv head, sequence, tensor K or V).
// Every work-group reads the old lengths; the (h = 0, K) work-group of a sequence
// writes the new ones to separate arrays, so no work-group can see a length that
// another has already advanced.  A rolling work-group stages its head's codebook
// in LDS, encodes one rolled token per thread, then moves the remaining rows down
// in chunks of at most n_roll rows with a barrier after each chunk (a chunk
// writes only rows that earlier chunks have finished reading), then writes the
// new row.

#include "nearest.h"

namespace pqkv {
namespace {

constexpr int kAppThreads = 512;

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

template <int D, int DSUB, typename RT>
__global__ __launch_bounds__(kAppThreads) void append_kernel(AppendArgs a) {
    constexpr int M = D / DSUB;
    constexpr int U = D * (int)sizeof(RT) / 16;  // 16-byte units per row
    __shared__ float4 cbs4[kLdsRows * D / 4];
    const float* cbs = reinterpret_cast<const float*>(cbs4);

    const int h = blockIdx.x;
    const int b = blockIdx.y;
    const int tensor = blockIdx.z;  // 0 = K, 1 = V
    const int tid = threadIdx.x;

    int64_t T = a.hist_in[b];
    int64_t R = a.recent_in[b];
    const int n_roll = a.n_roll;
    const bool ok = T >= 0 && R >= 0 && R <= a.r_cap && (R < a.r_cap || T + n_roll <= a.t_cap);
    if (!ok) {
        if (h == 0 && tensor == 0 && tid == 0) {
            a.hist_out[b] = (int32_t)T;
            a.recent_out[b] = (int32_t)R;
        }
        return;
    }

    RT* rows = static_cast<RT*>(tensor ? a.rv : a.rk) + ((int64_t)b * a.Hkv + h) * a.r_cap * D;
    if (R == a.r_cap) {
        // roll: encode rows 0..n_roll-1 into history positions T..T+n_roll-1
        const float* cb = (tensor ? a.cb_v : a.cb_k) + (int64_t)h * a.K * D;
        const float4* src = reinterpret_cast<const float4*>(cb);
        for (int i = tid; i < a.K * D / 4; i += kAppThreads) cbs4[i] = src[i];
        __syncthreads();
        uint8_t* plane = (tensor ? a.codes_v : a.codes_k) + ((int64_t)b * a.Hkv + h) * a.t_cap * M;
        if (tid < n_roll) {
            float xv[D];
            Row<RT>::template load<D>(rows + (int64_t)tid * D, xv);
            const int64_t t = T + tid;
            write_nearest_codes<D, DSUB>(xv, cbs, a.K, code_slot<M>(plane, t), (int)(t & (kTileTokens - 1)));
        }
        __syncthreads();  // every rolled row has been read
        // move rows n_roll..R-1 down to 0..R-n_roll-1
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
    dim3 grid((unsigned)a.Hkv, (unsigned)batch, 2u);
    hipLaunchKernelGGL((append_kernel<D, DSUB, RT>), grid, dim3(kAppThreads), 0, stream, a);
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
