// Small kernels: the standalone ad-LUT and the two-state log-sum-exp merge.
//
// MILLION write-up (DAC 2025), page "MILLION", Fig. 7 paragraph: the query x
// codebook asymmetric-distance table, and the combination of separately
// computed attention blocks.

#include <hip/hip_fp16.h>

#include "pqkv_internal.h"

namespace pqkv {
namespace {

__device__ inline float to_f32(float v) { return v; }
__device__ inline float to_f32(__half v) { return __half2float(v); }

// ----------------------------------------------------------------------------
// Standalone ad-LUT: lut[b][hq][m][c] = q_m . C_K[h][c][m] (unscaled).
template <int DSUB, typename QT>
__global__ __launch_bounds__(256) void lut_kernel(const QT* __restrict__ q, const float* __restrict__ cb,
                                                  float* __restrict__ lut, int D, int K, int Hq, int Hkv) {
    __shared__ float qs[128];
    const int row = blockIdx.x;
    const int hq = row % Hq;
    const int h = hq / (Hq / Hkv);
    const int M = D / DSUB;
    for (int e = threadIdx.x; e < D; e += 256) qs[e] = to_f32(q[(int64_t)row * D + e]);
    __syncthreads();
    const float* cbh = cb + (int64_t)h * K * M * DSUB;
    float* dst = lut + (int64_t)row * M * K;
    for (int e = threadIdx.x; e < M * K; e += 256) {
        const int m = e / K;
        const int c = e % K;
        const float* cc = cbh + ((int64_t)c * M + m) * DSUB;
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < DSUB; ++i) s = fmaf(qs[m * DSUB + i], cc[i], s);
        dst[e] = s;
    }
}

// ----------------------------------------------------------------------------
// Merge two normalised attention states, one wave per row.
__global__ __launch_bounds__(256) void merge_states_kernel(int64_t n_rows, int d, const float* out_a,
                                                           const float* lse_a, const float* out_b,
                                                           const float* lse_b, float* out, float* lse) {
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= n_rows) return;
    const float la = lse_a[row];
    const float lb = lse_b[row];
    const float mu = fmaxf(la, lb);
    float wa = 0.0f, wb = 0.0f, lo = -INFINITY;
    if (mu != -INFINITY) {
        wa = la == -INFINITY ? 0.0f : expf(la - mu);
        wb = lb == -INFINITY ? 0.0f : expf(lb - mu);
        const float den = wa + wb;
        lo = mu + logf(den);
        wa /= den;
        wb /= den;
    }
    const float* ra = out_a + row * d;
    const float* rb = out_b + row * d;
    float* ro = out + row * d;
    for (int e = lane; e < d; e += 64) {
        const float va = ra[e];
        const float vb = rb[e];
        ro[e] = (mu == -INFINITY) ? 0.0f : wa * va + wb * vb;
    }
    if (lane == 0) lse[row] = lo;
}

}  // namespace

hipError_t launch_build_lut(const pqkv_dims& d, int32_t batch, const void* q, pqkv_dtype qt,
                            const float* cb, float* lut, hipStream_t stream) {
    const dim3 grid((unsigned)(batch * d.n_q_heads));
    if (d.d_sub == 2) {
        if (qt == PQKV_F16)
            hipLaunchKernelGGL((lut_kernel<2, __half>), grid, dim3(256), 0, stream,
                               static_cast<const __half*>(q), cb, lut, d.head_dim, d.n_centroids,
                               d.n_q_heads, d.n_kv_heads);
        else
            hipLaunchKernelGGL((lut_kernel<2, float>), grid, dim3(256), 0, stream,
                               static_cast<const float*>(q), cb, lut, d.head_dim, d.n_centroids,
                               d.n_q_heads, d.n_kv_heads);
    } else {
        if (qt == PQKV_F16)
            hipLaunchKernelGGL((lut_kernel<4, __half>), grid, dim3(256), 0, stream,
                               static_cast<const __half*>(q), cb, lut, d.head_dim, d.n_centroids,
                               d.n_q_heads, d.n_kv_heads);
        else
            hipLaunchKernelGGL((lut_kernel<4, float>), grid, dim3(256), 0, stream,
                               static_cast<const float*>(q), cb, lut, d.head_dim, d.n_centroids,
                               d.n_q_heads, d.n_kv_heads);
    }
    return hipGetLastError();
}

hipError_t launch_merge_states(int64_t n_rows, int32_t head_dim, const float* out_a,
                               const float* lse_a, const float* out_b, const float* lse_b,
                               float* out, float* lse, hipStream_t stream) {
    const unsigned blocks = (unsigned)((n_rows + 3) / 4);
    hipLaunchKernelGGL(merge_states_kernel, dim3(blocks), dim3(256), 0, stream, n_rows, head_dim, out_a,
                       lse_a, out_b, lse_b, out, lse);
    return hipGetLastError();
}

}  // namespace pqkv
