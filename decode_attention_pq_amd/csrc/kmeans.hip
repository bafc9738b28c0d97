// pqkv_fit_codebooks: Lloyd k-means of every (kv head, subspace) codebook of one
// tensor, on the GPU.
//
// MILLION write-up (DAC 2025), page "MILLION": the Fig. 5 paragraph clusters the
// fused channels with k-means; the paragraph after it splits the head vector into
// subspaces of dimension 2 or 4, one codebook per subspace; the Fig. 6 paragraph
// trains the codebooks offline on calibration data.
//
// Per (head, subspace) problem, one work-group of 256 threads:
//   1. the problem's n subvectors are staged in LDS (fp32 holds fp16/fp32 inputs
//      exactly);
//   2. initialisation: walk the given permutation and keep each point that is not
//      equal to one already kept, until K are kept (one wave; every candidate is
//      compared against the kept ones across the lanes, then a ballot); if fewer
//      than K distinct points exist, the remaining slots copy slot 0;
//   3. `iters` Lloyd iterations: every point takes its nearest centroid (squared
//      distance, strict '<' in ascending centroid order, so the lowest index wins
//      ties), then thread c moves centroid c to the mean of its members, summing
//      them in point order; an empty cluster keeps its centroid.  While assigning,
//      each point also sets its 32-point block's bit in its centroid's block mask,
//      so thread c scans only the blocks that hold members of c (in ascending
//      order, which keeps the point order of the sums).
// Arithmetic is fp64 with every product and sum rounded on its own (no fused
// multiply-add), so distances, sums and means are the IEEE results of the plain
// definition, whatever the thread count.

#include "pqkv_internal.h"

#include <hip/hip_fp16.h>

namespace pqkv {
namespace {

constexpr int kKmThreads = 256;
constexpr int kBlkPts = 32;                                   // points per mask bit
constexpr int kMaskWords = (PQKV_MAX_FIT_POINTS + kBlkPts * 32 - 1) / (kBlkPts * 32);  // per centroid

template <typename XT>
__device__ inline float elem(const XT* p) {
    if constexpr (sizeof(XT) == 2)
        return __half2float(*reinterpret_cast<const __half*>(p));
    else
        return *reinterpret_cast<const float*>(p);
}

// Nearest centroid of a point (its fp32 values widened to fp64), by the plain
// scan's rule: the running minimum starts at centroid 0 and moves only on a
// strictly smaller distance, so the first minimum wins and NaN distances never win.  With
// K a multiple of 16 the scan runs in unrolled blocks of 16 whose running index is
// the block-relative position (an inline constant of the select); block 0 starts
// from centroid 0's distance like the plain scan, later blocks from +inf, and a
// block's winner replaces the running one only if strictly smaller, which picks
// the same centroid as the plain scan.
template <int DSUB>
__device__ __forceinline__ double sqdist_d(const double (&x)[DSUB], const double* c) {
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < DSUB; ++j) {
        const double t = __dsub_rn(x[j], c[j]);
        s = __dadd_rn(s, __dmul_rn(t, t));
    }
    return s;
}

template <int DSUB>
__device__ __forceinline__ int nearest_centroid(const double (&x)[DSUB], const double* C, int K) {
    constexpr int BS = 16;  // centroids per unrolled block
    if ((K & (BS - 1)) == 0) {
        double best = 0.0;
        int bi = 0;
        for (int c0 = 0; c0 < K; c0 += BS) {
            // block 0 starts from centroid 0's distance (which then never moves it)
            double bb = c0 == 0 ? sqdist_d<DSUB>(x, C) : INFINITY;
            int br = 0;
            double cv[BS][DSUB];
#pragma unroll
            for (int r = 0; r < BS; ++r)
#pragma unroll
                for (int j = 0; j < DSUB; ++j) cv[r][j] = C[(c0 + r) * DSUB + j];
#pragma unroll
            for (int r = 0; r < BS; ++r) {
                const double dc = sqdist_d<DSUB>(x, cv[r]);
                if (dc < bb) {
                    bb = dc;
                    br = r;
                }
            }
            if (c0 == 0 || bb < best) {
                best = bb;
                bi = c0 + br;
            }
        }
        return bi;
    }
    int best = 0;
    double bd = sqdist_d<DSUB>(x, C);
    for (int c = 1; c < K; ++c) {
        const double dc = sqdist_d<DSUB>(x, C + c * DSUB);
        if (dc < bd) {
            bd = dc;
            best = c;
        }
    }
    return best;
}

struct KmArgs {
    const void* x;
    int64_t n, s_tok, s_head;
    const int32_t* order;
    int iters, K, M, Hkv;
    float* cb;
    int32_t* kept;
};

template <int DSUB, typename XT>
__global__ __launch_bounds__(kKmThreads) void kmeans_kernel(KmArgs a) {
    extern __shared__ float dyn[];
    __shared__ double C[kLdsRows * DSUB];
    __shared__ int kept_s;
    __shared__ uint32_t bmask[kLdsRows * kMaskWords];  // centroid c's blocks: bmask[c * kMaskWords ...]
    const int m = blockIdx.x;
    const int h = blockIdx.y;
    const int tid = threadIdx.x;
    const int64_t n = a.n;
    const int K = a.K;
    float* pts = dyn;                                                   // [n][DSUB]
    uint8_t* asg = reinterpret_cast<uint8_t*>(dyn + n * DSUB);          // [n]

    const XT* x = static_cast<const XT*>(a.x) + h * a.s_head + m * DSUB;
    for (int64_t i = tid; i < n; i += kKmThreads)
#pragma unroll
        for (int j = 0; j < DSUB; ++j) pts[i * DSUB + j] = elem(x + i * a.s_tok + j);
    __syncthreads();

    // ---- initialisation (wave 0)
    if (tid < 64) {
        const int32_t* ord = a.order + ((int64_t)h * a.M + m) * n;
        int kept = 0;
        for (int64_t i = 0; i < n && kept < K; ++i) {
            const int32_t pi = ord[i];
            if (pi < 0 || pi >= n) continue;  // not a point index
            const float* p = pts + (int64_t)pi * DSUB;
            bool dup = false;
            for (int k = tid; k < kept; k += 64) {
                bool same = true;
#pragma unroll
                for (int j = 0; j < DSUB; ++j) same = same && C[k * DSUB + j] == (double)p[j];
                dup = dup || same;
            }
            if (!__any(dup)) {
                if (tid == 0)
#pragma unroll
                    for (int j = 0; j < DSUB; ++j) C[kept * DSUB + j] = (double)p[j];
                ++kept;
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
            }
        }
        if (tid == 0) kept_s = kept;
    }
    __syncthreads();
    const int kept = kept_s;
    for (int k = kept + tid; k < K; k += kKmThreads)
#pragma unroll
        for (int j = 0; j < DSUB; ++j) C[k * DSUB + j] = kept > 0 ? C[j] : 0.0;
    __syncthreads();

    // ---- Lloyd iterations
    const int mask_words = (int)((n + kBlkPts * 32 - 1) / (kBlkPts * 32));
    for (int i = tid; i < K * kMaskWords; i += kKmThreads) bmask[i] = 0u;
    __syncthreads();
    for (int it = 0; it < a.iters; ++it) {
        for (int64_t i = tid; i < n; i += kKmThreads) {
            double xd[DSUB];
#pragma unroll
            for (int j = 0; j < DSUB; ++j) xd[j] = (double)pts[i * DSUB + j];
            const int c = nearest_centroid<DSUB>(xd, C, K);
            asg[i] = (uint8_t)c;
            atomicOr(&bmask[c * kMaskWords + (int)(i / (kBlkPts * 32))], 1u << ((i / kBlkPts) & 31));
        }
        __syncthreads();
        // the update reads only assignments and points, so centroid c can be
        // replaced as soon as its own sums are done
        if (tid < K) {
            double sum[DSUB];
#pragma unroll
            for (int j = 0; j < DSUB; ++j) sum[j] = 0.0;
            int64_t cnt = 0;
            auto add = [&](int64_t i) {
                ++cnt;
#pragma unroll
                for (int j = 0; j < DSUB; ++j) sum[j] = __dadd_rn(sum[j], (double)pts[i * DSUB + j]);
            };
            // within a block, the assignments four at a time: a word that holds no
            // byte equal to this centroid costs a few integer operations; a word that
            // may hold one is checked byte by byte, in point order
            const uint32_t pat = (uint32_t)tid * 0x01010101u;
            const uint32_t* a4 = reinterpret_cast<const uint32_t*>(asg);
            for (int w = 0; w < mask_words; ++w) {
                uint32_t bits = bmask[tid * kMaskWords + w];
                bmask[tid * kMaskWords + w] = 0u;  // cleared for the next iteration
                while (bits) {
                    const int64_t i0 = ((int64_t)w * 32 + __builtin_ctz(bits)) * kBlkPts;
                    bits &= bits - 1;
                    const int64_t i1 = i0 + kBlkPts < n ? i0 + kBlkPts : n;
                    int64_t i = i0;
                    for (; i + 4 <= i1; i += 4) {
                        const uint32_t wv = a4[i / 4];
                        const uint32_t mz = wv ^ pat;
                        if ((mz - 0x01010101u) & ~mz & 0x80808080u) {  // some byte of mz is zero
#pragma unroll
                            for (int k = 0; k < 4; ++k)
                                if (((wv >> (8 * k)) & 0xffu) == (uint32_t)tid) add(i + k);
                        }
                    }
                    for (; i < i1; ++i)
                        if (asg[i] == tid) add(i);
                }
            }
            if (cnt > 0)
#pragma unroll
                for (int j = 0; j < DSUB; ++j) C[tid * DSUB + j] = __ddiv_rn(sum[j], (double)cnt);
        }
        __syncthreads();
    }

    if (tid < K)
#pragma unroll
        for (int j = 0; j < DSUB; ++j)
            a.cb[(((int64_t)h * K + tid) * a.M + m) * DSUB + j] = __double2float_rn(C[tid * DSUB + j]);
    if (a.kept && tid == 0) a.kept[(int64_t)h * a.M + m] = kept;
}

template <int DSUB, typename XT>
hipError_t launch_typed(const KmArgs& a, hipStream_t stream) {
    // points (fp32) and their one-byte assignments; with the static centroids and block
    // masks, 8192 points at d_sub 4 take 152 KiB of the 160 KiB
    const size_t dyn = (size_t)a.n * DSUB * sizeof(float) + (size_t)a.n;
    auto kern = kmeans_kernel<DSUB, XT>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)a.M, (unsigned)a.Hkv), dim3(kKmThreads), dyn, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_kmeans(const pqkv_dims& d, const void* x, pqkv_dtype xt, int64_t n, int64_t s_tok,
                         int64_t s_head, const int32_t* order, int32_t iters, float* cb, int32_t* kept,
                         hipStream_t stream) {
    KmArgs a{x, n, s_tok, s_head, order, iters, d.n_centroids, d.head_dim / d.d_sub, d.n_kv_heads, cb, kept};
    if (d.d_sub == 2)
        return xt == PQKV_F16 ? launch_typed<2, __half>(a, stream) : launch_typed<2, float>(a, stream);
    return xt == PQKV_F16 ? launch_typed<4, __half>(a, stream) : launch_typed<4, float>(a, stream);
}

}  // namespace pqkv
