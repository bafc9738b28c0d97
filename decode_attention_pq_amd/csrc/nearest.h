// Device helpers shared by the kernels that quantise head vectors: row loads and
// the nearest-centroid scan of one token.
//
// MILLION write-up (DAC 2025), page "MILLION": the paragraph after Fig. 5 splits
// the head vector into subspaces of dimension 2 or 4; the Fig. 6 paragraph
// encodes the KV cache with the offline-trained codebooks.  The code of a
// subvector is the index of the centroid at the smallest squared Euclidean
// distance, the lowest index winning exact ties.
#pragma once

#include <hip/hip_fp16.h>

#include "pqkv_internal.h"

namespace pqkv {

template <typename T>
struct Row;

template <>
struct Row<float> {
    template <int D>
    __device__ static void load(const float* __restrict__ p, float (&v)[D]) {
        const float4* p4 = reinterpret_cast<const float4*>(p);
#pragma unroll
        for (int i = 0; i < D / 4; ++i) {
            float4 t = p4[i];
            v[4 * i + 0] = t.x;
            v[4 * i + 1] = t.y;
            v[4 * i + 2] = t.z;
            v[4 * i + 3] = t.w;
        }
    }
};

template <>
struct Row<__half> {
    template <int D>
    __device__ static void load(const __half* __restrict__ p, float (&v)[D]) {
        const uint4* p4 = reinterpret_cast<const uint4*>(p);
#pragma unroll
        for (int i = 0; i < D / 8; ++i) {
            uint4 t = p4[i];
            const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                __half2 h2 = *reinterpret_cast<const __half2*>(&w[k]);
                float2 f = __half22float2(h2);
                v[8 * i + 2 * k + 0] = f.x;
                v[8 * i + 2 * k + 1] = f.y;
            }
        }
    }
};

// Codes of one token: for every subspace m, the centroid c < K of the codebook
// `cbs` ([c][m][j], on chip) nearest to row xv, by the sum of squared fp32
// differences (never the expanded |x|^2 - 2x.c + |c|^2 form), strict '<' in
// ascending c.  Byte m goes to the rotated position of token slot `slot` in the
// tile whose slot-0 chunk base is `dst` (the code-cache layout of pqkv.h).
template <int D, int DSUB>
__device__ inline void write_nearest_codes(const float (&xv)[D], const float* cbs, int K, uint8_t* dst,
                                           int slot) {
    constexpr int M = D / DSUB;
#pragma unroll
    for (int m = 0; m < M; ++m) {
        float best = INFINITY;
        int bi = 0;
        const float* cm = cbs + m * DSUB;
#pragma unroll 4
        for (int c = 0; c < K; ++c) {
            const float* cc = cm + c * D;
            float dd = 0.0f;
#pragma unroll
            for (int j = 0; j < DSUB; ++j) {
                const float e = xv[m * DSUB + j] - cc[j];
                dd = fmaf(e, e, dd);
            }
            if (dd < best) {
                best = dd;
                bi = c;
            }
        }
        const int p = (m - slot) & (M - 1);
        dst[(p >> 4) * (kTileTokens * 16) + (p & 15)] = (uint8_t)bi;
    }
}

// The same for subspaces m0 .. m0 + MW - 1 only.  xv holds those subspaces' values
// (MW * DSUB floats, subspace m0 first); `cbs` points at subspace m0 of centroid 0
// of an on-chip codebook whose centroid rows are CS floats apart.
template <int D, int DSUB, int MW, int CS>
__device__ inline void write_nearest_codes_slice(const float (&xv)[MW * DSUB], const float* cbs, int K,
                                                 uint8_t* dst, int slot, int m0) {
    constexpr int M = D / DSUB;
#pragma unroll
    for (int mi = 0; mi < MW; ++mi) {
        float best = INFINITY;
        int bi = 0;
        const float* cm = cbs + mi * DSUB;
#pragma unroll 4
        for (int c = 0; c < K; ++c) {
            const float* cc = cm + c * CS;
            float dd = 0.0f;
#pragma unroll
            for (int j = 0; j < DSUB; ++j) {
                const float e = xv[mi * DSUB + j] - cc[j];
                dd = fmaf(e, e, dd);
            }
            if (dd < best) {
                best = dd;
                bi = c;
            }
        }
        const int p = (m0 + mi - slot) & (M - 1);
        dst[(p >> 4) * (kTileTokens * 16) + (p & 15)] = (uint8_t)bi;
    }
}

// Byte address of token t's slot-0 chunk in plane `plane` (t_cap*M bytes).
template <int M>
__device__ inline uint8_t* code_slot(uint8_t* plane, int64_t t) {
    return plane + (t >> 6) * (kTileTokens * M) + (t & (kTileTokens - 1)) * 16;
}

}  // namespace pqkv
