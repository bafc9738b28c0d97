// Device helpers shared by the kernels that quantise head vectors: subvector loads
// and the nearest-centroid scan.
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

// Subvector loads: DSUB consecutive elements (DSUB = 2 or 4, naturally aligned)
// as fp32.
template <int DSUB>
__device__ inline void load_sub(const float* __restrict__ p, float (&v)[DSUB]) {
    if constexpr (DSUB == 4) {
        const float4 t = *reinterpret_cast<const float4*>(p);
        v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    } else {
        const float2 t = *reinterpret_cast<const float2*>(p);
        v[0] = t.x; v[1] = t.y;
    }
}

template <int DSUB>
__device__ inline void load_sub(const __half* __restrict__ p, float (&v)[DSUB]) {
    if constexpr (DSUB == 4) {
        const uint2 t = *reinterpret_cast<const uint2*>(p);
        const float2 a = __half22float2(*reinterpret_cast<const __half2*>(&t.x));
        const float2 b = __half22float2(*reinterpret_cast<const __half2*>(&t.y));
        v[0] = a.x; v[1] = a.y; v[2] = b.x; v[3] = b.y;
    } else {
        const uint32_t t = *reinterpret_cast<const uint32_t*>(p);
        const float2 a = __half22float2(*reinterpret_cast<const __half2*>(&t));
        v[0] = a.x; v[1] = a.y;
    }
}

// Squared distance of subvector xs to the centroid at cc: fp32 differences,
// squared and summed in subspace order (never the expanded |x|^2 - 2x.c + |c|^2
// form, whose cancellation would move codes).
template <int DSUB, typename C>
__device__ inline float sq_dist(const float (&xs)[DSUB], const C& cc) {
    float dd = 0.0f;
#pragma unroll
    for (int j = 0; j < DSUB; ++j) {
        const float e = xs[j] - cc[j];
        dd = fmaf(e, e, dd);
    }
    return dd;
}

// Index of the centroid nearest to xs among the K centroids at cm, cm + CS, ...
// (on chip): the smallest squared distance, strict '<' in ascending order, so
// the lowest index wins exact ties and NaN distances never win.
//
// When K is a multiple of 64 the scan runs in blocks of 64 fully unrolled
// centroids.  Inside a block the running index is the block-relative position,
// an inline constant of the select instruction, so a (subvector, centroid) pair
// costs the distance plus one compare and two selects, with no index register
// to maintain.  A block's winner replaces the running one only if strictly
// smaller, which keeps the first minimum overall.
template <int DSUB, int CS>
__device__ inline int nearest_code(const float (&xs)[DSUB], const float* cm, int K) {
    float best = INFINITY;
    int bi = 0;
    if ((K & 63) == 0) {
        // centroid values are read in groups of G (64 floats in registers) before
        // the group's distances, so the LDS latency is paid once per group
        constexpr int G = 64 / DSUB;
        for (int c0 = 0; c0 < K; c0 += 64) {
            const float* cb = cm + c0 * CS;
            float bb = INFINITY;
            int br = 0;
#pragma unroll
            for (int g0 = 0; g0 < 64; g0 += G) {
                float cv[G][DSUB];
#pragma unroll
                for (int r = 0; r < G; ++r) load_sub<DSUB>(cb + (g0 + r) * CS, cv[r]);
#pragma unroll
                for (int r = 0; r < G; ++r) {
                    const float dd = sq_dist<DSUB>(xs, cv[r]);
                    if (dd < bb) {
                        bb = dd;
                        br = g0 + r;
                    }
                }
            }
            if (bb < best) {
                best = bb;
                bi = c0 + br;
            }
        }
    } else {
#pragma unroll 4
        for (int c = 0; c < K; ++c) {
            const float dd = sq_dist<DSUB>(xs, cm + c * CS);
            if (dd < best) {
                best = dd;
                bi = c;
            }
        }
    }
    return bi;
}

// Byte m of a token's code goes to the rotated position of its slot in the tile
// whose slot-0 chunk base is `dst` (the code-cache layout of pqkv.h).
template <int M>
__device__ inline void put_code(uint8_t* dst, int slot, int m, int code) {
    const int p = (m - slot) & (M - 1);
    dst[(p >> 4) * (kTileTokens * 16) + (p & 15)] = (uint8_t)code;
}

// Codes of subspaces m0 .. m0 + MW - 1 of one token.  xv holds those subspaces'
// values (MW * DSUB floats, subspace m0 first); `cbs` points at subspace m0 of
// centroid 0 of an on-chip codebook whose centroid rows are CS floats apart.
template <int D, int DSUB, int MW, int CS>
__device__ inline void write_nearest_codes_slice(const float (&xv)[MW * DSUB], const float* cbs, int K,
                                                 uint8_t* dst, int slot, int m0) {
#pragma unroll
    for (int mi = 0; mi < MW; ++mi) {
        float xs[DSUB];
#pragma unroll
        for (int j = 0; j < DSUB; ++j) xs[j] = xv[mi * DSUB + j];
        put_code<D / DSUB>(dst, slot, m0 + mi, nearest_code<DSUB, CS>(xs, cbs + mi * DSUB, K));
    }
}

// Byte address of token t's slot-0 chunk in plane `plane` (t_cap*M bytes).
template <int M>
__device__ inline uint8_t* code_slot(uint8_t* plane, int64_t t) {
    return plane + (t >> 6) * (kTileTokens * M) + (t & (kTileTokens - 1)) * 16;
}

}  // namespace pqkv
