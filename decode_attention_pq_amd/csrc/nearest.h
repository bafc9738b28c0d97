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

// Codes of NT subvectors xs[0..NT) of one subspace: for each, the index of the
// nearest of the K centroids of an on-chip codebook (centroid c at
// cm + c*CS + (c/16)*PAD: PAD floats after every 16 rows), i.e. the smallest
// squared distance, the lowest index among equal ones, NaN distances never
// winning (a subvector whose distances are all NaN or +inf gets code 0).  Every
// centroid value read serves all NT subvectors.
//
// When K is a multiple of 64 the scan takes two passes over the same fp32
// distances.  The first keeps only the minimum of every sub-block of 16
// centroids (three-operand mins, no index bookkeeping) and, across sub-blocks,
// the first one whose minimum is strictly smaller than all before it.  The
// second recomputes that sub-block's 16 distances, bit for bit the same
// instructions, and takes the first one equal to the minimum.  A pair then
// costs the distance plus half a min in the first pass, and 1/16 of a distance,
// compare and select in the second, where a single pass needs a compare and two
// selects per pair.  Lanes read different sub-blocks in the second pass; the
// PAD floats between sub-blocks put them on different LDS banks.
template <int DSUB, int CS, int PAD, int NT>
__device__ inline void nearest_codes(const float (&xs)[NT][DSUB], const float* cm, int K, int (&code)[NT]) {
    constexpr int SB = 16;  // centroids per sub-block
    auto row = [&](int c) { return cm + c * CS + (c / SB) * PAD; };
    if ((K & 63) == 0) {
        constexpr int G = 64 / DSUB;  // centroids whose values are read together (64 floats)
        static_assert(G % SB == 0, "a load group holds whole sub-blocks");
        float best[NT];
        int bsb[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            best[n] = INFINITY;
            bsb[n] = 0;
        }
        for (int c0 = 0; c0 < K; c0 += 64) {
            const float* cb = row(c0);
#pragma unroll
            for (int g0 = 0; g0 < 64; g0 += G) {
                // centroid values are read in groups of G before their distances, so
                // the LDS latency is paid once per group
                float cv[G][DSUB];
#pragma unroll
                for (int r = 0; r < G; ++r) load_sub<DSUB>(cb + (g0 + r) * CS + ((g0 + r) / SB) * PAD, cv[r]);
#pragma unroll
                for (int k = 0; k < G / SB; ++k) {
#pragma unroll
                    for (int n = 0; n < NT; ++n) {
                        float d[SB];
#pragma unroll
                        for (int r = 0; r < SB; ++r) d[r] = sq_dist<DSUB>(xs[n], cv[k * SB + r]);
                        const float t0 = fminf(fminf(d[0], d[1]), d[2]);
                        const float t1 = fminf(fminf(d[3], d[4]), d[5]);
                        const float t2 = fminf(fminf(d[6], d[7]), d[8]);
                        const float t3 = fminf(fminf(d[9], d[10]), d[11]);
                        const float t4 = fminf(fminf(d[12], d[13]), d[14]);
                        const float u0 = fminf(fminf(t0, t1), t2);
                        const float u1 = fminf(fminf(t3, t4), d[15]);
                        const float sm = fminf(u0, u1);
                        if (sm < best[n]) {
                            best[n] = sm;
                            bsb[n] = (c0 + g0) / SB + k;
                        }
                    }
                }
            }
        }
        // second pass: the first centroid of sub-block bsb at distance `best`,
        // scanned downwards so the lowest matching index is the one kept
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const float* sb = row(bsb[n] * SB);
            int idx = 0;
#pragma unroll
            for (int r = SB - 1; r >= 0; --r) {
                float cv[DSUB];
                load_sub<DSUB>(sb + r * CS, cv);
                idx = sq_dist<DSUB>(xs[n], cv) == best[n] ? r : idx;
            }
            // no distance below +inf: code 0, as the plain scan gives (this also holds
            // when a non-finite codebook mixes +inf and NaN distances)
            code[n] = best[n] < INFINITY ? bsb[n] * SB + idx : 0;
        }
        return;
    }
    float best[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        best[n] = INFINITY;
        code[n] = 0;
    }
#pragma unroll 4
    for (int c = 0; c < K; ++c) {
        float cv[DSUB];
        load_sub<DSUB>(row(c), cv);
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const float dd = sq_dist<DSUB>(xs[n], cv);
            if (dd < best[n]) {
                best[n] = dd;
                code[n] = c;
            }
        }
    }
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
// centroid 0 of an on-chip codebook whose centroid rows are CS floats apart, with
// PAD floats after every 16 rows.
template <int D, int DSUB, int MW, int CS, int PAD>
__device__ inline void write_nearest_codes_slice(const float (&xv)[MW * DSUB], const float* cbs, int K,
                                                 uint8_t* dst, int slot, int m0) {
#pragma unroll
    for (int mi = 0; mi < MW; ++mi) {
        float xs[1][DSUB];
#pragma unroll
        for (int j = 0; j < DSUB; ++j) xs[0][j] = xv[mi * DSUB + j];
        int code[1];
        nearest_codes<DSUB, CS, PAD, 1>(xs, cbs + mi * DSUB, K, code);
        put_code<D / DSUB>(dst, slot, m0 + mi, code[0]);
    }
}

// Byte address of token t's slot-0 chunk in plane `plane` (t_cap*M bytes).
template <int M>
__device__ inline uint8_t* code_slot(uint8_t* plane, int64_t t) {
    return plane + (t >> 6) * (kTileTokens * M) + (t & (kTileTokens - 1)) * 16;
}

}  // namespace pqkv
