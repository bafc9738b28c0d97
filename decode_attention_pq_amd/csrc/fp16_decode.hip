// Dense fp16 decode attention (split-K flash decoding): the full-precision
// baseline the MILLION write-up measures its decode speed against (Fig. 12
// paragraph: time per output token against an FP16 cache at up to 32K context).
// It reads the whole fp16 K/V cache, 4*d bytes per cached token and kv head, so
// at the same shape it moves 2*d_sub times the history bytes of the PQ path.
//
// gfx950 design:
//   - One work-group of 256 threads (4 waves) per (sequence, kv head, token
//     split); it serves every query head of its kv head, so each K/V row is read
//     once per group of query heads.
//   - A load instruction brings 1 KiB: 16 bytes (8 fp16 elements) per lane, d/8
//     lanes per token, so a wave reads 64/(d/8) consecutive cache rows at once,
//     fully coalesced.  A wave takes steps of 8 such loads for K and 8 for V, with
//     the next step's loads in flight while the current one is used.
//   - Scores: v_dot2 of fp16 pairs into fp32, then a DPP sum over the token's
//     lanes; an online softmax per wave (running max, rescaled sums); values
//     accumulate in fp32, each lane for its 8 elements.
//   - Waves combine through LDS; the work-group publishes (max, sum, output) and
//     the last work-group of a (sequence, kv head) merges every split, as the PQ
//     decode kernel does; a unit with one split writes out and lse directly.

#include <hip/hip_fp16.h>

#include "pqkv_internal.h"

namespace pqkv {
namespace {

constexpr float kLn2 = 0.6931471805599453f;
constexpr int kThreads = kFp16Threads;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 8;  // load instructions per tensor per wave step

template <int CTRL, int ROWS>
__device__ inline float dpp_f(float v, float id) {
    return __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp((int)__float_as_uint(id), (int)__float_as_uint(v),
                                                                   CTRL, ROWS, 0xF, false));
}

// Sum over the LPT lanes of a token's row (LPT = 8 or 16): quad permutes, then
// mirrors inside half rows and rows; every lane of the row ends with the total.
template <int LPT>
__device__ inline float row_sum(float v) {
    v += dpp_f<0xB1, 0xF>(v, 0.0f);   // quad_perm [1,0,3,2]
    v += dpp_f<0x4E, 0xF>(v, 0.0f);   // quad_perm [2,3,0,1]
    v += dpp_f<0x141, 0xF>(v, 0.0f);  // row_half_mirror
    if constexpr (LPT == 16) v += dpp_f<0x140, 0xF>(v, 0.0f);  // row_mirror
    return v;
}

template <typename Op>
__device__ inline float wave_reduce(float v, float id, Op op) {
    v = op(v, dpp_f<0xB1, 0xF>(v, id));
    v = op(v, dpp_f<0x4E, 0xF>(v, id));
    v = op(v, dpp_f<0x141, 0xF>(v, id));
    v = op(v, dpp_f<0x140, 0xF>(v, id));
    v = op(v, dpp_f<0x142, 0xA>(v, id));  // row_bcast:15
    v = op(v, dpp_f<0x143, 0xC>(v, id));  // row_bcast:31
    return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 63));
}

__device__ inline float wave_max(float v) {
    return wave_reduce(v, -INFINITY, [](float x, float y) { return fmaxf(x, y); });
}

__device__ inline float wave_sum(float v) {
    return wave_reduce(v, 0.0f, [](float x, float y) { return x + y; });
}

__device__ uint4 g_zero_row[64];  // read by the loads of rows past the split

__device__ inline void publish(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ inline float collect(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ inline float dot8(const uint4 k, const uint4 q, float acc) {
    const uint32_t kw[4] = {k.x, k.y, k.z, k.w};
    const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, kw[i]), __builtin_bit_cast(half2_t, qw[i]), acc,
                                     false);
    return acc;
}

__device__ inline void unpack8(const uint4 v, float (&f)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float2 t = __half22float2(__builtin_bit_cast(__half2, w[i]));
        f[2 * i] = t.x;
        f[2 * i + 1] = t.y;
    }
}

struct Fp16Args {
    int Hq, Hkv, n_split, n_items;
    int64_t split_tokens;
    const int32_t* seq_len;
    const __half* q;
    const __half* k;
    const __half* v;
    int64_t t_cap;
    int64_t max_len;
    float scale_log2;
    int pstride;
    float* partials;
    uint32_t* counters;
    float* out;
    float* lse;
};

template <int D, int G>
__global__ __launch_bounds__(kThreads) void fp16_decode_kernel(Fp16Args a) {
    constexpr int LPT = D / 8;     // lanes per token
    constexpr int TPI = 64 / LPT;  // tokens per load instruction
    constexpr int TPS = kUnroll * TPI;  // tokens per wave step
    __shared__ float ored[kWaves][G][D];
    __shared__ float wm[kWaves][G], wl[kWaves][G];
    __shared__ int last_flag;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // XCD-aware mapping (ids that share id mod 8 take contiguous items), items head-major
    const int L = blockIdx.x;
    const int xcd = L & 7;
    const int item = xcd * (a.n_items >> 3) + (xcd < (a.n_items & 7) ? xcd : (a.n_items & 7)) + (L >> 3);
    const int unit = item / a.n_split;
    const int split = item - unit * a.n_split;
    const int batch = a.n_items / (a.Hkv * a.n_split);
    const int b = unit % batch;
    const int h = unit / batch;
    const int hq0 = h * G;

    int64_t T = a.seq_len[b];
    T = T < 0 ? 0 : (T > a.max_len ? a.max_len : T);
    const int ns = T > 0 ? (int)((T + a.split_tokens - 1) / a.split_tokens) : 1;
    if (split >= ns) return;
    const int64_t t0 = (int64_t)split * a.split_tokens;
    const int64_t t1 = T < t0 + a.split_tokens ? T : t0 + a.split_tokens;

    const int row = lane / LPT;        // token slot inside a load
    const int e0 = (lane % LPT) * 8;   // this lane's 8 elements
    uint4 qv[G];
#pragma unroll
    for (int j = 0; j < G; ++j)
        qv[j] = *reinterpret_cast<const uint4*>(a.q + ((int64_t)b * a.Hq + hq0 + j) * D + e0);

    const int64_t plane = ((int64_t)b * a.Hkv + h) * a.t_cap * D;
    const __half* kb = a.k + plane;
    const __half* vb = a.v + plane;
    const int64_t n_steps = (t1 - t0 + TPS - 1) / TPS;  // wave steps of this split, shared round-robin
    auto tok = [&](int64_t st, int i) { return t0 + st * TPS + i * TPI + row; };
    auto load_step = [&](uint4 (&kr)[kUnroll], uint4 (&vr)[kUnroll], int64_t st) {
#pragma unroll
        for (int i = 0; i < kUnroll; ++i) {
            const int64_t t = tok(st, i);
            const bool ok = t < t1;
            kr[i] = *reinterpret_cast<const uint4*>(ok ? kb + t * D + e0 : reinterpret_cast<const __half*>(g_zero_row));
        }
#pragma unroll
        for (int i = 0; i < kUnroll; ++i) {
            const int64_t t = tok(st, i);
            const bool ok = t < t1;
            vr[i] = *reinterpret_cast<const uint4*>(ok ? vb + t * D + e0 : reinterpret_cast<const __half*>(g_zero_row));
        }
    };

    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        m[j] = -INFINITY;
        l[j] = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[j][k] = 0.0f;
    }
    uint4 kc[kUnroll], vc[kUnroll], kn[kUnroll], vn[kUnroll];
    int64_t st = wave;
    if (st < n_steps) load_step(kc, vc, st);
    for (; st < n_steps; st += kWaves) {
        const bool more = st + kWaves < n_steps;
        if (more) load_step(kn, vn, st + kWaves);
        float s[kUnroll][G];
#pragma unroll
        for (int i = 0; i < kUnroll; ++i) {
            const bool ok = tok(st, i) < t1;
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const float dsum = row_sum<LPT>(dot8(kc[i], qv[j], 0.0f));
                s[i][j] = ok ? dsum * a.scale_log2 : -INFINITY;
            }
        }
#pragma unroll
        for (int j = 0; j < G; ++j) {
            float mx = s[0][j];
#pragma unroll
            for (int i = 1; i < kUnroll; ++i) mx = fmaxf(mx, s[i][j]);
            const float mnew = fmaxf(m[j], wave_max(mx));  // finite: the step holds a token
            const float r = exp2f(m[j] - mnew);
            m[j] = mnew;
            l[j] *= r;
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[j][k] *= r;
        }
#pragma unroll
        for (int i = 0; i < kUnroll; ++i) {
            float vf[8];
            unpack8(vc[i], vf);
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const float p = exp2f(s[i][j] - m[j]);
                l[j] += p;
#pragma unroll
                for (int k = 0; k < 8; ++k) acc[j][k] = fmaf(p, vf[k], acc[j][k]);
            }
        }
        if (more) {
#pragma unroll
            for (int i = 0; i < kUnroll; ++i) {
                kc[i] = kn[i];
                vc[i] = vn[i];
            }
        }
    }
    // rows of the wave hold different tokens: add them up (every lane of a row counted
    // its row's weights, so the weight sum is the wave sum over LPT)
#pragma unroll
    for (int j = 0; j < G; ++j) {
        l[j] = wave_sum(l[j]) * (1.0f / LPT);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            float x = acc[j][k];
#pragma unroll
            for (int off = LPT; off < 64; off *= 2) x += __shfl_xor(x, off);
            acc[j][k] = x;
        }
    }
    if (lane < LPT) {
#pragma unroll
        for (int j = 0; j < G; ++j)
#pragma unroll
            for (int k = 0; k < 8; ++k) ored[wave][j][e0 + k] = acc[j][k];
    }
    if (lane == 0) {
#pragma unroll
        for (int j = 0; j < G; ++j) {
            wm[wave][j] = m[j];
            wl[wave][j] = l[j];
        }
    }
    __syncthreads();

    // combine the waves: element e of head j per thread
    float* part_base = a.partials + ((int64_t)(b * a.Hq + hq0) * a.n_split + split) * a.pstride;
    const int64_t head_step = (int64_t)a.n_split * a.pstride;
    for (int x = tid; x < G * D; x += kThreads) {
        const int j = x / D, e = x - j * D;
        float mall = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) mall = fmaxf(mall, wm[w][j]);
        float o = 0.0f, ls = 0.0f;
        if (mall != -INFINITY) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float f = exp2f(wm[w][j] - mall);  // 0 for a wave without tokens
                o = fmaf(f, ored[w][j][e], o);
                ls = fmaf(f, wl[w][j], ls);
            }
        }
        const int64_t orow = (int64_t)b * a.Hq + hq0 + j;
        if (ns == 1) {
            a.out[orow * D + e] = mall != -INFINITY ? o / ls : 0.0f;
            if (e == 0) a.lse[orow] = mall != -INFINITY ? (mall + log2f(ls)) * kLn2 : -INFINITY;
        } else {
            float* part = part_base + j * head_step;
            publish(part + e, o);
            if (e == 0) {
                publish(part + D, mall);
                publish(part + D + 1, ls);
            }
        }
    }
    if (ns == 1) return;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const uint32_t done = __hip_atomic_fetch_add(a.counters + unit, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last_flag = (done == (uint32_t)(ns - 1));
    }
    __syncthreads();
    if (!last_flag) return;
    const float* prow0 = a.partials + (int64_t)(b * a.Hq + hq0) * a.n_split * a.pstride;
    for (int x = tid; x < G * D; x += kThreads) {
        const int j = x / D, e = x - j * D;
        const float* prow = prow0 + j * head_step;
        float mall = -INFINITY, ls = 0.0f, o = 0.0f;
        for (int s0 = 0; s0 < ns; s0 += 8) {  // eight splits' loads in flight at once
            float pm[8], pl[8], po[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const float* ps = prow + (int64_t)(s0 + u < ns ? s0 + u : ns - 1) * a.pstride;
                pm[u] = collect(ps + D);
                pl[u] = collect(ps + D + 1);
                po[u] = collect(ps + e);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (s0 + u >= ns || pm[u] == -INFINITY) continue;
                const float mnew = fmaxf(mall, pm[u]);
                const float r = exp2f(mall - mnew);  // 0 while nothing has been folded in
                const float f = exp2f(pm[u] - mnew);
                ls = fmaf(f, pl[u], ls * r);
                o = fmaf(f, po[u], o * r);
                mall = mnew;
            }
        }
        const int64_t orow = (int64_t)b * a.Hq + hq0 + j;
        a.out[orow * D + e] = mall != -INFINITY ? o / ls : 0.0f;
        if (e == 0) a.lse[orow] = mall != -INFINITY ? (mall + log2f(ls)) * kLn2 : -INFINITY;
    }
    if (tid == 0) __hip_atomic_store(a.counters + unit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, int G>
hipError_t launch_g(const Fp16Plan& p, int32_t batch, const Fp16Call& c, hipStream_t stream) {
    Fp16Args a;
    a.Hq = c.n_q_heads;
    a.Hkv = c.n_kv_heads;
    a.n_split = p.n_split;
    a.split_tokens = p.split_tokens;
    a.n_items = (int)((int64_t)batch * c.n_kv_heads * p.n_split);
    a.seq_len = c.seq_len;
    a.q = static_cast<const __half*>(c.q);
    a.k = static_cast<const __half*>(c.k);
    a.v = static_cast<const __half*>(c.v);
    a.t_cap = c.t_cap;
    a.max_len = c.max_len;
    a.scale_log2 = c.scale * 1.4426950408889634f;
    a.pstride = p.partial_stride;
    a.partials = c.partials;
    a.counters = c.counters;
    a.out = c.out;
    a.lse = c.lse;
    hipLaunchKernelGGL((fp16_decode_kernel<D, G>), dim3((unsigned)a.n_items), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const Fp16Plan& p, int32_t batch, const Fp16Call& c, hipStream_t stream) {
    switch (c.n_q_heads / c.n_kv_heads) {
        case 1: return launch_g<D, 1>(p, batch, c, stream);
        case 2: return launch_g<D, 2>(p, batch, c, stream);
        case 4: return launch_g<D, 4>(p, batch, c, stream);
        default: return launch_g<D, 8>(p, batch, c, stream);
    }
}

}  // namespace

hipError_t launch_fp16_decode(const Fp16Plan& p, int32_t batch, const Fp16Call& c, hipStream_t stream) {
    return c.head_dim == 64 ? launch_d<64>(p, batch, c, stream) : launch_d<128>(p, batch, c, stream);
}

}  // namespace pqkv
