// The library's host side (argument validation and split planning in api.cpp)
// under AddressSanitizer and UndefinedBehaviorSanitizer, built with g++ and no GPU:
// the kernel launchers are stubs that record what they were asked to launch.
// Every entry point is called with valid and invalid arguments, and the plans of a
// sweep of shapes are checked against the invariants the kernels rely on.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../decode_attention_pq_amd/csrc/api.cpp"

namespace pqkv {
static int g_launches = 0;
static DecodeArgs g_args;
static DecodePlan g_plan;
hipError_t launch_encode(const pqkv_dims&, const void*, pqkv_dtype, int32_t, int64_t, int64_t, int64_t, int64_t,
                         const float*, uint8_t*, int64_t, int64_t, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_build_lut(const pqkv_dims&, int32_t, const void*, pqkv_dtype, const float*, float*, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_append(const pqkv_dims&, int32_t, const void*, const void*, void*, void*, pqkv_dtype, int64_t,
                         const int32_t*, const int32_t*, int32_t*, int32_t*, int32_t, const float*, const float*,
                         uint8_t*, uint8_t*, int64_t, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_kmeans(const pqkv_dims&, const void*, pqkv_dtype, int64_t, int64_t, int64_t, const int32_t*, int32_t,
                         float*, int32_t*, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_merge_states(int64_t, int32_t, const float*, const float*, const float*, const float*, float*, float*,
                               hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_decode(const pqkv_dims&, int32_t, pqkv_dtype, pqkv_dtype, const DecodePlan& plan,
                         const DecodeArgs& a, hipStream_t) {
    ++g_launches;
    g_args = a;
    g_plan = plan;
    return hipSuccess;
}
hipError_t launch_fp16_decode(const Fp16Plan&, int32_t, const Fp16Call&, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
}  // namespace pqkv

static int fails = 0;
#define CHECK(c)                                                  \
    do {                                                          \
        if (!(c)) {                                               \
            std::fprintf(stderr, "FAIL line %d: %s\n", __LINE__, #c); \
            ++fails;                                              \
        }                                                         \
    } while (0)

int main() {
    // fake, suitably aligned device addresses: never dereferenced on the host
    void* F = reinterpret_cast<void*>(0x100000);
    const float* FF = static_cast<const float*>(F);
    const uint8_t* FB = static_cast<const uint8_t*>(F);
    const int32_t* FI = static_cast<const int32_t*>(F);
    std::vector<unsigned char> ws_host(1);  // a real pointer for the workspace arithmetic checks

    // plan sweep: the invariants the decode kernel relies on
    for (int d : {64, 128})
        for (int dsub : {2, 4})
            for (int hkv : {1, 2, 8, 32})
                for (int g : {1, 2, 4, 8})
                    for (int batch : {1, 3, 16, 64})
                        for (int64_t T : {0LL, 1LL, 63LL, 64LL, 511LL, 512LL, 4096LL, 4160LL, 31436LL, 32768LL,
                                          131072LL, 300000LL}) {
                            pqkv_dims dm = {d, dsub, 256, hkv * g, hkv};
                            const DecodePlan p = plan_decode(dm, batch, T);
                            const int M = d / dsub;
                            CHECK(p.qh >= 1 && g % p.qh == 0 && p.qh * M <= 64);
                            CHECK(p.n_groups * p.qh == g);
                            CHECK(p.units == (int64_t)batch * hkv * p.n_groups);
                            CHECK(p.units <= (int64_t)batch * dm.n_q_heads);  // one counter slot each
                            CHECK(p.partials_offset >= (size_t)p.units * 4 && p.partials_offset % 256 == 0);
                            CHECK(p.workspace_bytes >= p.partials_offset + (size_t)batch * dm.n_q_heads * p.n_split *
                                                                               p.partial_stride * 4);
                            if (T > 0) {
                                CHECK(p.split_tokens == (int64_t)p.rounds * kTokensPerRound);
                                CHECK((int64_t)p.n_split * p.split_tokens >= T);
                                CHECK((int64_t)(p.n_split - 1) * p.split_tokens < T);
                                CHECK(p.rounds >= 1 && p.rounds <= decode_kernel_rounds(M, p.qh, p.rounds));
                                CHECK(decode_kernel_rounds(M, p.qh, p.rounds) <= decode_max_rounds(M, p.qh));
                            } else {
                                CHECK(p.n_split == 1);
                            }
                            const Fp16Plan f = plan_fp16_decode(d, hkv * g, hkv, batch, T);
                            CHECK(f.n_split >= 1 && f.n_split <= 64 && f.split_tokens % 128 == 0);
                            CHECK((int64_t)f.n_split * f.split_tokens >= T);
                            CHECK(f.workspace_bytes >= f.partials_offset + (size_t)batch * hkv * g * f.n_split *
                                                                               f.partial_stride * 4);
                        }

    // work-group id -> item: every grid size maps its ids one to one onto its items, XCD
    // x (id mod 8) holding a contiguous block of ceil((n - x) / 8); with only `used` of
    // the items live (the device-side plan), exactly the ids that xcd_has_item keeps
    // cover [0, used) once each, in the same contiguous blocks
    for (int n = 1; n <= 4100; ++n) {
        std::vector<int> seen(n, 0);
        bool ok = true;
        for (int id = 0; id < n; ++id) {
            const int it = xcd_item(id, n);
            ok = ok && it >= 0 && it < n && !seen[it]++;
            const int x = id & 7, lo = x * (n >> 3) + (x < (n & 7) ? x : (n & 7));
            ok = ok && it - lo == (id >> 3) && (id >> 3) < (n - x + 7) / 8;
        }
        CHECK(ok);
        for (int used : {1, n / 3, n - 1, n}) {
            if (used < 1) continue;
            std::vector<int> hit(used, 0);
            bool ok2 = true;
            for (int id = 0; id < n; ++id)
                if (xcd_has_item(id, used)) {
                    const int it = xcd_item(id, used);
                    ok2 = ok2 && it >= 0 && it < used && !hit[it]++;
                }
            for (int i = 0; i < used; ++i) ok2 = ok2 && hit[i] == 1;
            CHECK(ok2);
        }
    }

    pqkv_dims dm = {128, 2, 256, 32, 32};
    const size_t need = pqkv_decode_workspace_bytes(&dm, 1, 32768);
    CHECK(need == 256 + 32 * 8 * 132 * 4);
    // a valid decode call reaches the launcher with the workspace split as documented
    ws_host.resize(need + 256);
    void* ws = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(ws_host.data()) + 255) / 256 * 256);
    int before = g_launches;
    CHECK(pqkv_decode_attention(&dm, 1, F, PQKV_F16, nullptr, FF, FF, FB, FB, 32768, FI, 32768, F, F, PQKV_F16, 128,
                                FI, 0.088f, (float*)F, (float*)F, ws, need, nullptr) == PQKV_OK);
    CHECK(g_launches == before + 1);
    CHECK(reinterpret_cast<void*>(g_args.counters) == ws);
    CHECK(reinterpret_cast<char*>(g_args.partials) == static_cast<char*>(ws) + 256);
    CHECK(g_plan.n_split == 8 && g_args.lut == nullptr && g_args.hist_len == FI);
    // with a table the key codebook is not passed on
    CHECK(pqkv_decode_attention(&dm, 1, F, PQKV_F16, FF, nullptr, FF, FB, FB, 32768, FI, 32768, F, F, PQKV_F16, 128,
                                FI, 0.088f, (float*)F, (float*)F, ws, need, nullptr) == PQKV_OK);
    CHECK(g_args.lut == FF && g_args.cb_k == nullptr);
    // no history: lengths, codes and codebooks may be null, and the kernel gets no lengths
    CHECK(pqkv_decode_attention(&dm, 1, F, PQKV_F16, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr, 0, F, F,
                                PQKV_F16, 128, FI, 0.088f, (float*)F, (float*)F, ws, need, nullptr) == PQKV_OK);
    CHECK(g_args.hist_len == nullptr && g_args.max_hist == 0);
    // invalid arguments enqueue nothing
    before = g_launches;
    CHECK(pqkv_decode_attention(&dm, 1, F, PQKV_F16, nullptr, FF, FF, FB, FB, 32768, nullptr, 32768, F, F, PQKV_F16,
                                128, FI, 0.088f, (float*)F, (float*)F, ws, need, nullptr) == PQKV_ERR_INVALID);
    CHECK(pqkv_decode_attention(&dm, 1, (char*)F + 8, PQKV_F16, nullptr, FF, FF, FB, FB, 32768, FI, 32768, F, F,
                                PQKV_F16, 128, FI, 0.088f, (float*)F, (float*)F, ws, need, nullptr) == PQKV_ERR_INVALID);
    CHECK(pqkv_decode_attention(&dm, 1, F, PQKV_F16, nullptr, FF, FF, FB, FB, 32768, FI, 32768, F, F, PQKV_F16, 128,
                                FI, 0.088f, (float*)F, (float*)F, ws, need - 1, nullptr) == PQKV_ERR_WORKSPACE);
    pqkv_dims odd = {128, 2, 250, 32, 32};
    CHECK(pqkv_decode_attention(&odd, 1, F, PQKV_F16, FF, nullptr, FF, FB, FB, 32768, FI, 32768, F, F, PQKV_F16, 128,
                                FI, 0.088f, (float*)F, (float*)F, ws, need, nullptr) == PQKV_ERR_UNSUPPORTED);
    CHECK(g_launches == before);
    // the other entry points
    CHECK(pqkv_encode(&dm, F, PQKV_F16, 1, 100, 0, 4096, 128, FF, (uint8_t*)F, 128, 0, nullptr) == PQKV_OK);
    CHECK(pqkv_encode(&dm, F, PQKV_F16, 1, 100, 0, 4096, 128, FF, (uint8_t*)F, 64, 0, nullptr) == PQKV_ERR_INVALID);
    CHECK(pqkv_build_lut(&dm, 2, F, PQKV_F16, FF, (float*)F, nullptr) == PQKV_OK);
    CHECK(pqkv_merge(10, 128, FF, FF, FF, FF, (float*)F, (float*)F, nullptr) == PQKV_OK);
    CHECK(pqkv_fit_codebooks(&dm, F, PQKV_F16, 4096, 4096, 128, FI, 10, (float*)F, nullptr, nullptr) == PQKV_OK);
    {
        int32_t* L4 = reinterpret_cast<int32_t*>(0x200000);
        CHECK(pqkv_append_kv(&dm, 2, F, F, F, F, PQKV_F16, 128, L4, L4 + 64, L4 + 128, L4 + 192, 64, FF, FF,
                             (uint8_t*)F, (uint8_t*)F, 4096, 1000, nullptr) == PQKV_OK);
        CHECK(pqkv_append_kv(&dm, 2, F, F, F, F, PQKV_F16, 128, L4, L4 + 1, L4 + 128, L4 + 192, 64, FF, FF,
                             (uint8_t*)F, (uint8_t*)F, 4096, 1000, nullptr) == PQKV_OK);
        CHECK(pqkv_append_kv(&dm, 2, F, F, F, F, PQKV_F16, 128, L4, L4 + 64, L4 + 1, L4 + 192, 64, FF, FF,
                             (uint8_t*)F, (uint8_t*)F, 4096, 1000, nullptr) == PQKV_ERR_INVALID);  // out overlaps in
    }
    // the fp16 baseline
    const size_t fneed = pqkv_fp16_decode_workspace_bytes(&dm, 1, 32768);
    CHECK(fneed > 0 && pqkv_fp16_decode_workspace_bytes(&odd, 1, 100) > 0);
    pqkv_dims g3 = {128, 2, 256, 24, 8};  // 3 query heads per kv head: not built
    CHECK(pqkv_fp16_decode_workspace_bytes(&g3, 1, 100) == 0);
    ws_host.resize(fneed + 256);
    ws = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(ws_host.data()) + 255) / 256 * 256);
    CHECK(pqkv_fp16_decode_attention(&dm, 1, F, F, F, 32768, FI, 32768, 0.088f, (float*)F, (float*)F, ws, fneed,
                                     nullptr) == PQKV_OK);
    CHECK(pqkv_fp16_decode_attention(&dm, 1, F, F, F, 32768, FI, 40000, 0.088f, (float*)F, (float*)F, ws, fneed,
                                     nullptr) == PQKV_ERR_INVALID);
    CHECK(pqkv_fp16_decode_attention(&g3, 1, F, F, F, 32768, FI, 100, 0.088f, (float*)F, (float*)F, ws, fneed,
                                     nullptr) == PQKV_ERR_UNSUPPORTED);
    std::printf(fails ? "api_host_sanitize: %d failures\n" : "api_host_sanitize: ok\n", fails);
    return fails != 0;
}
