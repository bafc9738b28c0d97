// Streaming-rate probe for gfx950: how fast a plain kernel reads code tiles laid out
// as the PQ decode kernel reads them, with the same work-group shape and no other work.
// Test infrastructure only (not part of libpqkv); its output is the practical HBM read
// ceiling quoted for the decode kernel.
//
// Shape of the 32K-context decode (32 heads x 8 splits, one work-group of 512 threads
// per piece): 256 work-groups each read 2 x 256 KiB (a K and a V plane slice of 4096
// tokens x 64 bytes) as 64-token tiles of 4 KiB, one 16-byte non-temporal load per lane
// per 1 KiB chunk; a wave walks tiles wave, wave + 8, ... with three tiles in flight.
// The grid reads 128 MiB per launch; launches rotate over 8 such buffers (1 GiB), so
// no launch is served from the last-level cache.  The same kernel on 128, 32 and 8
// work-groups (each still reading its 512 KiB) gives the rate one CU reaches when most
// of the others are idle.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kGroups = 256;
constexpr int kTileBytes = 4096;                         // 64 tokens x 64 code bytes
constexpr int kTilesPerPlane = 4096 * 64 / kTileBytes;   // 64 tiles per 256 KiB slice
constexpr int kRounds = kTilesPerPlane / kWaves;         // tiles per wave per plane
constexpr size_t kGroupBytes = 2 * (size_t)kTilesPerPlane * kTileBytes;
constexpr size_t kBufBytes = kGroupBytes * kGroups;      // 128 MiB
constexpr int kBuffers = 8;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ inline void load_tile(u32x4 (&t)[4], const uint8_t* base, int tile, int lane) {
    const uint8_t* p = base + (size_t)tile * kTileBytes + lane * 16;
#pragma unroll
    for (int c = 0; c < 4; ++c) t[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + c * 1024));
}

__global__ __launch_bounds__(kThreads) void stream(const uint8_t* __restrict__ buf, uint32_t* out) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const uint8_t* g = buf + (size_t)blockIdx.x * kGroupBytes;
    constexpr int kSteps = 2 * kRounds;  // K plane tiles, then V plane tiles
    auto tile_of = [&](int s) { return (s < kRounds ? s : s - kRounds) * kWaves + wave; };
    auto plane_of = [&](int s) { return g + (s < kRounds ? 0 : (size_t)kTilesPerPlane * kTileBytes); };
    u32x4 ring[4][4];
    uint32_t acc = 0;
#pragma unroll
    for (int s = 0; s < 3; ++s) load_tile(ring[s], plane_of(s), tile_of(s), lane);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        if (s + 3 < kSteps) load_tile(ring[(s + 3) % 4], plane_of(s + 3), tile_of(s + 3), lane);
#pragma unroll
        for (int c = 0; c < 4; ++c) acc ^= ring[s % 4][c].x ^ ring[s % 4][c].y ^ ring[s % 4][c].z ^ ring[s % 4][c].w;
    }
    if (acc == 0x12345678u) out[blockIdx.x] = acc;  // keeps the loads live
}

}  // namespace

int main() {
    uint8_t* buf[kBuffers];
    for (int i = 0; i < kBuffers; ++i) {
        if (hipMalloc(&buf[i], kBufBytes) != hipSuccess || hipMemset(buf[i], i, kBufBytes) != hipSuccess) {
            std::fprintf(stderr, "allocation failed\n");
            return 1;
        }
    }
    uint32_t* out = nullptr;
    if (hipMalloc(&out, kGroups * sizeof(uint32_t)) != hipSuccess) return 1;
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return 1;
    constexpr int kWarm = 200, kLaunches = 400;
    for (int i = 0; i < kWarm; ++i) stream<<<kGroups, kThreads>>>(buf[i % kBuffers], out);
    if (hipGetLastError() != hipSuccess || hipDeviceSynchronize() != hipSuccess) return 1;
    float best = 1e30f;
    for (int rep = 0; rep < 3; ++rep) {
        if (hipEventRecord(e0) != hipSuccess) return 1;
        for (int i = 0; i < kLaunches; ++i) stream<<<kGroups, kThreads>>>(buf[i % kBuffers], out);
        if (hipGetLastError() != hipSuccess || hipEventRecord(e1) != hipSuccess || hipEventSynchronize(e1) != hipSuccess)
            return 1;
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, e0, e1) != hipSuccess) return 1;
        best = ms < best ? ms : best;
    }
    const double us = best * 1e3 / kLaunches;
    std::printf("code-tile stream: %zu bytes per launch, %.2f us per launch (launch gaps included), %.1f GB/s, "
                "%.1f%% of 8 TB/s\n", kBufBytes, us, kBufBytes / (us * 1e-6) / 1e9, kBufBytes / (us * 1e-6) / 8e12 * 100);
    std::printf("  256 work-groups: %.1f GB/s per work-group\n", kGroupBytes / (us * 1e-6) / 1e9);
    for (int groups : {128, 32, 8}) {  // the first `groups` slices of each buffer
        float part = 1e30f;
        for (int rep = 0; rep < 3; ++rep) {
            if (hipEventRecord(e0) != hipSuccess) return 1;
            for (int i = 0; i < kLaunches; ++i) stream<<<groups, kThreads>>>(buf[i % kBuffers], out);
            if (hipGetLastError() != hipSuccess || hipEventRecord(e1) != hipSuccess || hipEventSynchronize(e1) != hipSuccess)
                return 1;
            float ms = 0.0f;
            if (hipEventElapsedTime(&ms, e0, e1) != hipSuccess) return 1;
            part = ms < part ? ms : part;
        }
        const double pus = part * 1e3 / kLaunches;
        std::printf("  %3d work-groups: %.2f us per launch, %.1f GB/s in all, %.1f GB/s per work-group\n", groups, pus,
                    groups * kGroupBytes / (pus * 1e-6) / 1e9, kGroupBytes / (pus * 1e-6) / 1e9);
    }
    for (int i = 0; i < kBuffers; ++i) (void)hipFree(buf[i]);
    (void)hipFree(out);
    return 0;
}
