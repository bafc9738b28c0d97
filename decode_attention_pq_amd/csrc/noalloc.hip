// pqkv_decode_attention_noalloc: the decode entry point for callers that cannot
// allocate (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  It runs the same kernels as pqkv_decode_attention with the
// workspace replaced by a file-scope device array.
//
// Layout of the array (per device): completion counters at bytes [0, 64 KiB), one
// u32 per (sequence, query head), at most PQKV_NOALLOC_MAX_ROWS of them; the
// per-split partials from byte 64 KiB on.  The counters are zero between calls
// (each call's last work-group of a unit resets its counter), so the fixed place
// keeps them valid for calls of any size.

#include <mutex>

#include "pqkv_internal.h"

namespace pqkv {
namespace {

constexpr size_t kCounterBytes = (size_t)PQKV_NOALLOC_MAX_ROWS * sizeof(uint32_t);
static_assert(kCounterBytes % 256 == 0, "the partials start 256-byte aligned");

// One copy per device, held until the process ends.  In host code this name is a
// host-side stand-in, never a device address: every use goes through the address
// hipGetSymbolAddress returns for the current device.
__device__ __align__(256) unsigned char scratch[PQKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // scratch's device address, per device (null until set up)

__global__ void clear_u32(uint32_t* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// The current device's copy of the scratch array, set up on the first call on that
// device: its address, and its counters cleared on `stream` (a fill kernel, not a
// memset, so that a call under stream capture records a kernel node).
pqkv_status scratch_on_current_device(hipStream_t stream, void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return PQKV_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return PQKV_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PQKV_ERR_HIP;
        const int n = (int)(kCounterBytes / sizeof(uint32_t));
        hipLaunchKernelGGL(clear_u32, dim3((n + 255) / 256), dim3(256), 0, stream, static_cast<uint32_t*>(p), n);
        if (hipGetLastError() != hipSuccess) return PQKV_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return PQKV_OK;
}

}  // namespace
}  // namespace pqkv

using namespace pqkv;

extern "C" pqkv_status pqkv_decode_attention_noalloc(
    const pqkv_dims* dims, int32_t batch, const void* q, pqkv_dtype q_dtype, const float* lut,
    const float* codebook_k, const float* codebook_v, const uint8_t* codes_k, const uint8_t* codes_v,
    int64_t t_cap, const int32_t* hist_len, int64_t max_hist_len, const void* recent_k, const void* recent_v,
    pqkv_dtype recent_dtype, int64_t r_cap, const int32_t* recent_len, float softmax_scale, float* out,
    float* lse, hipStream_t stream) {
    DecodePlan plan{};
    const pqkv_status st =
        check_decode_args(dims, batch, q, q_dtype, lut, codebook_k, codebook_v, codes_k, codes_v, t_cap, hist_len,
                          max_hist_len, recent_k, recent_v, recent_dtype, r_cap, recent_len, softmax_scale, out,
                          lse, &plan);
    if (st != PQKV_OK || batch == 0) return st;
    // the sizes the array holds: one counter per (sequence, query head), and the partials
    const size_t partial_bytes = plan.workspace_bytes - plan.partials_offset;
    if ((int64_t)batch * dims->n_q_heads > PQKV_NOALLOC_MAX_ROWS ||
        partial_bytes > PQKV_NOALLOC_SCRATCH_BYTES - kCounterBytes)
        return PQKV_ERR_WORKSPACE;
    void* base = nullptr;
    const pqkv_status ss = scratch_on_current_device(stream, &base);
    if (ss != PQKV_OK) return ss;
    const DecodeArgs a = decode_args(q, lut, codebook_k, codebook_v, codes_k, codes_v, t_cap, hist_len,
                                     max_hist_len, recent_k, recent_v, r_cap, recent_len, softmax_scale, out, lse,
                                     static_cast<uint32_t*>(base),
                                     reinterpret_cast<float*>(static_cast<char*>(base) + kCounterBytes));
    return launch_decode(*dims, batch, q_dtype, recent_dtype, plan, a, stream) == hipSuccess ? PQKV_OK
                                                                                             : PQKV_ERR_HIP;
}
