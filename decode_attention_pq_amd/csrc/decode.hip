// Decode dispatch: the kernel family of the call's shape and table source (each
// family is built in a translation unit of its own, decode_m*.hip).
#include "pqkv_internal.h"

namespace pqkv {

hipError_t launch_decode_m64d2(const pqkv_dims& d, int32_t batch, pqkv_dtype qt, pqkv_dtype rt,
                          const DecodePlan& plan, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_m64d2_lut(const pqkv_dims& d, int32_t batch, pqkv_dtype qt, pqkv_dtype rt,
                          const DecodePlan& plan, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_m32d4(const pqkv_dims& d, int32_t batch, pqkv_dtype qt, pqkv_dtype rt,
                          const DecodePlan& plan, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_m32d4_lut(const pqkv_dims& d, int32_t batch, pqkv_dtype qt, pqkv_dtype rt,
                          const DecodePlan& plan, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_m32d2(const pqkv_dims& d, int32_t batch, pqkv_dtype qt, pqkv_dtype rt,
                          const DecodePlan& plan, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_m32d2_lut(const pqkv_dims& d, int32_t batch, pqkv_dtype qt, pqkv_dtype rt,
                          const DecodePlan& plan, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_m16d4(const pqkv_dims& d, int32_t batch, pqkv_dtype qt, pqkv_dtype rt,
                          const DecodePlan& plan, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_m16d4_lut(const pqkv_dims& d, int32_t batch, pqkv_dtype qt, pqkv_dtype rt,
                          const DecodePlan& plan, const DecodeArgs& a, hipStream_t stream);

hipError_t launch_decode(const pqkv_dims& d, int32_t batch, pqkv_dtype qt, pqkv_dtype rt,
                         const DecodePlan& plan, const DecodeArgs& a, hipStream_t stream) {
    const int M = d.head_dim / d.d_sub;
    const bool ext = a.lut != nullptr;
    if (M == 64) return (ext ? launch_decode_m64d2_lut : launch_decode_m64d2)(d, batch, qt, rt, plan, a, stream);
    if (M == 32 && d.d_sub == 4)
        return (ext ? launch_decode_m32d4_lut : launch_decode_m32d4)(d, batch, qt, rt, plan, a, stream);
    if (M == 32) return (ext ? launch_decode_m32d2_lut : launch_decode_m32d2)(d, batch, qt, rt, plan, a, stream);
    return (ext ? launch_decode_m16d4_lut : launch_decode_m16d4)(d, batch, qt, rt, plan, a, stream);
}

}  // namespace pqkv
