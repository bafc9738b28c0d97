// Decode kernel builds for 64 subspaces of dimension 2, ad-LUT built in the kernel.
#include "decode_kernel.h"

namespace pqkv {

hipError_t launch_decode_m64d2(const pqkv_dims& d, int32_t batch, pqkv_dtype qt, pqkv_dtype rt, const DecodePlan& plan,
                         const DecodeArgs& a, hipStream_t stream) {
    return launch_family<64, 2, false>(d, batch, qt, rt, plan, a, stream);
}

}  // namespace pqkv

#ifdef PQKV_TIMELINE
// Probe builds only: point the 64-subspace kernels' stamps at `buf` (NULL: off).
extern "C" int pqkv_timeline_set_m64d2(void* buf) {
    return (int)hipMemcpyToSymbol(HIP_SYMBOL(pqkv::g_timeline), &buf, sizeof(buf));
}
#endif
