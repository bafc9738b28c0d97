// Decode kernel builds for 32 subspaces of dimension 4, ad-LUT built in the kernel.
#include "decode_kernel.h"

namespace pqkv {

hipError_t launch_decode_m32d4(const pqkv_dims& d, int32_t batch, pqkv_dtype qt, pqkv_dtype rt, const DecodePlan& plan,
                         const DecodeArgs& a, hipStream_t stream) {
    return launch_family<32, 4, false>(d, batch, qt, rt, plan, a, stream);
}

}  // namespace pqkv

#ifdef PQKV_TIMELINE
// Probe builds only: point the 32-subspace, d_sub 4 kernels' stamps at `buf` (NULL: off).
extern "C" int pqkv_timeline_set_m32d4(void* buf) {
    return (int)hipMemcpyToSymbol(HIP_SYMBOL(pqkv::g_timeline), &buf, sizeof(buf));
}
#endif
