// Decode kernel builds for 16 subspaces of dimension 4, ad-LUT built in the kernel.
#include "decode_kernel.h"

namespace pqkv {

hipError_t launch_decode_m16d4(const pqkv_dims& d, int32_t batch, pqkv_dtype qt, pqkv_dtype rt, const DecodePlan& plan,
                         const DecodeArgs& a, hipStream_t stream) {
    return launch_family<16, 4, false>(d, batch, qt, rt, plan, a, stream);
}

}  // namespace pqkv
