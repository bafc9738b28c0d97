// Decode kernel builds for 64 subspaces of dimension 2, ad-LUT read from the materialised table.
#include "decode_kernel.h"

namespace pqkv {

hipError_t launch_decode_m64d2_lut(const pqkv_dims& d, int32_t batch, pqkv_dtype qt, pqkv_dtype rt, const DecodePlan& plan,
                         const DecodeArgs& a, hipStream_t stream) {
    return launch_family<64, 2, true>(d, batch, qt, rt, plan, a, stream);
}

}  // namespace pqkv
