// Decode-attention kernels for head_dim 256 (instantiations of decode_impl.h).
#include "decode_impl.h"

namespace cdattn {
int launch_decode_d256(int GS, int SP, const DecodeArgs &a, int64_t n_wg, hipStream_t stream) {
  return dec::launch_d<256>(GS, SP, a, n_wg, stream);
}
}  // namespace cdattn
