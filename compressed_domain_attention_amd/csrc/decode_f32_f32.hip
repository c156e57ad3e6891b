// Decode-attention kernels for f32 key rows and f32 value rows
// (instantiations of decode_impl.h for every head_dim, group size and
// padded kept-row count).
#include "decode_impl.h"

namespace cdattn {
int launch_decode_f32_f32(int D, int GS, int SP, const DecodeArgs &a, int64_t n_wg, hipStream_t stream) {
  return dec::launch_fmt<F32, F32>(D, GS, SP, a, n_wg, stream);
}
}  // namespace cdattn
