// Decode-attention kernels for bf16 key rows and i8 value rows, rows whose head_dim is narrower than the compute width (64, 128 or 256: runtime row pitch, masked query columns):
// instantiations of decode_impl.h for every compute width, group size and
// padded kept-row count.
#include "decode_impl.h"

namespace cdattn {
int launch_decode_bf16_i8_pad(int D, int GS, int SP, const DecodeArgs &a, int64_t n_wg, hipStream_t stream) {
  return dec::by_dim<BF16, I8>(D, GS, SP, dec::LaunchOp<false>{a, n_wg, stream});
}
int resident_decode_bf16_i8_pad(int D, int GS, int SP) {
  return dec::by_dim<BF16, I8>(D, GS, SP, dec::ResidentOp<false>{});
}
}  // namespace cdattn
