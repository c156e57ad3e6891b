// Decode-attention kernels for f32 key rows and bf16 value rows, rows whose head_dim is the compute width (64, 128 or 256):
// instantiations of decode_impl.h for every compute width, group size and
// padded kept-row count.
#include "decode_impl.h"

namespace cdattn {
int launch_decode_f32_bf16(int D, int GS, int SP, const DecodeArgs &a, int64_t n_wg, hipStream_t stream) {
  return dec::by_dim<F32, BF16>(D, GS, SP, dec::LaunchOp<true>{a, n_wg, stream});
}
int resident_decode_f32_bf16(int D, int GS, int SP) {
  return dec::by_dim<F32, BF16>(D, GS, SP, dec::ResidentOp<true>{});
}
}  // namespace cdattn
