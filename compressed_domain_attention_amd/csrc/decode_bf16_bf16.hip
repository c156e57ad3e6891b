// Decode-attention kernels for bf16 key rows and bf16 value rows
// (instantiations of decode_impl.h for every head_dim, group size and
// padded kept-row count).
#include "decode_impl.h"

namespace cdattn {
int launch_decode_bf16_bf16(int D, int GS, int SP, const DecodeArgs &a, int64_t n_wg, hipStream_t stream) {
  return dec::launch_fmt<BF16, BF16>(D, GS, SP, a, n_wg, stream);
}
}  // namespace cdattn
