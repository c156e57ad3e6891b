// Structural operations on the compressed archive: the materialised view,
// the exact crop and the batch gather.
//
// Method: flashcodec-kv 1.0.0, cache.py ``_CodecStream``:
//  * ``read`` / ``_decode_pending``: the decoded view of a stream is the
//    archived blocks decoded (X_hat = M^T C, README "Math") followed by the
//    raw tail; it is memoised and append-only, so a read decodes only the
//    blocks archived since the previous one.
//  * ``crop``: trailing tokens are removed without re-compressing anything;
//    when the cut falls inside the archive, the boundary block leaves it and
//    its first tokens come back as the raw tail, taken from the decoded view.
//  * ``select_batch``: rows of the batch axis are gathered (beam reorder).
//
// Arithmetic contract of the decoded view (bit-exact, shared with the CPU
// reference by specification only):
//   x_hat[n*R + i][d] = sum over j = 0..S-1, in that order, starting from
//                       +0.0, of fp64(A[i][j]) * c_hat[j][d]
//   with c_hat = fp64(code) * fp64(scale) for int8 rows (exact) and the
//   stored value for float rows; every product and sum is a separately
//   rounded fp64 operation (no fused multiply-add: A * c_hat is not exact).
//   fp32 output: fp32(x_hat) (RNE); bf16 output: bf16(fp32(x_hat)) (RNE, RNE).
//
// The view is streaming work (S fp64 multiply-adds per output element, about
// 4 flop per byte moved at S = 4): plain fp64 VALU, lanes along head_dim,
// 4 elements per lane, one (b, h, block) per group of D/4 lanes.  Writes of
// R tokens per block dominate the traffic.

#include "internal.h"

namespace cdattn {
namespace {

__device__ inline uint16_t bf16_of(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Four consecutive output elements, rounded to the view format and stored.
__device__ inline void store4(void *dst, int64_t off, int out, float a, float b, float c, float d) {
  if (out == BF16) {
    const uint32_t lo = (uint32_t)bf16_of(a) | ((uint32_t)bf16_of(b) << 16);
    const uint32_t hi = (uint32_t)bf16_of(c) | ((uint32_t)bf16_of(d) << 16);
    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(dst) + off) = make_uint2(lo, hi);
  } else {
    *reinterpret_cast<float4 *>(static_cast<float *>(dst) + off) = make_float4(a, b, c, d);
  }
}

// Four consecutive raw (bf16 / fp32) elements as floats.
__device__ inline float4 load4_raw(const void *src, int64_t off, int raw) {
  if (raw == BF16) {
    const uint2 w = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(src) + off);
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                       __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u));
  }
  return *reinterpret_cast<const float4 *>(static_cast<const float *>(src) + off);
}

// fp64 values of four consecutive elements of one coefficient row.
template <int RF>
__device__ inline void load_row4(const void *rows, const float *scales, int64_t row, int D, int d0,
                                 double (&c)[4]) {
  const int64_t off = row * D + d0;
  if constexpr (RF == I8) {
    const uint32_t w = *reinterpret_cast<const uint32_t *>(static_cast<const int8_t *>(rows) + off);
    const double sc = (double)scales[row];
#pragma unroll
    for (int e = 0; e < 4; ++e) c[e] = (double)(int)(int8_t)(w >> (8 * e)) * sc;   // exact
  } else if constexpr (RF == BF16) {
    const uint2 w = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(rows) + off);
    c[0] = (double)__uint_as_float(w.x << 16);
    c[1] = (double)__uint_as_float(w.x & 0xFFFF0000u);
    c[2] = (double)__uint_as_float(w.y << 16);
    c[3] = (double)__uint_as_float(w.y & 0xFFFF0000u);
  } else {
    const float4 w = *reinterpret_cast<const float4 *>(static_cast<const float *>(rows) + off);
    c[0] = (double)w.x;
    c[1] = (double)w.y;
    c[2] = (double)w.z;
    c[3] = (double)w.w;
  }
}

// Work items: BH * nblk blocks (decoded), then BH tails (copied) when
// copy_tail is set.  A group of D/4 lanes takes one item, 4 elements each.
template <int RF, int SP>
__global__ __launch_bounds__(256) void view_kernel(ViewArgs a) {
  const int lpi = a.D / 4;                       // lanes per item
  const int64_t item = (int64_t)blockIdx.x * (256 / lpi) + threadIdx.x / lpi;
  const int d0 = 4 * (threadIdx.x % lpi);
  const int64_t nb_items = a.BH * a.nblk;
  const int R = a.R, S = a.S;
  if (item < nb_items) {
    const int64_t bh = item / a.nblk, n = a.blk0 + item % a.nblk;
    const int64_t b = bh / a.H, h = bh % a.H;
    const int64_t row0 = (bh * a.cap + n) * S;   // first coefficient row of the block
    double c[SP][4];
#pragma unroll
    for (int j = 0; j < SP; ++j) {
      if (j < S) {
        load_row4<RF>(a.rows, a.scales, row0 + j, a.D, d0, c[j]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) c[j][e] = 0.0;
      }
    }
    const int64_t tbase = b * a.o_sb + h * a.o_sh + ((n - a.blk0) * R + a.o_t0) * a.o_st + d0;
    for (int i = 0; i < a.tok_limit; ++i) {
#pragma clang fp contract(off)   // products and sums rounded separately (the contract)
      double x[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int j = 0; j < SP; ++j) {
        if (j < S) {
          const double Aij = (double)a.A[i * S + j];
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = x[e] + Aij * c[j][e];
        }
      }
      store4(a.dst, tbase + i * a.o_st, a.out, (float)x[0], (float)x[1], (float)x[2], (float)x[3]);
    }
  } else if (item < nb_items + (a.n_copy > 0 ? a.BH : 0)) {
    const int64_t bh = item - nb_items;
    const int64_t b = bh / a.H, h = bh % a.H;
    const int64_t src = bh * (int64_t)R * a.D + d0;
    const int64_t dst = b * a.o_sb + h * a.o_sh + (a.nblk * R + a.o_t0) * a.o_st + d0;
    for (int i = 0; i < a.n_copy; ++i) {
      const float4 v = load4_raw(a.tail, src + (int64_t)i * a.D, a.raw);
      store4(a.dst, dst + i * a.o_st, a.out, v.x, v.y, v.z, v.w);
    }
  }
}

// Batch gather: unit u = (i, h) of the destination copies the archived rows,
// their scales and the R tail slots of source row idx[i], head h.
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs g) {
  const int64_t u = blockIdx.y;                          // i * H + h within this launch
  const int64_t i = g.i0 + u / g.H, h = u % g.H;
  const int64_t sb = g.idx[u / g.H];
  const int64_t s_bh = sb * g.H + h, d_bh = i * g.H + h;
  const int64_t stride = (int64_t)gridDim.x * 256;
  const int64_t t0 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  {   // rows: the first n_blocks*S*D*eb bytes of the (b, h) slab, 16 bytes per lane
    const uint4 *src = reinterpret_cast<const uint4 *>(static_cast<const char *>(g.src_rows) + s_bh * g.slab_bytes);
    uint4 *dst = reinterpret_cast<uint4 *>(static_cast<char *>(g.dst_rows) + d_bh * g.dst_slab_bytes);
    for (int64_t k = t0; k < g.row_bytes / 16; k += stride) dst[k] = src[k];
  }
  if (g.src_scales) {
    const float *src = g.src_scales + s_bh * g.scale_slab;
    float *dst = g.dst_scales + d_bh * g.dst_scale_slab;
    for (int64_t k = t0; k < g.n_scales; k += stride) dst[k] = src[k];
  }
  {   // tail: all R slots
    const uint4 *src = reinterpret_cast<const uint4 *>(static_cast<const char *>(g.src_tail) + s_bh * g.tail_bytes);
    uint4 *dst = reinterpret_cast<uint4 *>(static_cast<char *>(g.dst_tail) + d_bh * g.tail_bytes);
    for (int64_t k = t0; k < g.tail_bytes / 16; k += stride) dst[k] = src[k];
  }
}

template <int RF>
int launch_view_rf(int SP, const ViewArgs &a, int64_t n_wg, hipStream_t stream) {
  switch (SP) {
    case 2: hipLaunchKernelGGL((view_kernel<RF, 2>), dim3((unsigned)n_wg), dim3(256), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((view_kernel<RF, 4>), dim3((unsigned)n_wg), dim3(256), 0, stream, a); break;
    case 8: hipLaunchKernelGGL((view_kernel<RF, 8>), dim3((unsigned)n_wg), dim3(256), 0, stream, a); break;
    case 16: hipLaunchKernelGGL((view_kernel<RF, 16>), dim3((unsigned)n_wg), dim3(256), 0, stream, a); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace

int launch_view(const ViewArgs &a, hipStream_t stream) {
  const int SP = a.S <= 2 ? 2 : (a.S <= 4 ? 4 : (a.S <= 8 ? 8 : 16));
  const int64_t items = a.BH * a.nblk + (a.n_copy > 0 ? a.BH : 0);
  const int64_t per_wg = 256 / (a.D / 4);
  const int64_t n_wg = (items + per_wg - 1) / per_wg;
  if (n_wg == 0) return 0;
  if (n_wg > 0x7FFFFFFF) return -1;
  switch (a.rf) {
    case I8: return launch_view_rf<I8>(SP, a, n_wg, stream);
    case BF16: return launch_view_rf<BF16>(SP, a, n_wg, stream);
    case F32: return launch_view_rf<F32>(SP, a, n_wg, stream);
    default: return -1;
  }
}

int launch_gather(const GatherArgs &g, int64_t n_units, hipStream_t stream) {
  if (n_units == 0) return 0;
  const int64_t work = g.row_bytes / 16 > g.tail_bytes / 16 ? g.row_bytes / 16 : g.tail_bytes / 16;
  int64_t gx = (work + 255) / 256;
  if (gx < 1) gx = 1;
  if (gx > 64) gx = 64;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)gx, (unsigned)n_units), dim3(256), 0, stream, g);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace cdattn
