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
// 8 elements per lane (16-byte bf16 stores; 4 per lane when S > 8), one
// (b, h, block) per group of D/8 lanes, the basis staged in LDS as fp64.
// Writes of R tokens per block dominate the traffic.

#include "basis_dev.h"
#include "internal.h"

namespace cdattn {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats to a packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ inline uint32_t bf16_pair(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// EPL (4 or 8) consecutive output elements, rounded to the view format.
template <int EPL>
__device__ inline void store_out(void *dst, int64_t off, int out, const float (&v)[EPL]) {
  if (out == BF16) {
    uint32_t w[EPL / 2];
#pragma unroll
    for (int k = 0; k < EPL / 2; ++k) w[k] = bf16_pair(v[2 * k], v[2 * k + 1]);
    uint16_t *p = static_cast<uint16_t *>(dst) + off;
    if constexpr (EPL == 8)
      *reinterpret_cast<uint4 *>(p) = make_uint4(w[0], w[1], w[2], w[3]);
    else
      *reinterpret_cast<uint2 *>(p) = make_uint2(w[0], w[1]);
  } else {
    float *p = static_cast<float *>(dst) + off;
#pragma unroll
    for (int k = 0; k < EPL / 4; ++k)
      reinterpret_cast<float4 *>(p)[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
  }
}

// EPL consecutive raw (bf16 / fp32) elements as floats.
template <int EPL>
__device__ inline void load_raw(const void *src, int64_t off, int raw, float (&v)[EPL]) {
  if (raw == BF16) {
    const uint32_t *p = reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(src) + off);
#pragma unroll
    for (int k = 0; k < EPL / 2; ++k) {
      const uint32_t w = p[k];
      v[2 * k] = __uint_as_float(w << 16);
      v[2 * k + 1] = __uint_as_float(w & 0xFFFF0000u);
    }
  } else {
    const float *p = static_cast<const float *>(src) + off;
#pragma unroll
    for (int k = 0; k < EPL; ++k) v[k] = p[k];
  }
}

// One coefficient row's EPL consecutive elements as raw 32-bit words (and
// its scale for int8 rows), then their fp64 values: all rows of a block are
// requested before any is converted, so their loads are in flight together.
template <int RF, int EPL>
struct RowWords {
  static constexpr int NW = RF == I8 ? EPL / 4 : (RF == BF16 ? EPL / 2 : EPL);
  uint32_t w[NW];
  float sc;
  __device__ inline void load(const void *rows, const float *scales, int64_t row, int D, int d0) {
    const uint32_t *p = reinterpret_cast<const uint32_t *>(static_cast<const char *>(rows) +
                                                           (row * D + d0) * (RF == I8 ? 1 : (RF == BF16 ? 2 : 4)));
#pragma unroll
    for (int k = 0; k < NW; ++k) w[k] = p[k];
    sc = RF == I8 ? scales[row] : 1.0f;
  }
  __device__ inline void values(double (&c)[EPL]) const {
    if constexpr (RF == I8) {
      const double s = (double)sc;
#pragma unroll
      for (int k = 0; k < NW; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) c[4 * k + e] = (double)(int)(int8_t)(w[k] >> (8 * e)) * s;   // exact
    } else if constexpr (RF == BF16) {
#pragma unroll
      for (int k = 0; k < NW; ++k) {
        c[2 * k] = (double)__uint_as_float(w[k] << 16);
        c[2 * k + 1] = (double)__uint_as_float(w[k] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) c[e] = (double)__uint_as_float(w[e]);
    }
  }
};

// Grid: x = chunks of items, y = kv head, z = batch row.  Item k of (b, h) is
// block blk0 + k (decoded) for k < nblk; item nblk copies the raw tail when
// n_copy > 0.  A group of D/EPL lanes takes one item, EPL elements each; the
// threads past the last whole group (when D/EPL does not divide 256) take no
// item.
template <int RF, int SP, int EPL>
__global__ __launch_bounds__(256) void view_kernel(ViewArgs a) {
  __shared__ double sA[kMaxR * SP];   // A[i][j] as fp64, zero past column S
  constexpr int NAU = (kMaxR * SP + 255) / 256;   // basis entries staged per thread
  const int lpi = a.D / EPL;                     // lanes per item
  const int ipw = 256 / lpi;                     // items per workgroup
  const int64_t k = (int)threadIdx.x < ipw * lpi ? (int64_t)blockIdx.x * ipw + threadIdx.x / lpi : INT64_MAX;
  const int d0 = EPL * (threadIdx.x % lpi);
  const int64_t h = blockIdx.y, b = blockIdx.z;
  const int64_t bh = b * a.H + h;
  const int R = a.R, S = a.S;
  // The basis entries (from the table) and the block's coefficient rows are
  // requested together (rows past S repeat row S-1, in range, and are zeroed
  // below); the basis is staged once its words land.
  const int nA = R * SP;
  float av[NAU];
#pragma unroll
  for (int u = 0; u < NAU; ++u) {
    const int t = (int)threadIdx.x + 256 * u, tc = t < nA ? t : nA - 1;
    const int j = tc % SP;
    av[u] = synthesis_entry(a.png, R, tc / SP, j < S ? j : 0);
  }
  RowWords<RF, EPL> rw[SP];
  if (k < a.nblk) {
    const int64_t row0 = (bh * a.cap + a.blk0 + k) * S;   // first coefficient row of the block
#pragma unroll
    for (int j = 0; j < SP; ++j) rw[j].load(a.rows, a.scales, row0 + (j < S ? j : S - 1), a.D, d0);
  }
#pragma unroll
  for (int u = 0; u < NAU; ++u) {
    const int t = (int)threadIdx.x + 256 * u;
    if (t < nA) sA[t] = t % SP < S ? (double)av[u] : 0.0;
  }
  __syncthreads();
  if (k < a.nblk) {
    const int64_t tbase = b * a.o_sb + h * a.o_sh + (k * R + a.o_t0) * a.o_st + d0;
    if constexpr (SP <= 16) {
      double c[SP][EPL];
#pragma unroll
      for (int j = 0; j < SP; ++j) {
        rw[j].values(c[j]);
        if (j >= S) {
#pragma unroll
          for (int e = 0; e < EPL; ++e) c[j][e] = 0.0;
        }
      }
#pragma unroll 2
      for (int i = 0; i < a.tok_limit; ++i) {
#pragma clang fp contract(off)   // products and sums rounded separately (the contract)
        double x[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) x[e] = 0.0;
        // Columns j >= S add 0 * 0 = +0.0, which leaves x unchanged: x starts
        // at +0.0 and round-to-nearest sums never produce -0.0 from it.
#pragma unroll
        for (int j = 0; j < SP; ++j) {
          const double Aij = sA[i * SP + j];
#pragma unroll
          for (int e = 0; e < EPL; ++e) x[e] = x[e] + Aij * c[j][e];
        }
        float o[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] = (float)x[e];
        store_out<EPL>(a.dst, tbase + i * a.o_st, a.out, o);
      }
    } else {
      // more than 16 kept rows: the rows stay as stored words and each is
      // widened where it is used (the same products and sums, in the same
      // order, without holding SP x EPL doubles)
      for (int i = 0; i < a.tok_limit; ++i) {
#pragma clang fp contract(off)   // products and sums rounded separately (the contract)
        double x[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) x[e] = 0.0;
#pragma unroll
        for (int j = 0; j < SP; ++j) {
          double cj[EPL];
          rw[j].values(cj);
          const double Aij = sA[i * SP + j];
#pragma unroll
          for (int e = 0; e < EPL; ++e) x[e] = x[e] + Aij * (j < S ? cj[e] : 0.0);
        }
        float o[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] = (float)x[e];
        store_out<EPL>(a.dst, tbase + i * a.o_st, a.out, o);
      }
    }
  } else if (k == a.nblk && a.n_copy > 0) {
    const int64_t src = bh * (int64_t)R * a.D + d0;
    const int64_t dst = b * a.o_sb + h * a.o_sh + (a.nblk * R + a.o_t0) * a.o_st + d0;
    for (int i = 0; i < a.n_copy; ++i) {
      float v[EPL];
      load_raw<EPL>(a.tail, src + (int64_t)i * a.D, a.raw, v);
      store_out<EPL>(a.dst, dst + i * a.o_st, a.out, v);
    }
  }
}

// Batch gather: unit u = (i, h) of the destination copies the archived rows,
// their scales and the R tail slots of source row idx[i], head h, in words
// of W bytes (16, or 8 when a slab of int8 rows with head_dim % 16 == 8 and
// an odd row count is not a multiple of 16 bytes).
template <typename W>
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs g) {
  const int64_t u = blockIdx.y;                          // i * H + h within this launch
  const int64_t i = g.i0 + u / g.H, h = u % g.H;
  const int64_t sb = g.idx[u / g.H];
  const int64_t s_bh = sb * g.H + h, d_bh = i * g.H + h;
  const int64_t stride = (int64_t)gridDim.x * 256;
  const int64_t t0 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  {   // rows: the first n_blocks*S*D*eb bytes of the (b, h) slab
    const W *src = reinterpret_cast<const W *>(static_cast<const char *>(g.src_rows) + s_bh * g.slab_bytes);
    W *dst = reinterpret_cast<W *>(static_cast<char *>(g.dst_rows) + d_bh * g.dst_slab_bytes);
    for (int64_t k = t0; k < g.row_bytes / (int64_t)sizeof(W); k += stride) dst[k] = src[k];
  }
  if (g.src_scales) {
    const float *src = g.src_scales + s_bh * g.scale_slab;
    float *dst = g.dst_scales + d_bh * g.dst_scale_slab;
    for (int64_t k = t0; k < g.n_scales; k += stride) dst[k] = src[k];
  }
  {   // tail: all R slots
    const W *src = reinterpret_cast<const W *>(static_cast<const char *>(g.src_tail) + s_bh * g.tail_bytes);
    W *dst = reinterpret_cast<W *>(static_cast<char *>(g.dst_tail) + d_bh * g.tail_bytes);
    for (int64_t k = t0; k < g.tail_bytes / (int64_t)sizeof(W); k += stride) dst[k] = src[k];
  }
}

template <int RF>
int launch_view_rf(int SP, const ViewArgs &a, dim3 grid, hipStream_t stream) {
  switch (SP) {
    case 2: hipLaunchKernelGGL((view_kernel<RF, 2, 8>), grid, dim3(256), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((view_kernel<RF, 4, 8>), grid, dim3(256), 0, stream, a); break;
    case 8: hipLaunchKernelGGL((view_kernel<RF, 8, 8>), grid, dim3(256), 0, stream, a); break;
    case 16: hipLaunchKernelGGL((view_kernel<RF, 16, 4>), grid, dim3(256), 0, stream, a); break;
    case 32: hipLaunchKernelGGL((view_kernel<RF, 32, 4>), grid, dim3(256), 0, stream, a); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace

int launch_view(const ViewArgs &a, hipStream_t stream) {
  const int SP = a.S <= 2 ? 2 : (a.S <= 4 ? 4 : (a.S <= 8 ? 8 : (a.S <= 16 ? 16 : 32)));
  const int EPL = SP >= 16 ? 4 : 8;
  const int64_t items = a.nblk + (a.n_copy > 0 ? 1 : 0);   // per (b, h)
  const int64_t per_wg = 256 / (a.D / EPL);
  const int64_t gx = (items + per_wg - 1) / per_wg;
  const int64_t B = a.BH / a.H;
  if (gx == 0) return 0;
  if (gx > 0x7FFFFFFF || a.H > 65535 || B > 65535) return -1;
  const dim3 grid((unsigned)gx, (unsigned)a.H, (unsigned)B);
  switch (a.rf) {
    case I8: return launch_view_rf<I8>(SP, a, grid, stream);
    case BF16: return launch_view_rf<BF16>(SP, a, grid, stream);
    case F32: return launch_view_rf<F32>(SP, a, grid, stream);
    default: return -1;
  }
}

int launch_gather(const GatherArgs &g, int64_t n_units, hipStream_t stream) {
  if (n_units == 0) return 0;
  const int64_t work = g.row_bytes / 16 > g.tail_bytes / 16 ? g.row_bytes / 16 : g.tail_bytes / 16;
  // about one word per thread: a grid-stride loop copies word by word (each
  // store waits for its load), so the grid, not the loop, carries the
  // parallelism (a cap of 64 workgroups per unit left 16 round trips per
  // thread with one batch row)
  int64_t gx = (work + 255) / 256;
  if (gx < 1) gx = 1;
  if (gx > 1024) gx = 1024;
  const bool w16 = (g.slab_bytes | g.dst_slab_bytes | g.row_bytes | g.tail_bytes) % 16 == 0;
  if (w16)
    hipLaunchKernelGGL(gather_kernel<uint4>, dim3((unsigned)gx, (unsigned)n_units), dim3(256), 0, stream, g);
  else
    hipLaunchKernelGGL(gather_kernel<uint2>, dim3((unsigned)gx, (unsigned)n_units), dim3(256), 0, stream, g);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace cdattn
