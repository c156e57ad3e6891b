// Block DCT-II encode of raw key/value tokens into the compressed archive,
// and the single-token append that archives a block when it completes.
//
// Method: flashcodec-kv 1.0.0 README, section "Math" (JPEG item): every
// complete block X of R tokens (R x D) is stored as the S lowest rows of
// C = M X, M the orthonormal DCT-II; README paragraph on 8-bit
// quantisation and cache.py ``_archive_spec``: optional int8 codes with one
// fp32 scale per (block, frequency) row; cache.py ``append``: complete
// blocks are archived, the remainder stays raw in the tail.
//
// Arithmetic contract (bit-exact, shared with the CPU reference by
// specification only):
//   c[j][d] = sum over i = 0..R-1, in that order, starting from +0.0, of
//             fp64(M[j][i]) * fp64(x[i][d])      (products exact in fp64)
//   fp32 rows: fp32(c) (RNE);  bf16 rows: bf16(fp32(c)) (RNE, RNE)
//   int8 rows: a = max_d |c|, scale = fp32(a / 127) (fp64 divide, RNE),
//              code = clamp(rint_even(c / fp64(scale)), -127, 127),
//              scale == 0 -> all codes 0.
// The quotient c / scale is evaluated as c * (1 / scale); within 1e-9 of a
// half-integer it is recomputed with an IEEE fp64 division.  The product
// differs from the correctly rounded quotient by < 6e-14 for |c/scale| <=
// 192 (the largest quotient, reached when a / 127 rounds to an fp32
// subnormal), so both round to the same integer everywhere outside that band.
//
// The encode is streaming work (S fp64 FMAs per input element): plain fp64
// VALU, one wave per block, lanes along head_dim.  MFMA is not used because
// the contract fixes the order of the R additions.

#include "basis_dev.h"
#include "internal.h"

namespace cdattn {
namespace {

__device__ inline uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Load EPL consecutive raw elements (bf16 or fp32) as floats.
template <int EPL>
__device__ inline void load_raw(const void *base, int64_t elem_off, int raw, float (&x)[EPL]) {
  if (raw == BF16) {
    const uint16_t *p = static_cast<const uint16_t *>(base) + elem_off;
    if constexpr (EPL == 1) {
      x[0] = __uint_as_float((uint32_t)p[0] << 16);
    } else if constexpr (EPL == 2) {
      uint32_t w = *reinterpret_cast<const uint32_t *>(p);
      x[0] = __uint_as_float(w << 16);
      x[1] = __uint_as_float(w & 0xFFFF0000u);
    } else {
      uint2 w = *reinterpret_cast<const uint2 *>(p);
      x[0] = __uint_as_float(w.x << 16);
      x[1] = __uint_as_float(w.x & 0xFFFF0000u);
      x[2] = __uint_as_float(w.y << 16);
      x[3] = __uint_as_float(w.y & 0xFFFF0000u);
    }
  } else {
    const float *p = static_cast<const float *>(base) + elem_off;
#pragma unroll
    for (int e = 0; e < EPL; ++e) x[e] = p[e];
  }
}

// The same with the raw format fixed at compile time (no branch, so the
// loads of several tokens stay in flight together).
template <int EPL, int RAW>
__device__ inline void load_raw_t(const void *base, int64_t elem_off, float (&x)[EPL]) {
  if constexpr (RAW == BF16) {
    const uint16_t *p = static_cast<const uint16_t *>(base) + elem_off;
    if constexpr (EPL == 1) {
      x[0] = __uint_as_float((uint32_t)p[0] << 16);
    } else if constexpr (EPL == 2) {
      const uint32_t w = *reinterpret_cast<const uint32_t *>(p);
      x[0] = __uint_as_float(w << 16);
      x[1] = __uint_as_float(w & 0xFFFF0000u);
    } else {
      const uint2 w = *reinterpret_cast<const uint2 *>(p);
      x[0] = __uint_as_float(w.x << 16);
      x[1] = __uint_as_float(w.x & 0xFFFF0000u);
      x[2] = __uint_as_float(w.y << 16);
      x[3] = __uint_as_float(w.y & 0xFFFF0000u);
    }
  } else {
    const float *p = static_cast<const float *>(base) + elem_off;
#pragma unroll
    for (int e = 0; e < EPL; ++e) x[e] = p[e];
  }
}

template <int EPL>
__device__ inline void store_raw(void *base, int64_t elem_off, int raw, const float (&x)[EPL]) {
  if (raw == BF16) {
    uint16_t *p = static_cast<uint16_t *>(base) + elem_off;
#pragma unroll
    for (int e = 0; e < EPL; ++e) p[e] = (uint16_t)(__float_as_uint(x[e]) >> 16);  // exact: x holds bf16 values
  } else {
    float *p = static_cast<float *>(base) + elem_off;
#pragma unroll
    for (int e = 0; e < EPL; ++e) p[e] = x[e];
  }
}

// Wave maximum of non-negative doubles.  Their bit patterns order like
// unsigned 64-bit integers, so both halves move through DPP / gfx950
// half-wave swaps (no LDS) and the larger pattern wins.
template <int CTRL>
__device__ inline uint64_t dpp64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}
__device__ inline uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ inline double wave_max_f64(double v) {
  uint64_t u = __builtin_bit_cast(uint64_t, v);
  u = umax64(u, dpp64<0xB1>(u));    // quad_perm [1,0,3,2]
  u = umax64(u, dpp64<0x4E>(u));    // quad_perm [2,3,0,1]
  u = umax64(u, dpp64<0x141>(u));   // row_half_mirror
  u = umax64(u, dpp64<0x140>(u));   // row_mirror
  {
    const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)u, (uint32_t)u, false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
    u = umax64(((uint64_t)hi[0] << 32) | lo[0], ((uint64_t)hi[1] << 32) | lo[1]);
  }
  {
    const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)u, (uint32_t)u, false, false);
    const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
    u = umax64(((uint64_t)hi[0] << 32) | lo[0], ((uint64_t)hi[1] << 32) | lo[1]);
  }
  return __builtin_bit_cast(double, u);
}

__device__ inline int8_t quantise(double c, float s32, double inv) {
  if (s32 == 0.0f) return 0;
  double y = c * inv;
  double r = rint(y);
  if (fabs(y - floor(y) - 0.5) < 1e-9) r = rint(c / (double)s32);
  // clamp to [-127, 127]: the lower bound in fp64, the upper bound on the
  // integer.  For finite c, |c / scale| is at most 127 up to the rounding of
  // the scale, i.e. about 127 * 1.5 ~ 190 when a / 127 is an fp32 subnormal,
  // which fits an int.  Non-finite input has no defined codes (the contract
  // covers finite tokens): fmax keeps r from being NaN so the conversion
  // stays defined.
  r = fmax(r, -127.0);
  return (int8_t)min((int)r, 127);
}

// Rows j0 .. j0+JP-1 of block `n` (call-relative) of stream row (b, h): one
// wave, lane holding head_dim elements [d0, d0+EPL) (d0c: where it reads
// them; lanes past head_dim read column 0 and store nothing).  U tokens per
// round, their loads all in flight together (token i comes from src0 below
// split_i, else from src1; indices past R repeat token R-1 and are not
// used).  Products are added in token order (the contract's summation
// order).  A round's basis entries are requested from the table with its
// tokens, lane jj * U + u of mr holding row j0 + jj, token i0 + u, and each
// product takes its entry with a lane read at a constant lane (no scalar
// load and wait per product).
template <int EPL, int JP, int U, int RAW>
__device__ void encode_sums(const EncodeArgs &a, int j0, int64_t b, int64_t h, int64_t n, int d0c,
                            double (&c)[JP][EPL]) {
  const int R = a.R, S = a.S;
  const int lane = threadIdx.x & 63;
  constexpr int NM = (JP * U + 63) / 64;
  for (int i0 = 0; i0 < R; i0 += U) {
    float mr[NM];
#pragma unroll
    for (int q = 0; q < NM; ++q) {
      const int l = 64 * q + lane, jj = l / U, u = l % U, j = j0 + jj, i = i0 + u;
      const bool in = jj < JP && j < S && i < R;
      const float m = analysis_entry(a.png, R, in ? j : 0, in ? i : 0);   // unconditional load
      mr[q] = in ? m : 0.0f;
    }
    float x[U][EPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u < R ? i0 + u : R - 1;
      const bool f0 = i < a.split_i;
      const void *src = f0 ? a.src0 : a.src1;
      const int64_t off = f0 ? b * a.s0_b + h * a.s0_h + (n * R + i) * a.s0_t + d0c : b * a.s1_b + h * a.s1_h + d0c;
      load_raw_t<EPL, RAW>(src, off, x[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u;
      if (i < R) {
#pragma unroll
        for (int jj = 0; jj < JP; ++jj) {
          const int j = j0 + jj;
          if (j < S) {
            const double m = (double)__int_as_float(
                __builtin_amdgcn_readlane(__float_as_int(mr[(jj * U + u) / 64]), (jj * U + u) % 64));
#pragma unroll
            for (int e = 0; e < EPL; ++e) c[jj][e] = fma(m, (double)x[u][e], c[jj][e]);
          }
        }
      }
    }
  }
}

// Encode block `n` (call-relative) of stream row (b, h) into archive slot
// a.n0 + n, JP rows per pass over the tokens.  One wave; lane owns head_dim
// elements [lane*EPL, lane*EPL+EPL).  U tokens' loads in flight per round:
// sixteen for a lone block (latency bound), eight when many blocks are in
// flight.
template <int EPL, int JP, bool PIPE>
__device__ void encode_block(const EncodeArgs &a, int64_t b, int64_t h, int64_t n, int lane) {
  const int d0 = lane * EPL;
  const bool dlive = d0 < a.D;
  const int d0c = dlive ? d0 : 0;
  const int S = a.S;
  constexpr int U = PIPE ? 16 : 8;
  const int64_t slot = (b * a.H + h) * a.cap + a.n0 + n;
  for (int j0 = 0; j0 < S; j0 += JP) {
    double c[JP][EPL];
#pragma unroll
    for (int jj = 0; jj < JP; ++jj)
#pragma unroll
      for (int e = 0; e < EPL; ++e) c[jj][e] = 0.0;  // +0.0
    if (a.raw == BF16)
      encode_sums<EPL, JP, U, BF16>(a, j0, b, h, n, d0c, c);
    else
      encode_sums<EPL, JP, U, F32>(a, j0, b, h, n, d0c, c);
#pragma unroll
    for (int jj = 0; jj < JP; ++jj) {
      const int j = j0 + jj;
      if (j >= S) break;
      const int64_t row = (slot * S + j) * a.D + d0;
      if (a.fmt == F32) {
        if (dlive) {
          float *p = static_cast<float *>(a.rows) + row;
#pragma unroll
          for (int e = 0; e < EPL; ++e) p[e] = (float)c[jj][e];
        }
      } else if (a.fmt == BF16) {
        if (dlive) {
          uint16_t *p = static_cast<uint16_t *>(a.rows) + row;
#pragma unroll
          for (int e = 0; e < EPL; ++e) p[e] = bf16_rne((float)c[jj][e]);
        }
      } else {
        double amax = 0.0;
#pragma unroll
        for (int e = 0; e < EPL; ++e) amax = fmax(amax, fabs(c[jj][e]));
        amax = wave_max_f64(dlive ? amax : 0.0);
        const float s32 = (float)(amax / 127.0);
        const double inv = s32 != 0.0f ? 1.0 / (double)s32 : 0.0;
        if (dlive) {
          int8_t *p = static_cast<int8_t *>(a.rows) + row;
#pragma unroll
          for (int e = 0; e < EPL; ++e) p[e] = quantise(c[jj][e], s32, inv);
        }
        if (lane == 0) a.scales[slot * S + j] = s32;
      }
    }
  }
}

// The raw remainder of an encode call into tail slots 0 .. n_copy-1, eight
// tokens' loads in flight per round.
template <int EPL, int RAW>
__device__ void copy_tail(const EncodeArgs &a, int64_t b, int64_t h, int64_t bh, int lane) {
  const int d0 = lane * EPL;
  if (d0 >= a.D) return;
  for (int i0 = 0; i0 < a.n_copy; i0 += 8) {
    float x[8][EPL];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u < a.n_copy ? i0 + u : a.n_copy - 1;
      load_raw_t<EPL, RAW>(a.src0, b * a.s0_b + h * a.s0_h + (a.n_new * a.R + i) * a.s0_t + d0, x[u]);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (i0 + u < a.n_copy) store_raw<EPL>(a.tail, ((bh * a.R) + i0 + u) * a.D + d0, RAW, x[u]);
  }
}

// Grid: x = (b, h) * per_bh + wave-group; each wave one block (or the tail copy).
template <int EPL, int JP>
__global__ __launch_bounds__(64 * kEncodeWaves) void encode_kernel(EncodeArgs a, int64_t per_bh) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t bh = blockIdx.x / per_bh;
  const int64_t n = (blockIdx.x % per_bh) * kEncodeWaves + wave;
  const int64_t b = bh / a.H, h = bh % a.H;
  if (n < a.n_new) {
    encode_block<EPL, JP, false>(a, b, h, n, lane);
  } else if (n == a.n_new && a.n_copy > 0) {
    // raw remainder -> tail slots 0 .. n_copy-1, verbatim
    if (a.raw == BF16)
      copy_tail<EPL, BF16>(a, b, h, bh, lane);
    else
      copy_tail<EPL, F32>(a, b, h, bh, lane);
  }
}

// Maximum of non-negative doubles over aligned groups of LPB lanes (8, 16
// or 32), the same bit-pattern ordering as wave_max_f64.
template <int LPB>
__device__ inline double group_max_f64(double v) {
  uint64_t u = __builtin_bit_cast(uint64_t, v);
  u = umax64(u, dpp64<0xB1>(u));    // quad_perm [1,0,3,2]
  u = umax64(u, dpp64<0x4E>(u));    // quad_perm [2,3,0,1]
  u = umax64(u, dpp64<0x141>(u));   // row_half_mirror: eight lanes
  if constexpr (LPB >= 16) u = umax64(u, dpp64<0x140>(u));   // row_mirror: sixteen
  if constexpr (LPB >= 32) {
    const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)u, (uint32_t)u, false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
    u = umax64(((uint64_t)hi[0] << 32) | lo[0], ((uint64_t)hi[1] << 32) | lo[1]);
  }
  return __builtin_bit_cast(double, u);
}

// Bulk encode with wide lanes: a lane owns eight consecutive head_dim
// elements of one block (16-byte token loads), LPB = D/8 lanes per block and
// 64/LPB blocks per wave, blocks numbered across (b, h) rows.  All RP (>= R)
// token loads are in flight together.  The S coefficient rows are then
// formed JC at a time: each token is widened to fp64 once per pass and
// feeds the JC rows' sums, each element by the same fp64 FMA chain in token
// order as encode_block, so rows, codes and scales are identical.  A pass
// past row S - 1 computes sums that are never stored (zero entries past row R - 1).
// Each token's sums sit behind its own (uniform) u < R test even when
// R == RP: the branch keeps the scheduler from widening every token at once,
// which would take twice the registers.  Waves past the block waves copy the
// raw remainder of one (b, h) row each.  A pass's basis entries sit in one
// register (lane jj * RP + u holds row j0 + jj, token u), requested at the
// start of the pass (for the first pass right after the tokens), and each FMA
// takes its entry with a lane read at a constant lane: no memory wait inside
// the token loop.  A
// head_dim below the compute width LPB * 8 leaves the lanes past it reading
// column 0 and storing nothing.
template <int LPB, int RP, int JC, int RAW>
__global__ __launch_bounds__(64 * kEncodeWaves) __attribute__((amdgpu_waves_per_eu(
    RAW == BF16 ? (RP == 8 ? 4 : 3) : (RP == 8 ? 3 : 2)))) void encode_wide_kernel(EncodeArgs a, int64_t BH,
                                                                         int64_t block_waves) {
  constexpr int DP = LPB * 8, BPW = 64 / LPB, EPL = DP / 64;
  constexpr int WPT = RAW == BF16 ? 1 : 2;   // 16-byte words per token and lane
  const int lane = threadIdx.x & 63;
  const int64_t gw = (int64_t)blockIdx.x * kEncodeWaves + (threadIdx.x >> 6);
  const int R = a.R, S = a.S;
  if (gw >= block_waves) {
    const int64_t bh = gw - block_waves;
    if (bh < BH && a.n_copy > 0) copy_tail<EPL, RAW>(a, bh / a.H, bh % a.H, bh, lane);
    return;
  }
  const int64_t total = BH * a.n_new;
  const int64_t gb = gw * BPW + lane / LPB;
  const bool live = gb < total;
  const int64_t gbc = live ? gb : total - 1;
  const int64_t bh = gbc / a.n_new, n = gbc % a.n_new;
  const int64_t b = bh / a.H, h = bh % a.H;
  const int d0 = (lane % LPB) * 8;
  const bool dlive = d0 < a.D;
  const char *src = static_cast<const char *>(a.src0) +
                    (b * a.s0_b + h * a.s0_h + n * R * a.s0_t + (dlive ? d0 : 0)) * (RAW == BF16 ? 2 : 4);
  const int64_t tstride = a.s0_t * (RAW == BF16 ? 2 : 4);
  static_assert(JC * RP <= 64, "a pass's basis entries fit one register");
  // entries of the pass that starts at row j0 (unconditional load: no branch around it)
  auto pass_entries = [&](int j0) {
    const int jj = lane / RP, u = lane % RP, j = j0 + jj;
    const bool in = jj < JC && u < R && j < R;
    const float m = analysis_entry(a.png, R, in ? j : 0, in ? u : 0);
    return in ? m : 0.0f;
  };
  uint4 x[RP][WPT];
#pragma unroll
  for (int u = 0; u < RP; ++u) {
    const int i = u < R ? u : R - 1;
#pragma unroll
    for (int w = 0; w < WPT; ++w) x[u][w] = *reinterpret_cast<const uint4 *>(src + i * tstride + 16 * w);
  }
  auto elem = [&](int u, int e) -> double {
    if constexpr (RAW == BF16) {
      const uint32_t wd = (&x[u][0].x)[e / 2];
      return (double)__uint_as_float(e % 2 ? wd & 0xFFFF0000u : wd << 16);
    } else {
      return (double)__uint_as_float((&x[u][e / 4].x)[e % 4]);
    }
  };
  const int64_t slot = (b * a.H + h) * a.cap + a.n0 + n;
  for (int j0 = 0; j0 < S; j0 += JC) {
    const float mcur = pass_entries(j0);   // the first pass's requested after the tokens
    double c[JC][8];
#pragma unroll
    for (int jj = 0; jj < JC; ++jj)
#pragma unroll
      for (int e = 0; e < 8; ++e) c[jj][e] = 0.0;   // +0.0
#pragma unroll
    for (int u = 0; u < RP; ++u) {
      if (u < R) {
        double xd[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) xd[e] = elem(u, e);
#pragma unroll
        for (int jj = 0; jj < JC; ++jj) {
          const double m = (double)__int_as_float(__builtin_amdgcn_readlane(__float_as_int(mcur), jj * RP + u));
#pragma unroll
          for (int e = 0; e < 8; ++e) c[jj][e] = fma(m, xd[e], c[jj][e]);
        }
      }
    }
#pragma unroll
    for (int jj = 0; jj < JC; ++jj) {
      const int j = j0 + jj;
      if (j >= S) break;
      const int64_t row = (slot * S + j) * a.D + d0;
      if (a.fmt == F32) {
        if (live && dlive) {
          float4 *p = reinterpret_cast<float4 *>(static_cast<float *>(a.rows) + row);
          p[0] = make_float4((float)c[jj][0], (float)c[jj][1], (float)c[jj][2], (float)c[jj][3]);
          p[1] = make_float4((float)c[jj][4], (float)c[jj][5], (float)c[jj][6], (float)c[jj][7]);
        }
      } else if (a.fmt == BF16) {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          w[k] = (uint32_t)bf16_rne((float)c[jj][2 * k]) | ((uint32_t)bf16_rne((float)c[jj][2 * k + 1]) << 16);
        if (live && dlive)
          *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(a.rows) + row) = make_uint4(w[0], w[1], w[2], w[3]);
      } else {
        double amax = 0.0;
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmax(amax, fabs(c[jj][e]));
        amax = group_max_f64<LPB>(dlive ? amax : 0.0);
        const float s32 = (float)(amax / 127.0);
        const double inv = s32 != 0.0f ? 1.0 / (double)s32 : 0.0;
        uint32_t w[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e / 4] |= (uint32_t)(uint8_t)quantise(c[jj][e], s32, inv) << (8 * (e % 4));
        if (live && dlive) *reinterpret_cast<uint2 *>(static_cast<int8_t *>(a.rows) + row) = make_uint2(w[0], w[1]);
        if (live && lane % LPB == 0) a.scales[slot * S + j] = s32;
      }
    }
    // The token words count as changed here, so a second pass widens them
    // again instead of the first pass hoisting RP x 8 doubles.
#pragma unroll
    for (int u = 0; u < RP; ++u)
#pragma unroll
      for (int w = 0; w < WPT; ++w) asm volatile("" : "+v"(x[u][w].x), "+v"(x[u][w].y), "+v"(x[u][w].z), "+v"(x[u][w].w));
  }
}

// Grid: x = (b, h), y = stream (0 keys, 1 values); one wave each.
template <int EPL, int JP>
__global__ __launch_bounds__(64) void append_kernel(AppendArgs A) {
  const EncodeArgs &a = A.e[blockIdx.y];
  const int lane = threadIdx.x;
  const int64_t bh = blockIdx.x;
  const int64_t b = bh / a.H, h = bh % a.H;
  if (A.complete) {
    // tail slots 0..R-2 plus the new token form the block; slot R-1 of the
    // tail is not written since the tail empties.
    encode_block<EPL, JP, true>(a, b, h, 0, lane);
  } else {
    const int d0 = lane * EPL;
    if (d0 >= a.D) return;
    float x[EPL];
    load_raw<EPL>(a.src1, b * a.s1_b + h * a.s1_h + d0, a.raw, x);
    store_raw<EPL>(a.tail, ((bh * a.R) + A.t) * a.D + d0, a.raw, x);
  }
}

// Rows per pass of the one-wave-per-block encode: the padded keep count, at
// most eight.
int rows_per_pass(int S) { return S <= 2 ? 2 : (S <= 4 ? 4 : 8); }

template <int EPL>
int launch_encode_epl(const EncodeArgs &e, int64_t BH, hipStream_t stream) {
  const int64_t units = e.n_new + (e.n_copy > 0 ? 1 : 0);
  if (units == 0) return 0;
  const int64_t per_bh = (units + kEncodeWaves - 1) / kEncodeWaves;
  if (per_bh * BH > 0x7FFFFFFF) return -1;
  const dim3 grid((unsigned)(per_bh * BH)), block(64 * kEncodeWaves);
  switch (rows_per_pass(e.S)) {
    case 2: hipLaunchKernelGGL((encode_kernel<EPL, 2>), grid, block, 0, stream, e, per_bh); break;
    case 4: hipLaunchKernelGGL((encode_kernel<EPL, 4>), grid, block, 0, stream, e, per_bh); break;
    default: hipLaunchKernelGGL((encode_kernel<EPL, 8>), grid, block, 0, stream, e, per_bh); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

template <int EPL>
int launch_append_epl(const AppendArgs &A, int64_t BH, hipStream_t stream) {
  const dim3 grid((unsigned)BH, 2), block(64);
  switch (rows_per_pass(A.e[0].S)) {
    case 2: hipLaunchKernelGGL((append_kernel<EPL, 2>), grid, block, 0, stream, A); break;
    case 4: hipLaunchKernelGGL((append_kernel<EPL, 4>), grid, block, 0, stream, A); break;
    default: hipLaunchKernelGGL((append_kernel<EPL, 8>), grid, block, 0, stream, A); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace

template <int LPB, int RP, int JC>
int launch_encode_wide(const EncodeArgs &e, int64_t BH, hipStream_t stream) {
  constexpr int BPW = 64 / LPB;
  const int64_t block_waves = (BH * e.n_new + BPW - 1) / BPW;
  const int64_t waves = block_waves + (e.n_copy > 0 ? BH : 0);
  if (waves == 0) return 0;
  if ((waves + kEncodeWaves - 1) / kEncodeWaves > 0x7FFFFFFF) return -1;
  const dim3 grid((unsigned)((waves + kEncodeWaves - 1) / kEncodeWaves)), block(64 * kEncodeWaves);
  if (e.raw == BF16)
    hipLaunchKernelGGL((encode_wide_kernel<LPB, RP, JC, BF16>), grid, block, 0, stream, e, BH, block_waves);
  else
    hipLaunchKernelGGL((encode_wide_kernel<LPB, RP, JC, F32>), grid, block, 0, stream, e, BH, block_waves);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// Rows per pass: S itself up to 4 (no unused sums), else passes of 4.
template <int LPB, int RP>
int launch_encode_wide_j(const EncodeArgs &e, int64_t BH, hipStream_t stream) {
  switch (e.S) {
    case 1:
    case 2: return launch_encode_wide<LPB, RP, 2>(e, BH, stream);
    case 3: return launch_encode_wide<LPB, RP, 3>(e, BH, stream);
    default: return launch_encode_wide<LPB, RP, 4>(e, BH, stream);
  }
}

template <int LPB>
int launch_encode_wide_r(const EncodeArgs &e, int64_t BH, hipStream_t stream) {
  return e.R <= 8 ? launch_encode_wide_j<LPB, 8>(e, BH, stream) : launch_encode_wide_j<LPB, 16>(e, BH, stream);
}

// Returns 0 on success, 1 on a HIP launch error, -1 if no kernel exists.
// Blocks of up to 16 tokens from one source with 16-byte aligned rows take
// the wide-lane kernel; the rest one wave per block.  The kernels work at
// the compute width of the head_dim (64, 128 or 256).
int launch_encode(const EncodeArgs &e, int64_t BH, hipStream_t stream) {
  const int DP = pad_dim(e.D);
  const bool wide = e.split_i == e.R && e.R <= 16 && (e.raw == BF16 || e.raw == F32) &&
                    ((uintptr_t)e.src0 | (uintptr_t)e.rows) % 16 == 0 && e.s0_b % 8 == 0 && e.s0_h % 8 == 0 &&
                    e.s0_t % 8 == 0;
  if (wide) {
    switch (DP) {
      case 64: return launch_encode_wide_r<8>(e, BH, stream);
      case 128: return launch_encode_wide_r<16>(e, BH, stream);
      default: return launch_encode_wide_r<32>(e, BH, stream);
    }
  }
  switch (DP) {
    case 64: return launch_encode_epl<1>(e, BH, stream);
    case 128: return launch_encode_epl<2>(e, BH, stream);
    default: return launch_encode_epl<4>(e, BH, stream);
  }
}

int launch_append(const AppendArgs &A, int64_t BH, hipStream_t stream) {
  switch (pad_dim(A.e[0].D)) {
    case 64: return launch_append_epl<1>(A, BH, stream);
    case 128: return launch_append_epl<2>(A, BH, stream);
    default: return launch_append_epl<4>(A, BH, stream);
  }
}

}  // namespace cdattn
