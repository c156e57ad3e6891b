// Decode attention directly over the compressed archive (no K/V view).
//
// Method: flashcodec-kv 1.0.0 README, "Materialization-free decode
// attention": with a block stored as rows C (S x D) and synthesis A
// (R x S), q . K[p] = (q . C^T) A[p] and sum_p prob_p V[p] = (prob A) C.
// triton_attention.py: per block s = rows . q, logits = A s * scale, online
// softmax, w = p A, acc += w . rows; split over chunks of blocks, each split
// writes (max, sum, acc) and a combine merges them (flash-decoding).
//
// MI355X design (one workgroup = one (b, kv head, query group, split)):
//  * all GS query heads of a group run in one workgroup, so every
//    coefficient byte is read from HBM once and dequantised once;
//  * 8 waves per workgroup; each wave walks tiles of TR coefficient rows
//    (8 KB of int8 at any head_dim) with 16-byte loads per lane;
//  * K phase: lane = 16 consecutive head_dim elements of one row; int8 codes
//    become exact fp16 (byte permute + one packed fp16 subtract) and are
//    dotted with the query in fp16 pairs accumulating in fp32
//    (v_dot2c_f32_f16); the row sum is a DPP butterfly inside 16-lane rows.
//    The query is pre-scaled by a power of two into fp16 range (exact for
//    every bf16 value within 2^28 of the largest |q|);
//  * logit phase: lane = (block, head); A comes from kernel arguments
//    (scalar loads), logits and weights stay in registers, softmax in base 2
//    with log2(e) folded into the scale, one rescale of acc per tile;
//  * V phase: lane = EV consecutive head_dim elements of one row, fp32 FMAs
//    into per-lane accumulators; rows are reduced across lanes once per wave;
//  * waves merge in LDS, the workgroup writes one partial, and the last
//    workgroup to arrive on the (b, kv head, group) counter combines all
//    splits and writes the output (no second launch).
#pragma once

#include <math.h>

#include "internal.h"

namespace cdattn {
namespace dec {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float xshfl(float v, int mask) { return __shfl_xor(v, mask, 64); }

// Sum over aligned groups of L consecutive lanes; every lane gets its group's sum.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (L >= 2) v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
  if constexpr (L >= 4) v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
  if constexpr (L >= 8) v += dpp<0x141>(v);   // row_half_mirror
  if constexpr (L >= 16) v += dpp<0x140>(v);  // row_mirror
  if constexpr (L >= 32) v += xshfl(v, 16);
  if constexpr (L >= 64) v += xshfl(v, 32);
  return v;
}

template <int L>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (L >= 2) v = fmaxf(v, dpp<0xB1>(v));
  if constexpr (L >= 4) v = fmaxf(v, dpp<0x4E>(v));
  if constexpr (L >= 8) v = fmaxf(v, dpp<0x141>(v));
  if constexpr (L >= 16) v = fmaxf(v, dpp<0x140>(v));
  if constexpr (L >= 32) v = fmaxf(v, xshfl(v, 16));
  if constexpr (L >= 64) v = fmaxf(v, xshfl(v, 32));
  return v;
}

// Reduce over the lanes congruent modulo L (every lane gets its class result).
template <int L, bool MAX>
__device__ __forceinline__ float strided(float v) {
  auto op = [](float x, float y) { return MAX ? fmaxf(x, y) : x + y; };
  if constexpr (L <= 1) v = op(v, dpp<0x121>(v));   // row_ror:1
  if constexpr (L <= 2) v = op(v, dpp<0x122>(v));   // row_ror:2
  if constexpr (L <= 4) v = op(v, dpp<0x124>(v));   // row_ror:4
  if constexpr (L <= 8) v = op(v, dpp<0x128>(v));   // row_ror:8
  if constexpr (L <= 16) v = op(v, xshfl(v, 16));
  if constexpr (L <= 32) v = op(v, xshfl(v, 32));
  return v;
}

__device__ __forceinline__ float readlane(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Four int8 codes -> two exact fp16 pairs: (c ^ 0x80) is c + 128 as a byte;
// fp16 0x64XX = 1024 + byte, and subtracting 1152 leaves c exactly.
__device__ __forceinline__ void i8x4_to_h2(uint32_t w, h2 &lo, h2 &hi) {
  const uint32_t x = w ^ 0x80808080u;
  const uint32_t p0 = __builtin_amdgcn_perm(0x64646464u, x, 0x04010400u);
  const uint32_t p1 = __builtin_amdgcn_perm(0x64646464u, x, 0x04030402u);
  const h2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  lo = __builtin_bit_cast(h2, p0) - bias;
  hi = __builtin_bit_cast(h2, p1) - bias;
}

__device__ __forceinline__ float i8b(uint32_t w, int k) { return (float)(int8_t)(w >> (8 * k)); }

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Make the compiler treat the query registers as redefined here, so that
// conversions of them are not hoisted out of the tile loop (they would each
// hold a register for the whole loop).
template <int GS>
__device__ __forceinline__ void opaque(h2 (&qh)[GS][8]) {
#pragma unroll
  for (int g = 0; g < GS; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t u = __builtin_bit_cast(uint32_t, qh[g][e]);
      asm volatile("" : "+v"(u));
      qh[g][e] = __builtin_bit_cast(h2, u);
    }
}

template <int D, int GS>
struct Cfg {
  static constexpr int W = kDecodeWaves;
  static constexpr int LK = D / 16;                 // lanes per K row
  static constexpr int RK = 64 / LK;                // K rows per step
  static constexpr int EV = (64 / GS) < 16 ? (64 / GS) : 16;   // V elements per lane
  static constexpr int LV = D / EV;                 // lanes per V row
  static constexpr int RV = 64 / LV;                // V rows per step
  static constexpr int TR = 8192 / D;               // rows per tile
  static constexpr int KSTEPS = TR / RK;
  static constexpr int VSTEPS = TR / RV;
};

// Buffer resource over `bytes` bytes at p: loads at or past the end return 0,
// so tile edges need no branches (raw buffer, gfx9-family descriptor word).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload128(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ uint2 bload64(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}
__device__ __forceinline__ float bloadf(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

// ----------------------------------------------------------------- K phase --
// s[row][g] = cq[g] * kscale[row] * sum_d k[row][d] * qh[g][d], rows < nrows.
// Lane = 16 consecutive head_dim elements (chunk c) of row rr of each step.
template <int D, int GS, int F>
__device__ __forceinline__ void kphase(const void *base, const float *kscale, int nrows, int lane,
                                       const h2 (&qh)[GS][8], const float (&cq)[GS], float *sw) {
  using C = Cfg<D, GS>;
  constexpr int EB = F == I8 ? 1 : (F == BF16 ? 2 : 4);  // bytes per element = uint4 per lane
  constexpr int U = (F == I8 ? 8 : (F == BF16 ? 4 : 2)) / (GS >= 8 ? 2 : 1);   // steps per load group
  constexpr uint32_t STEP = C::RK * D * EB;              // bytes per step
  const int rr = lane / C::LK, c = lane % C::LK;
  const rsrc_t rk = make_rsrc(base, (uint32_t)nrows * D * EB);
  const rsrc_t rs = make_rsrc(kscale, kscale ? (uint32_t)nrows * 4 : 0u);
  const uint32_t voff = (uint32_t)(rr * D + c * 16) * EB;
  for (int s0 = 0; s0 < C::KSTEPS; s0 += U) {
    if (s0 * C::RK >= nrows) break;
    uint4 buf[U][EB];
    float ks[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int k = 0; k < EB; ++k) buf[u][k] = bload128(rk, voff + 16 * k, (s0 + u) * STEP);
      if constexpr (F == I8) ks[u] = bloadf(rs, (uint32_t)rr * 4, (s0 + u) * C::RK * 4);
      else ks[u] = 1.0f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if ((s0 + u) * C::RK >= nrows) break;
      const int row = (s0 + u) * C::RK + rr;
      float dot[GS];
#pragma unroll
      for (int g = 0; g < GS; ++g) dot[g] = 0.0f;
      if constexpr (F == I8) {
        const uint32_t wv[4] = {buf[u][0].x, buf[u][0].y, buf[u][0].z, buf[u][0].w};
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          h2 lo, hi;
          i8x4_to_h2(wv[q4], lo, hi);
#pragma unroll
          for (int g = 0; g < GS; ++g) {
            dot[g] = __builtin_amdgcn_fdot2(lo, qh[g][2 * q4], dot[g], false);
            dot[g] = __builtin_amdgcn_fdot2(hi, qh[g][2 * q4 + 1], dot[g], false);
          }
        }
      } else {
        // keep the fp16 -> fp32 query conversions inside the FMA (v_fma_mix)
        opaque(const_cast<h2 (&)[GS][8]>(qh));
        float kf[16];
        if constexpr (F == BF16) {
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const uint32_t wv[4] = {buf[u][k].x, buf[u][k].y, buf[u][k].z, buf[u][k].w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              kf[8 * k + 2 * t] = bf16lo(wv[t]);
              kf[8 * k + 2 * t + 1] = bf16hi(wv[t]);
            }
          }
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            kf[4 * k + 0] = __uint_as_float(buf[u][k].x);
            kf[4 * k + 1] = __uint_as_float(buf[u][k].y);
            kf[4 * k + 2] = __uint_as_float(buf[u][k].z);
            kf[4 * k + 3] = __uint_as_float(buf[u][k].w);
          }
        }
#pragma unroll
        for (int g = 0; g < GS; ++g)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            dot[g] = fmaf((float)qh[g][e].x, kf[2 * e], dot[g]);
            dot[g] = fmaf((float)qh[g][e].y, kf[2 * e + 1], dot[g]);
          }
      }
#pragma unroll
      for (int g = 0; g < GS; ++g) dot[g] = group_sum<C::LK>(dot[g]);
      if (c == 0 && row < nrows) {
#pragma unroll
        for (int g = 0; g < GS; ++g) sw[row * GS + g] = dot[g] * ks[u] * cq[g];
      }
    }
  }
}

// ----------------------------------------------------------------- V phase --
// acc[g][e] += sum over rows of w[row][g] * v[row][c*EV + e].  Rows at or past
// nrows load as zeros and their (finite, stale) weights contribute nothing.
template <int D, int GS, int F>
__device__ __forceinline__ void vphase(const void *base, int nrows, int lane, const float *sw,
                                       float (&acc)[GS][Cfg<D, GS>::EV]) {
  using C = Cfg<D, GS>;
  constexpr int EV = C::EV;
  constexpr int EB = F == I8 ? 1 : (F == BF16 ? 2 : 4);
  constexpr int DW = EV * EB / 4;                  // dwords per lane per step
  constexpr int U = (16 / DW) < 1 ? 1 : ((16 / DW) < C::VSTEPS ? (16 / DW) : C::VSTEPS);
  constexpr uint32_t STEP = C::RV * D * EB;
  const int rr = lane / C::LV, c = lane % C::LV;
  const rsrc_t rv = make_rsrc(base, (uint32_t)nrows * D * EB);
  const uint32_t voff = (uint32_t)(rr * D + c * EV) * EB;
  for (int s0 = 0; s0 < C::VSTEPS; s0 += U) {
    if (s0 * C::RV >= nrows) break;
    uint32_t buf[U][DW];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (DW % 4 == 0) {
#pragma unroll
        for (int k = 0; k < DW / 4; ++k) {
          const uint4 t = bload128(rv, voff + 16 * k, (s0 + u) * STEP);
          buf[u][4 * k] = t.x; buf[u][4 * k + 1] = t.y; buf[u][4 * k + 2] = t.z; buf[u][4 * k + 3] = t.w;
        }
      } else {
        const uint2 t = bload64(rv, voff, (s0 + u) * STEP);
        buf[u][0] = t.x; buf[u][1] = t.y;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if ((s0 + u) * C::RV >= nrows) break;
      const int row = (s0 + u) * C::RV + rr;
      float w[GS];
#pragma unroll
      for (int g = 0; g < GS; ++g) w[g] = sw[row * GS + g];
      float v[EV];
      if constexpr (F == I8) {
#pragma unroll
        for (int k = 0; k < DW; ++k)
#pragma unroll
          for (int t = 0; t < 4; ++t) v[4 * k + t] = i8b(buf[u][k], t);
      } else if constexpr (F == BF16) {
#pragma unroll
        for (int k = 0; k < DW; ++k) { v[2 * k] = bf16lo(buf[u][k]); v[2 * k + 1] = bf16hi(buf[u][k]); }
      } else {
#pragma unroll
        for (int k = 0; k < DW; ++k) v[k] = __uint_as_float(buf[u][k]);
      }
#pragma unroll
      for (int g = 0; g < GS; ++g)
#pragma unroll
        for (int e = 0; e < EV; ++e) acc[g][e] = fmaf(w[g], v[e], acc[g][e]);
    }
  }
}

// ------------------------------------------------------------ logit phase --
// Items (block n, head g) with g = lane % GS.  TAIL: every "block" is one raw
// token (R = S = 1, A = [1]).  Updates the running max, rescale factors and
// the lane's partial sum; overwrites sw with the value weights w * vscale.
template <int GS, int SP, bool TAIL>
__device__ __forceinline__ void logits(const DecodeArgs &a, const float *sA, float *sw, int nb, const float *__restrict__ vscale,
                                       int lane, float (&m_u)[GS], float &m_own, float &l_own,
                                       float (&alpha)[GS]) {
  const int S = TAIL ? 1 : a.S;
  const int R = TAIL ? 1 : a.R;
  const int g = lane % GS;
  const int items = nb * GS;
  float mx = -INFINITY;
  for (int i = lane; i < items; i += 64) {
    const int n = i / GS;
    float sv[SP];
#pragma unroll
    for (int j = 0; j < SP; ++j) sv[j] = (j < S) ? sw[(n * S + j) * GS + g] : 0.0f;
    if constexpr (TAIL) {
      mx = fmaxf(mx, sv[0]);
    } else {
      for (int r = 0; r < R; ++r) {
        const float *Ar = sA + r * SP;
        float z = 0.0f;
#pragma unroll
        for (int j = 0; j < SP; ++j) z = fmaf(Ar[j], sv[j], z);
        mx = fmaxf(mx, z);
      }
    }
  }
  mx = strided<GS, true>(mx);
  const float mnew_own = fmaxf(m_own, mx);
  const float alpha_own = __builtin_amdgcn_exp2f(m_own - mnew_own);
#pragma unroll
  for (int gg = 0; gg < GS; ++gg) {
    const float mn = fmaxf(m_u[gg], readlane(mx, gg));
    alpha[gg] = __builtin_amdgcn_exp2f(m_u[gg] - mn);
    m_u[gg] = mn;
  }
  m_own = mnew_own;
  float lsum = 0.0f;
  for (int i = lane; i < items; i += 64) {
    const int n = i / GS;
    float sv[SP];
#pragma unroll
    for (int j = 0; j < SP; ++j) sv[j] = (j < S) ? sw[(n * S + j) * GS + g] : 0.0f;
    float w[SP];
    if constexpr (TAIL) {
      const float p = __builtin_amdgcn_exp2f(sv[0] - m_own);
      lsum += p;
      w[0] = p;
    } else {
#pragma unroll
      for (int j = 0; j < SP; ++j) w[j] = 0.0f;
      for (int r = 0; r < R; ++r) {
        const float *Ar = sA + r * SP;
        float z = 0.0f;
#pragma unroll
        for (int j = 0; j < SP; ++j) z = fmaf(Ar[j], sv[j], z);
        const float p = __builtin_amdgcn_exp2f(z - m_own);
        lsum += p;
#pragma unroll
        for (int j = 0; j < SP; ++j) w[j] = fmaf(p, Ar[j], w[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < SP; ++j)
      if (j < S) sw[(n * S + j) * GS + g] = w[j] * (vscale ? vscale[n * S + j] : 1.0f);
  }
  l_own = l_own * alpha_own + lsum;
}

template <int D, int GS, int SP>
__global__ __launch_bounds__(64 * kDecodeWaves) void decode_kernel(DecodeArgs a) {
  using C = Cfg<D, GS>;
  constexpr int W = C::W, EV = C::EV;
  // per-wave s / w scratch during tiles, then the workgroup merge area
  constexpr int SW_FLOATS = C::TR * GS;
  constexpr int MERGE_FLOATS = W * GS * D + W * GS * 2;
  constexpr int COMB_FLOATS = 2 * 256 * GS + GS;   // ns <= 256
  constexpr int LDS_A = (W * SW_FLOATS > MERGE_FLOATS) ? W * SW_FLOATS : MERGE_FLOATS;
  constexpr int LDS_FLOATS = LDS_A > COMB_FLOATS ? LDS_A : COMB_FLOATS;
  __shared__ float lds[LDS_FLOATS];
  __shared__ float sA[kMaxR * SP];   // synthesis basis, copied once from the arguments
  __shared__ int last_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int split = blockIdx.x % a.ns;
  const int64_t pairq = blockIdx.x / a.ns;
  const int qg = (int)(pairq % a.NQG);
  const int64_t bh = pairq / a.NQG;
  const int64_t b = bh / a.H;
  const int h = (int)(bh % a.H);
  const int hq0 = h * a.G + qg * GS;
  // kernel arguments may live in host-coherent memory: read A once, here
  for (int i = tid; i < a.R * SP; i += 64 * W) sA[i] = a.A[i];
  __syncthreads();

  // ---- query: fp16 pairs of the lane's 16 K elements, pre-scaled per head
  h2 qh[GS][8];
  float cq[GS];
  {
    const int d0 = (lane % C::LK) * 16;
#pragma unroll
    for (int g = 0; g < GS; ++g) {
      const uint4 *qp = reinterpret_cast<const uint4 *>(a.q + b * a.q_sb + (int64_t)(hq0 + g) * a.q_sh + d0);
      const uint4 q0 = qp[0], q1 = qp[1];
      const uint32_t wv[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
      float qf[16];
      float amax = 0.0f;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        qf[2 * t] = bf16lo(wv[t]);
        qf[2 * t + 1] = bf16hi(wv[t]);
        amax = fmaxf(amax, fmaxf(fabsf(qf[2 * t]), fabsf(qf[2 * t + 1])));
      }
      amax = group_max<C::LK>(amax);
      int E = 0;
      if (amax > 0.0f) frexpf(amax, &E);
      const float up = ldexpf(1.0f, 15 - E);
#pragma unroll
      for (int t = 0; t < 8; ++t) qh[g][t] = h2{(_Float16)(qf[2 * t] * up), (_Float16)(qf[2 * t + 1] * up)};
      cq[g] = a.qk_scale * ldexpf(1.0f, E - 15);
    }
  }

  float m_u[GS], alpha[GS];
  float acc[GS][EV];
#pragma unroll
  for (int g = 0; g < GS; ++g) {
    m_u[g] = -INFINITY;
#pragma unroll
    for (int e = 0; e < EV; ++e) acc[g][e] = 0.0f;
  }
  float m_own = -INFINITY, l_own = 0.0f;
  float *sw = lds + wave * SW_FLOATS;
  // weights of rows past a tile's end are read but multiply zero data: keep
  // them finite from the start
  for (int i = lane; i < SW_FLOATS; i += 64) sw[i] = 0.0f;
  wave_lds_sync();

  const int S = a.S;
  const int NB = C::TR / S;
  const int64_t blk0 = (int64_t)split * a.chunk;
  const int64_t blk1 = (blk0 + a.chunk < a.n_blocks) ? blk0 + a.chunk : a.n_blocks;
  const int64_t nblk = blk1 > blk0 ? blk1 - blk0 : 0;
  const int ntiles = (int)((nblk + NB - 1) / NB);
  const int64_t k_bh = bh * a.k_bh_rows, v_bh = bh * a.v_bh_rows;
  const int kes = a.kf == I8 ? 1 : (a.kf == BF16 ? 2 : 4);
  const int ves = a.vf == I8 ? 1 : (a.vf == BF16 ? 2 : 4);

  for (int t = wave; t < ntiles; t += W) {
    opaque(qh);
    const int64_t tb0 = blk0 + (int64_t)t * NB;
    const int nb = (int)((blk1 - tb0) < NB ? (blk1 - tb0) : NB);
    const int nrows = nb * S;
    const int64_t row0 = tb0 * S;
    const char *kb = static_cast<const char *>(a.krows) + (k_bh + row0) * D * kes;
    const char *vb = static_cast<const char *>(a.vrows) + (v_bh + row0) * D * ves;
    const float *ksc = a.kf == I8 ? a.kscales + k_bh + row0 : nullptr;
    const float *vsc = a.vf == I8 ? a.vscales + v_bh + row0 : nullptr;
    if (a.kf == I8) kphase<D, GS, I8>(kb, ksc, nrows, lane, qh, cq, sw);
    else if (a.kf == BF16) kphase<D, GS, BF16>(kb, nullptr, nrows, lane, qh, cq, sw);
    else kphase<D, GS, F32>(kb, nullptr, nrows, lane, qh, cq, sw);
    wave_lds_sync();
    logits<GS, SP, false>(a, sA, sw, nb, vsc, lane, m_u, m_own, l_own, alpha);
#pragma unroll
    for (int g = 0; g < GS; ++g)
#pragma unroll
      for (int e = 0; e < EV; ++e) acc[g][e] *= alpha[g];
    wave_lds_sync();
    if (a.vf == I8) vphase<D, GS, I8>(vb, nrows, lane, sw, acc);
    else if (a.vf == BF16) vphase<D, GS, BF16>(vb, nrows, lane, sw, acc);
    else vphase<D, GS, F32>(vb, nrows, lane, sw, acc);
    wave_lds_sync();
  }

  // the raw tail: one wave of the last split, token by token
  if (a.n_tail > 0 && split == a.ns - 1 && wave == ntiles % W) {
    opaque(qh);
    const int nt = a.n_tail;
    const char *kt = static_cast<const char *>(a.ktail) + bh * (int64_t)a.R * D * (a.kraw == BF16 ? 2 : 4);
    const char *vt = static_cast<const char *>(a.vtail) + bh * (int64_t)a.R * D * (a.vraw == BF16 ? 2 : 4);
    if (a.kraw == BF16) kphase<D, GS, BF16>(kt, nullptr, nt, lane, qh, cq, sw);
    else kphase<D, GS, F32>(kt, nullptr, nt, lane, qh, cq, sw);
    wave_lds_sync();
    logits<GS, SP, true>(a, sA, sw, nt, nullptr, lane, m_u, m_own, l_own, alpha);
#pragma unroll
    for (int g = 0; g < GS; ++g)
#pragma unroll
      for (int e = 0; e < EV; ++e) acc[g][e] *= alpha[g];
    wave_lds_sync();
    if (a.vraw == BF16) vphase<D, GS, BF16>(vt, nt, lane, sw, acc);
    else vphase<D, GS, F32>(vt, nt, lane, sw, acc);
    wave_lds_sync();
  }

  // ---- wave totals: l over lanes of a head, acc over the rows of a step
  float l_u[GS];
  {
    const float lt = strided<GS, false>(l_own);
#pragma unroll
    for (int g = 0; g < GS; ++g) l_u[g] = readlane(lt, g);
  }
#pragma unroll
  for (int g = 0; g < GS; ++g)
#pragma unroll
    for (int e = 0; e < EV; ++e) acc[g][e] = strided<C::LV, false>(acc[g][e]);

  __syncthreads();   // all waves done with their sw scratch
  float *macc = lds;                    // [W][GS][D]
  float *mml = lds + W * GS * D;        // [W][GS][2]
  if (lane < C::LV) {
#pragma unroll
    for (int g = 0; g < GS; ++g)
#pragma unroll
      for (int e = 0; e < EV; ++e) macc[(wave * GS + g) * D + lane * EV + e] = acc[g][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < GS; ++g) {
      mml[(wave * GS + g) * 2] = m_u[g];
      mml[(wave * GS + g) * 2 + 1] = l_u[g];
    }
  }
  __syncthreads();

  // ---- workgroup partial
  float *pacc = a.part_acc + (pairq * a.ns + split) * GS * D;
  float *pml = a.part_ml + (pairq * a.ns + split) * GS * 2;
  for (int idx = tid; idx < GS * D; idx += 64 * W) {
    const int g = idx / D, d = idx % D;
    float m = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) m = fmaxf(m, mml[(w * GS + g) * 2]);
    float l = 0.0f, s = 0.0f;
    if (m != -INFINITY) {
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float lw = mml[(w * GS + g) * 2 + 1];
        if (lw > 0.0f) {
          const float f = __builtin_amdgcn_exp2f(mml[(w * GS + g) * 2] - m);
          l += lw * f;
          s += macc[(w * GS + g) * D + d] * f;
        }
      }
    }
    pacc[g * D + d] = s;
    if (d == 0) {
      pml[g * 2] = m;
      pml[g * 2 + 1] = l;
    }
  }

  // ---- split arrival; the last workgroup of (b, h, group) combines.
  // Writers only release (L2 write-back); the one combining workgroup
  // acquires (L2 invalidate).  A full fence in every workgroup would
  // invalidate the XCD's L2 once per workgroup.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(a.counters + pairq, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_flag = (old == (uint32_t)(a.ns - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!last_flag) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

  // (max, sum) of every split into LDS, one load per thread; then the
  // per-split weights; then every (head, d) output sums its split partials
  // with independent loads.  Partials of other workgroups are visible after
  // the acquire fence above.
  const float *Pacc = a.part_acc + pairq * a.ns * GS * D;
  const float *Pml = a.part_ml + pairq * a.ns * GS * 2;
  float *cml = lds;                     // [ns*GS][2]; later f = weight per split
  float *cM = lds + 2 * a.ns * GS;      // [GS] max, [GS] 1/sum
  for (int i = tid; i < a.ns * GS; i += 64 * W) {
    cml[2 * i] = Pml[2 * i];
    cml[2 * i + 1] = Pml[2 * i + 1];
  }
  __syncthreads();
  if (tid < GS) {
    float m = -INFINITY;
    for (int sp = 0; sp < a.ns; ++sp) m = fmaxf(m, cml[2 * (sp * GS + tid)]);
    float l = 0.0f;
    for (int sp = 0; sp < a.ns; ++sp) {
      const float li = cml[2 * (sp * GS + tid) + 1];
      const float f = li > 0.0f ? __builtin_amdgcn_exp2f(cml[2 * (sp * GS + tid)] - m) : 0.0f;
      l += li * f;
      cml[2 * (sp * GS + tid)] = f;
    }
    cM[tid] = 1.0f / l;
  }
  __syncthreads();
  for (int idx = tid; idx < GS * D; idx += 64 * W) {
    const int g = idx / D, d = idx % D;
    float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
    int sp = 0;
    for (; sp + 4 <= a.ns; sp += 4) {
      s0 = fmaf(cml[2 * ((sp + 0) * GS + g)], Pacc[((sp + 0) * GS + g) * D + d], s0);
      s1 = fmaf(cml[2 * ((sp + 1) * GS + g)], Pacc[((sp + 1) * GS + g) * D + d], s1);
      s2 = fmaf(cml[2 * ((sp + 2) * GS + g)], Pacc[((sp + 2) * GS + g) * D + d], s2);
      s3 = fmaf(cml[2 * ((sp + 3) * GS + g)], Pacc[((sp + 3) * GS + g) * D + d], s3);
    }
    for (; sp < a.ns; ++sp) s0 = fmaf(cml[2 * (sp * GS + g)], Pacc[(sp * GS + g) * D + d], s0);
    const float o = ((s0 + s1) + (s2 + s3)) * cM[g];
    const int64_t off = b * a.o_sb + (int64_t)(hq0 + g) * a.o_sh + d;
    if (a.out_f32) {
      static_cast<float *>(a.out)[off] = o;
    } else {
      uint32_t u = __float_as_uint(o);
      u += 0x7FFFu + ((u >> 16) & 1u);
      static_cast<uint16_t *>(a.out)[off] = (uint16_t)(u >> 16);
    }
  }
  if (tid == 0) a.counters[pairq] = 0u;
}

template <int D, int GS, int SP>
int launch_one(const DecodeArgs &a, int64_t n_wg, hipStream_t stream) {
  hipLaunchKernelGGL((decode_kernel<D, GS, SP>), dim3((unsigned)n_wg), dim3(64 * kDecodeWaves), 0, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

template <int D, int GS>
int launch_sp(int SP, const DecodeArgs &a, int64_t n_wg, hipStream_t stream) {
  switch (SP) {
    case 2: return launch_one<D, GS, 2>(a, n_wg, stream);
    case 4: return launch_one<D, GS, 4>(a, n_wg, stream);
    case 8: return launch_one<D, GS, 8>(a, n_wg, stream);
    case 16: return launch_one<D, GS, 16>(a, n_wg, stream);
    default: return -1;
  }
}

template <int D>
int launch_d(int GS, int SP, const DecodeArgs &a, int64_t n_wg, hipStream_t stream) {
  switch (GS) {
    case 1: return launch_sp<D, 1>(SP, a, n_wg, stream);
    case 2: return launch_sp<D, 2>(SP, a, n_wg, stream);
    case 4: return launch_sp<D, 4>(SP, a, n_wg, stream);
    case 8: return launch_sp<D, 8>(SP, a, n_wg, stream);
    default: return -1;
  }
}

}  // namespace dec
}  // namespace cdattn
