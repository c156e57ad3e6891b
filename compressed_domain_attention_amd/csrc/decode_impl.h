// Decode attention directly over the compressed archive (no K/V view).
//
// Method: flashcodec-kv 1.0.0 README, "Materialization-free decode
// attention": with a block stored as rows C (S x D) and synthesis A
// (R x S), q . K[p] = (q . C^T) A[p] and sum_p prob_p V[p] = (prob A) C.
// triton_attention.py: per block s = rows . q, logits = A s * scale, online
// softmax, w = p A, acc += w . rows; split over chunks of blocks, each split
// writes (max, sum, acc) and a combine merges them (flash-decoding).
//
// MI355X design.  One workgroup = one (b, kv head, query group, split) with
// all GS query heads of the group, so each coefficient byte is read from HBM
// once and converted once.  8 waves per workgroup, one workgroup per CU.
//  * Tiles of TR coefficient rows (about 8 KB of K+V) stream through
//    registers with 16-byte buffer loads per lane; each wave keeps the next
//    tile's loads in flight while it computes the current one (two register
//    buffers).  Buffer loads past a tile's end return zeros, so edges need
//    no branches.
//  * K phase: lane = 16 consecutive head_dim elements of one row; int8 codes
//    become exact fp16 (byte permute + one packed fp16 subtract) and are
//    dotted with the query in fp16 pairs accumulating in fp32
//    (v_dot2c_f32_f16); the row sum is a DPP butterfly inside 16-lane rows.
//    The query is pre-scaled by a power of two into fp16 range (exact for
//    every bf16 value within 2^28 of the largest |q|).
//  * Logit phase: lane = (block, head, 8 of the R tokens); the R x S basis A
//    sits in LDS; logits stay in registers; base-2 softmax with log2(e)
//    folded into the scale; one rescale of the accumulators per tile.
//  * V phase: lane = EV consecutive head_dim elements of one row; the value
//    weight w * vscale multiplies int8 codes converted by SDWA; fp32 FMAs
//    into per-lane accumulators, reduced across lanes once per wave.
//  * Waves merge in LDS; the workgroup publishes its partial with
//    device-scope stores, waits for them, and bumps a per-(b, h, group)
//    counter; the last workgroup to arrive combines all splits with
//    device-scope loads and writes the output (no second launch, and no L2
//    write-back or invalidate per workgroup).
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

// Sum / max over aligned groups of L consecutive lanes (every lane gets it).
template <int L, bool MAX>
__device__ __forceinline__ float group_red(float v) {
  auto op = [](float x, float y) { return MAX ? fmaxf(x, y) : x + y; };
  if constexpr (L >= 2) v = op(v, dpp<0xB1>(v));    // quad_perm [1,0,3,2]
  if constexpr (L >= 4) v = op(v, dpp<0x4E>(v));    // quad_perm [2,3,0,1]
  if constexpr (L >= 8) v = op(v, dpp<0x141>(v));   // row_half_mirror
  if constexpr (L >= 16) v = op(v, dpp<0x140>(v));  // row_mirror
  if constexpr (L >= 32) v = op(v, xshfl(v, 16));
  if constexpr (L >= 64) v = op(v, xshfl(v, 32));
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

// Reduce over the LR adjacent lanes of an item (LR in {1, 2, 4}), then over
// the items of the same head (lanes congruent modulo GS * LR).
template <int GS, bool MAX>
__device__ __forceinline__ float head_reduce(float v, int LR) {
  if (LR == 1) return strided<GS, MAX>(v);
  if (LR == 2) return strided<(GS * 2 < 64 ? GS * 2 : 64), MAX>(group_red<2, MAX>(v));
  return strided<(GS * 4 < 64 ? GS * 4 : 64), MAX>(group_red<4, MAX>(v));
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

// Keep the compiler from hoisting conversions of the query registers out of
// a loop (each would hold a register for the whole loop).
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

constexpr int ebytes(int F) { return F == I8 ? 1 : (F == BF16 ? 2 : 4); }
constexpr int cmin(int a, int b) { return a < b ? a : b; }
constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <int D, int GS, int KF, int VF>
struct Cfg {
  static constexpr int W = kDecodeWaves;
  static constexpr int EBK = ebytes(KF), EBV = ebytes(VF);
  static constexpr int TR = decode_tile_rows(D, KF, VF);   // rows per tile (K+V ~ 8 KB)
  static constexpr int LK = D / 16;                     // lanes per K row (16 elements each)
  static constexpr int RK = 64 / LK;                    // K rows per step
  static constexpr int KSTEPS = (TR + RK - 1) / RK;
  static constexpr int KQ = EBK;                        // uint4 per lane per K step
  static constexpr int EV = cmin(16, 64 / GS);          // V elements per lane
  static constexpr int LV = D / EV;                     // lanes per V row
  static constexpr int RV = 64 / LV;                    // V rows per step
  static constexpr int VSTEPS = (TR + RV - 1) / RV;
  static constexpr int VDW = EV * EBV / 4;              // dwords per lane per V step
};

// Registers of one in-flight tile.
template <int D, int GS, int KF, int VF>
struct TileBuf {
  using C = Cfg<D, GS, KF, VF>;
  uint4 k[C::KSTEPS][C::KQ];
  float ks[C::KSTEPS];
  uint32_t v[C::VSTEPS][C::VDW];
  float vs[C::VSTEPS];
};

// Where a tile lives and how many rows it has.
struct TileRef {
  const char *k;
  const char *v;
  const float *ks;
  const float *vs;
  int nrows;
};

template <int D, int GS, int KF, int VF>
__device__ __forceinline__ void issue_k(TileBuf<D, GS, KF, VF> &B, const TileRef &T, int lane) {
  using C = Cfg<D, GS, KF, VF>;
  const rsrc_t rk = make_rsrc(T.k, (uint32_t)T.nrows * D * C::EBK);
  const int rrk = lane / C::LK, ck = lane % C::LK;
  const uint32_t vk = (uint32_t)(rrk * D + ck * 16) * C::EBK;
#pragma unroll
  for (int s = 0; s < C::KSTEPS; ++s)
#pragma unroll
    for (int k = 0; k < C::KQ; ++k) B.k[s][k] = bload128(rk, vk + 16 * k, s * C::RK * D * C::EBK);
  if constexpr (KF == I8) {
    const rsrc_t rs = make_rsrc(T.ks, (uint32_t)T.nrows * 4);
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s) B.ks[s] = bloadf(rs, (uint32_t)rrk * 4, s * C::RK * 4);
  }
}

template <int D, int GS, int KF, int VF>
__device__ __forceinline__ void issue_v(TileBuf<D, GS, KF, VF> &B, const TileRef &T, int lane) {
  using C = Cfg<D, GS, KF, VF>;
  const rsrc_t rv = make_rsrc(T.v, (uint32_t)T.nrows * D * C::EBV);
  const int rrv = lane / C::LV, cv = lane % C::LV;
  const uint32_t vv = (uint32_t)(rrv * D + cv * C::EV) * C::EBV;
#pragma unroll
  for (int s = 0; s < C::VSTEPS; ++s) {
    if constexpr (C::VDW % 4 == 0) {
#pragma unroll
      for (int k = 0; k < C::VDW / 4; ++k) {
        const uint4 t = bload128(rv, vv + 16 * k, s * C::RV * D * C::EBV);
        B.v[s][4 * k] = t.x; B.v[s][4 * k + 1] = t.y; B.v[s][4 * k + 2] = t.z; B.v[s][4 * k + 3] = t.w;
      }
    } else {
      const uint2 t = bload64(rv, vv, s * C::RV * D * C::EBV);
      B.v[s][0] = t.x; B.v[s][1] = t.y;
    }
  }
  if constexpr (VF == I8) {
    const rsrc_t rs = make_rsrc(T.vs, (uint32_t)T.nrows * 4);
#pragma unroll
    for (int s = 0; s < C::VSTEPS; ++s) B.vs[s] = bloadf(rs, (uint32_t)rrv * 4, s * C::RV * 4);
  }
}

template <int D, int GS, int KF, int VF>
__device__ __forceinline__ void issue(TileBuf<D, GS, KF, VF> &B, const TileRef &T, int lane) {
  issue_k(B, T, lane);
  issue_v(B, T, lane);
}

// ----------------------------------------------------------------- K phase --
// s[row][g] = cq[g] * kscale[row] * sum_d k[row][d] * q[g][d].  Format F, 16
// elements per lane held in F's bytes (KQ uint4).
template <int D, int GS, int F, int STEPS, int KQ>
__device__ __forceinline__ void kcompute(const uint4 (&kb)[STEPS][KQ], const float (&ks)[STEPS], int nrows,
                                         int lane, h2 (&qh)[GS][8], const float (&cq)[GS], float *sw,
                                         int row_base = 0) {
  constexpr int LK = D / 16, RK = 64 / LK;
  const int rr = lane / LK, c = lane % LK;
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    if (row_base + s * RK >= nrows) break;
    const int row = row_base + s * RK + rr;
    float dot[GS];
#pragma unroll
    for (int g = 0; g < GS; ++g) dot[g] = 0.0f;
    if constexpr (F == I8) {
      const uint32_t wv[4] = {kb[s][0].x, kb[s][0].y, kb[s][0].z, kb[s][0].w};
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
      opaque(qh);   // keep the fp16 -> fp32 conversion inside v_fma_mix
      float kf[16];
      if constexpr (F == BF16) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const uint32_t wv[4] = {kb[s][k].x, kb[s][k].y, kb[s][k].z, kb[s][k].w};
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            kf[8 * k + 2 * t] = bf16lo(wv[t]);
            kf[8 * k + 2 * t + 1] = bf16hi(wv[t]);
          }
        }
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          kf[4 * k + 0] = __uint_as_float(kb[s][k].x);
          kf[4 * k + 1] = __uint_as_float(kb[s][k].y);
          kf[4 * k + 2] = __uint_as_float(kb[s][k].z);
          kf[4 * k + 3] = __uint_as_float(kb[s][k].w);
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
    for (int g = 0; g < GS; ++g) dot[g] = group_red<LK, false>(dot[g]);
    if (c == 0 && row < nrows) {
#pragma unroll
      for (int g = 0; g < GS; ++g) sw[row * GS + g] = dot[g] * (F == I8 ? ks[s] * cq[g] : cq[g]);
    }
  }
}

// ----------------------------------------------------------------- V phase --
// acc[g][e] += sum over rows of w[row][g] * vscale[row] * v[row][c*EV + e].
// Rows past nrows hold zero data (buffer range) and finite stale weights.
template <int D, int GS, int F, int STEPS, int VDW, int EV>
__device__ __forceinline__ void vcompute(const uint32_t (&vb)[STEPS][VDW], const float (&vs)[STEPS], int nrows,
                                         int lane, const float *sw, float (&acc)[GS][EV], int row_base = 0) {
  constexpr int LV = D / EV, RV = 64 / LV;
  const int rr = lane / LV;
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    if (row_base + s * RV >= nrows) break;
    const int row = row_base + s * RV + rr;
    float w[GS];
#pragma unroll
    for (int g = 0; g < GS; ++g) w[g] = sw[row * GS + g];
    if constexpr (F == I8) {
#pragma unroll
      for (int g = 0; g < GS; ++g) w[g] *= vs[s];
    }
    float v[EV];
    if constexpr (F == I8) {
#pragma unroll
      for (int k = 0; k < VDW; ++k)
#pragma unroll
        for (int t = 0; t < 4; ++t) v[4 * k + t] = i8b(vb[s][k], t);
    } else if constexpr (F == BF16) {
#pragma unroll
      for (int k = 0; k < VDW; ++k) { v[2 * k] = bf16lo(vb[s][k]); v[2 * k + 1] = bf16hi(vb[s][k]); }
    } else {
#pragma unroll
      for (int k = 0; k < VDW; ++k) v[k] = __uint_as_float(vb[s][k]);
    }
#pragma unroll
    for (int g = 0; g < GS; ++g)
#pragma unroll
      for (int e = 0; e < EV; ++e) acc[g][e] = fmaf(w[g], v[e], acc[g][e]);
  }
}

// ------------------------------------------------------------ logit phase --
// Items (block n, head g) laid out as lane = (n * GS + g) * LR + lr, where
// lr picks tokens lr*8 .. lr*8+7 of the block (LR = ceil(R / 8)).  Updates
// the running max (uniform m_u, per-lane m_own), the rescale factors and the
// lane's partial sum; overwrites sw with the value weights w = p A.
// TAIL: every "block" is one raw token (R = S = 1, A = [1]); the lane layout
// keeps the LR of the archive so every lane tracks the same head throughout,
// and only the first lane of an item contributes.
template <int SP>
__device__ __forceinline__ void load_row(const float *sA, int r, float (&a)[SP]) {
  if constexpr (SP % 4 == 0) {
#pragma unroll
    for (int j = 0; j < SP; j += 4) {
      const float4 t = *reinterpret_cast<const float4 *>(sA + r * SP + j);
      a[j] = t.x; a[j + 1] = t.y; a[j + 2] = t.z; a[j + 3] = t.w;
    }
  } else {
    const float2 t = *reinterpret_cast<const float2 *>(sA + r * SP);
    a[0] = t.x; a[1] = t.y;
  }
}

template <int GS, int SP, bool TAIL>
__device__ __forceinline__ void logits(const float *sA, float *sw, int nb, int R, int S, int LR, int lane,
                                       float (&m_u)[GS], float &m_own, float &l_own, float (&alpha)[GS]) {
  const int lr = lane % LR;
  const int g = (lane / LR) % GS;
  const int per_pass = 64 / LR;                 // items per pass
  const int items = nb * GS;
  // tokens of this lane in every block: lr*8 .. lr*8 + rc - 1
  const int rc = TAIL ? (lr == 0 ? 1 : 0) : ((R - lr * 8) < 8 ? (R - lr * 8) : 8);
  const bool full = !TAIL && (R % 8 == 0);      // uniform: every lane has 8 tokens
  float mx = -INFINITY;
  float zc[8];                                   // logits of the first pass
#pragma unroll
  for (int r8 = 0; r8 < 8; ++r8) zc[r8] = -INFINITY;
  for (int i0 = 0; i0 < items; i0 += per_pass) {
    const int i = i0 + lane / LR;
    const bool live = i < items;
    const int n = live ? i / GS : 0;
    float sv[SP];
#pragma unroll
    for (int j = 0; j < SP; ++j) sv[j] = (j < S) ? sw[(n * S + j) * GS + g] : 0.0f;
    if constexpr (TAIL) {
      if (live && rc) {
        zc[0] = sv[0];
        mx = fmaxf(mx, sv[0]);
      }
    } else if (full) {
#pragma unroll
      for (int r8 = 0; r8 < 8; ++r8) {
        float a[SP];
        load_row<SP>(sA, lr * 8 + r8, a);
        float z = 0.0f;
#pragma unroll
        for (int j = 0; j < SP; ++j) z = fmaf(a[j], sv[j], z);
        zc[r8] = z;
        mx = fmaxf(mx, live ? z : -INFINITY);
      }
    } else {
#pragma unroll
      for (int r8 = 0; r8 < 8; ++r8) {
        if (r8 < rc) {
          float a[SP];
          load_row<SP>(sA, lr * 8 + r8, a);
          float z = 0.0f;
#pragma unroll
          for (int j = 0; j < SP; ++j) z = fmaf(a[j], sv[j], z);
          zc[r8] = z;
          mx = fmaxf(mx, live ? z : -INFINITY);
        }
      }
    }
  }
  mx = head_reduce<GS, true>(mx, LR);
  const float mnew_own = fmaxf(m_own, mx);
  const float alpha_own = __builtin_amdgcn_exp2f(m_own - mnew_own);
#pragma unroll
  for (int gg = 0; gg < GS; ++gg) {
    const float mn = fmaxf(m_u[gg], readlane(mx, gg * LR));
    alpha[gg] = __builtin_amdgcn_exp2f(m_u[gg] - mn);
    m_u[gg] = mn;
  }
  m_own = mnew_own;
  const bool one_pass = items <= per_pass;
  float lsum = 0.0f;
  for (int i0 = 0; i0 < items; i0 += per_pass) {
    const int i = i0 + lane / LR;
    const bool live = i < items;
    const int n = live ? i / GS : 0;
    float sv[SP];
    if (!one_pass) {
#pragma unroll
      for (int j = 0; j < SP; ++j) sv[j] = (j < S) ? sw[(n * S + j) * GS + g] : 0.0f;
    }
    float w[SP];
#pragma unroll
    for (int j = 0; j < SP; ++j) w[j] = 0.0f;
    if constexpr (TAIL) {
      if (live && rc) {
        const float p = __builtin_amdgcn_exp2f((one_pass ? zc[0] : sv[0]) - m_own);
        lsum += p;
        w[0] = p;
      }
    } else {
#pragma unroll
      for (int r8 = 0; r8 < 8; ++r8) {
        if (full || r8 < rc) {
          float a[SP];
          load_row<SP>(sA, lr * 8 + r8, a);
          float z;
          if (one_pass) {
            z = zc[r8];
          } else {
            z = 0.0f;
#pragma unroll
            for (int j = 0; j < SP; ++j) z = fmaf(a[j], sv[j], z);
          }
          const float p = live ? __builtin_amdgcn_exp2f(z - m_own) : 0.0f;
          lsum += p;
#pragma unroll
          for (int j = 0; j < SP; ++j) w[j] = fmaf(p, a[j], w[j]);
        }
      }
    }
    if (LR == 2) {
#pragma unroll
      for (int j = 0; j < SP; ++j) w[j] = group_red<2, false>(w[j]);
    } else if (LR == 4) {
#pragma unroll
      for (int j = 0; j < SP; ++j) w[j] = group_red<4, false>(w[j]);
    }
    if (live && lr == 0) {
#pragma unroll
      for (int j = 0; j < SP; ++j)
        if (j < S) sw[(n * S + j) * GS + g] = w[j];
    }
  }
  l_own = l_own * alpha_own + lsum;
}

// acc *= alpha, skipped when no head's running max moved (the common case).
template <int GS, int EV>
__device__ __forceinline__ void rescale(float (&acc)[GS][EV], const float (&alpha)[GS]) {
  bool moved = false;
#pragma unroll
  for (int g = 0; g < GS; ++g) moved |= alpha[g] != 1.0f;
  if (moved) {
#pragma unroll
    for (int g = 0; g < GS; ++g)
#pragma unroll
      for (int e = 0; e < EV; ++e) acc[g][e] *= alpha[g];
  }
}

template <int D, int GS, int SP, int KF, int VF>
__device__ __forceinline__ void process_k(const TileBuf<D, GS, KF, VF> &B, int nrows, int lane, h2 (&qh)[GS][8],
                                          const float (&cq)[GS], float *sw) {
  using C = Cfg<D, GS, KF, VF>;
  kcompute<D, GS, KF, C::KSTEPS, C::KQ>(B.k, B.ks, nrows, lane, qh, cq, sw);
  wave_lds_sync();
}

template <int D, int GS, int SP, int KF, int VF>
__device__ __forceinline__ void process_lv(const TileBuf<D, GS, KF, VF> &B, int nrows, int S, int R, int LR,
                                           int lane, const float *sA, float *sw, float (&m_u)[GS], float &m_own,
                                           float &l_own, float (&acc)[GS][Cfg<D, GS, KF, VF>::EV]) {
  using C = Cfg<D, GS, KF, VF>;
  float alpha[GS];
  logits<GS, SP, false>(sA, sw, nrows / S, R, S, LR, lane, m_u, m_own, l_own, alpha);
  rescale(acc, alpha);
  wave_lds_sync();
  vcompute<D, GS, VF, C::VSTEPS, C::VDW, C::EV>(B.v, B.vs, nrows, lane, sw, acc);
  wave_lds_sync();
}

// The raw tail (< R tokens of bf16 / fp32) in one wave, one load step at a
// time so it needs few registers.  Every token is a block with R = S = 1.
template <int D, int GS, int SP, int RAWK, int RAWV, int EV>
__device__ __forceinline__ void tail_pass(const void *kt, const void *vt, int nt, int LR, int lane, h2 (&qh)[GS][8],
                                          const float (&cq)[GS], const float *sA, float *sw, float (&m_u)[GS],
                                          float &m_own, float &l_own, float (&acc)[GS][EV]) {
  constexpr int LK = D / 16, RK = 64 / LK, EBK = ebytes(RAWK), EBV = ebytes(RAWV);
  constexpr int LV = D / EV, RV = 64 / LV, VDW = EV * EBV / 4;
  const rsrc_t rk = make_rsrc(kt, (uint32_t)nt * D * EBK);
  const rsrc_t rv = make_rsrc(vt, (uint32_t)nt * D * EBV);
  const int rrk = lane / LK, ck = lane % LK;
  const float one[1] = {1.0f};
  for (int r0 = 0; r0 < nt; r0 += RK) {
    uint4 kb[1][EBK];
#pragma unroll
    for (int k = 0; k < EBK; ++k) kb[0][k] = bload128(rk, (uint32_t)(rrk * D + ck * 16) * EBK + 16 * k, r0 * D * EBK);
    kcompute<D, GS, RAWK, 1, EBK>(kb, one, nt, lane, qh, cq, sw, r0);
  }
  wave_lds_sync();
  float alpha[GS];
  logits<GS, SP, true>(sA, sw, nt, 1, 1, LR, lane, m_u, m_own, l_own, alpha);
  rescale(acc, alpha);
  wave_lds_sync();
  const int rrv = lane / LV, cv = lane % LV;
  const uint32_t off = (uint32_t)(rrv * D + cv * EV) * EBV;
  for (int r0 = 0; r0 < nt; r0 += RV) {
    uint32_t vb[1][VDW];
#pragma unroll
    for (int k = 0; k < VDW / 4; ++k) {
      const uint4 t = bload128(rv, off + 16 * k, r0 * D * EBV);
      vb[0][4 * k] = t.x; vb[0][4 * k + 1] = t.y; vb[0][4 * k + 2] = t.z; vb[0][4 * k + 3] = t.w;
    }
    vcompute<D, GS, RAWV, 1, VDW, EV>(vb, one, nt, lane, sw, acc, r0);
  }
  wave_lds_sync();
}

template <int D, int GS, int SP, int KF, int VF>
__global__ __launch_bounds__(64 * kDecodeWaves) void decode_kernel(DecodeArgs a) {
  using C = Cfg<D, GS, KF, VF>;
  constexpr int W = C::W, EV = C::EV;
  constexpr int SWR = C::TR > kMaxR ? C::TR : kMaxR;    // tile rows or tail tokens
  constexpr int SW_FLOATS = SWR * GS;
  constexpr int MERGE_FLOATS = W * GS * D + W * GS * 2;
  constexpr int COMB_FLOATS = 2 * kMaxSplits * GS + GS;
  constexpr int LDS_FLOATS = cmax(cmax(W * SW_FLOATS, MERGE_FLOATS), COMB_FLOATS);
  __shared__ float lds[LDS_FLOATS];
  __shared__ __attribute__((aligned(16))) float sA[kMaxR * SP];
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
  const int R = a.R, S = a.S;
  const int LR = R <= 8 ? 1 : (R <= 16 ? 2 : 4);

  // kernel arguments may sit in host-coherent memory: copy A to LDS once
  for (int i = tid; i < R * SP; i += 64 * W) sA[i] = a.A[i];
  float *sw = lds + wave * SW_FLOATS;
  // weights of rows past a tile's end multiply zero data: keep them finite
  for (int i = lane; i < SW_FLOATS; i += 64) sw[i] = 0.0f;
  __syncthreads();

  // ---- query: fp16 pairs of the lane's 16 K elements, pre-scaled per head;
  // done after the first tile's loads are issued so the latencies overlap
  h2 qh[GS][8];
  float cq[GS];
  auto setup_q = [&]() {
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
      amax = group_red<C::LK, true>(amax);
      int E = 0;
      if (amax > 0.0f) frexpf(amax, &E);
      const float up = ldexpf(1.0f, 15 - E);
#pragma unroll
      for (int t = 0; t < 8; ++t) qh[g][t] = h2{(_Float16)(qf[2 * t] * up), (_Float16)(qf[2 * t + 1] * up)};
      cq[g] = a.qk_scale * ldexpf(1.0f, E - 15);
    }
  };

  float m_u[GS];
  float acc[GS][EV];
#pragma unroll
  for (int g = 0; g < GS; ++g) {
    m_u[g] = -INFINITY;
#pragma unroll
    for (int e = 0; e < EV; ++e) acc[g][e] = 0.0f;
  }
  float m_own = -INFINITY, l_own = 0.0f;

  // ---- this wave's tiles: t = wave, wave + W, ... of the split
  const int NB = C::TR / S;
  const int64_t blk0 = (int64_t)split * a.chunk;
  const int64_t blk1 = (blk0 + a.chunk < a.n_blocks) ? blk0 + a.chunk : a.n_blocks;
  const int64_t nblk = blk1 > blk0 ? blk1 - blk0 : 0;
  const int ntiles = (int)((nblk + NB - 1) / NB);
  const int64_t k_bh = bh * a.k_bh_rows, v_bh = bh * a.v_bh_rows;
  auto tile_ref = [&](int t) {
    TileRef T;
    const int64_t tb0 = blk0 + (int64_t)t * NB;
    const int nb = (int)((blk1 - tb0) < NB ? (blk1 - tb0) : NB);
    const int64_t row0 = tb0 * S;
    T.k = static_cast<const char *>(a.krows) + (k_bh + row0) * D * C::EBK;
    T.v = static_cast<const char *>(a.vrows) + (v_bh + row0) * D * C::EBV;
    T.ks = KF == I8 ? a.kscales + k_bh + row0 : nullptr;
    T.vs = VF == I8 ? a.vscales + v_bh + row0 : nullptr;
    T.nrows = nb * S;
    return T;
  };

  if constexpr (GS <= 4) {
    // two register buffers: tile t + W is in flight while tile t is computed
    TileBuf<D, GS, KF, VF> bufA, bufB;
    int t = wave;
    if (t < ntiles) issue(bufA, tile_ref(t), lane);
    setup_q();
    for (; t < ntiles; t += 2 * W) {
      const int t1 = t + W;
      if (t1 < ntiles) issue(bufB, tile_ref(t1), lane);
      __builtin_amdgcn_sched_barrier(0);
      const int n0 = tile_ref(t).nrows;
      process_k<D, GS, SP, KF, VF>(bufA, n0, lane, qh, cq, sw);
      process_lv<D, GS, SP, KF, VF>(bufA, n0, S, R, LR, lane, sA, sw, m_u, m_own, l_own, acc);
      if (t1 < ntiles) {
        const int t2 = t1 + W;
        if (t2 < ntiles) issue(bufA, tile_ref(t2), lane);
        __builtin_amdgcn_sched_barrier(0);
        const int n1 = tile_ref(t1).nrows;
        process_k<D, GS, SP, KF, VF>(bufB, n1, lane, qh, cq, sw);
        process_lv<D, GS, SP, KF, VF>(bufB, n1, S, R, LR, lane, sA, sw, m_u, m_own, l_own, acc);
      }
    }
  } else {
    // one register buffer: the next tile's K rows are requested as soon as
    // this tile's K phase is done, its V rows as soon as the V phase is done
    TileBuf<D, GS, KF, VF> buf;
    int t = wave;
    if (t < ntiles) issue(buf, tile_ref(t), lane);
    setup_q();
    for (; t < ntiles; t += W) {
      const int tn = t + W;
      const int n0 = tile_ref(t).nrows;
      process_k<D, GS, SP, KF, VF>(buf, n0, lane, qh, cq, sw);
      if (tn < ntiles) issue_k(buf, tile_ref(tn), lane);
      __builtin_amdgcn_sched_barrier(0);
      process_lv<D, GS, SP, KF, VF>(buf, n0, S, R, LR, lane, sA, sw, m_u, m_own, l_own, acc);
      if (tn < ntiles) issue_v(buf, tile_ref(tn), lane);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- the raw tail: one wave of the last split
  if (a.n_tail > 0 && split == a.ns - 1 && wave == ntiles % W) {
    const int nt = a.n_tail;
    const char *kt = static_cast<const char *>(a.ktail) + bh * (int64_t)R * D * (a.kraw == BF16 ? 2 : 4);
    const char *vt = static_cast<const char *>(a.vtail) + bh * (int64_t)R * D * (a.vraw == BF16 ? 2 : 4);
    if (a.kraw == BF16 && a.vraw == BF16)
      tail_pass<D, GS, SP, BF16, BF16, EV>(kt, vt, nt, LR, lane, qh, cq, sA, sw, m_u, m_own, l_own, acc);
    else if (a.kraw == F32 && a.vraw == F32)
      tail_pass<D, GS, SP, F32, F32, EV>(kt, vt, nt, LR, lane, qh, cq, sA, sw, m_u, m_own, l_own, acc);
    else if (a.kraw == BF16)
      tail_pass<D, GS, SP, BF16, F32, EV>(kt, vt, nt, LR, lane, qh, cq, sA, sw, m_u, m_own, l_own, acc);
    else
      tail_pass<D, GS, SP, F32, BF16, EV>(kt, vt, nt, LR, lane, qh, cq, sA, sw, m_u, m_own, l_own, acc);
  }

  // ---- wave totals: l over the lanes of a head, acc over the rows of a step
  float l_u[GS];
  {
    const float lt = head_reduce<GS, false>(l_own, LR);
#pragma unroll
    for (int g = 0; g < GS; ++g) l_u[g] = readlane(lt, g * LR);
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

  // ---- the workgroup's partial, published with device-scope stores
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
    __hip_atomic_store(pacc + g * D + d, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (d == 0) {
      __hip_atomic_store(pml + g * 2, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(pml + g * 2 + 1, l, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // Device-scope stores are complete once this thread's memory counter
  // drains; only after every thread's have drained is the arrival counted.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(a.counters + pairq, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_flag = (old == (uint32_t)(a.ns - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!last_flag) return;

  // ---- last arrival: (max, sum) of every split into LDS, weights per split,
  // then every (head, d) sums its split partials with independent loads.
  const float *Pacc = a.part_acc + pairq * a.ns * GS * D;
  const float *Pml = a.part_ml + pairq * a.ns * GS * 2;
  float *cml = lds;                     // [ns*GS][2]; later the weight per split
  float *cM = lds + 2 * a.ns * GS;      // [GS] 1/sum
  for (int i = tid; i < a.ns * GS; i += 64 * W) {
    cml[2 * i] = __hip_atomic_load(Pml + 2 * i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    cml[2 * i + 1] = __hip_atomic_load(Pml + 2 * i + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
      const float p0 = __hip_atomic_load(Pacc + ((sp + 0) * GS + g) * D + d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const float p1 = __hip_atomic_load(Pacc + ((sp + 1) * GS + g) * D + d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const float p2 = __hip_atomic_load(Pacc + ((sp + 2) * GS + g) * D + d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const float p3 = __hip_atomic_load(Pacc + ((sp + 3) * GS + g) * D + d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s0 = fmaf(cml[2 * ((sp + 0) * GS + g)], p0, s0);
      s1 = fmaf(cml[2 * ((sp + 1) * GS + g)], p1, s1);
      s2 = fmaf(cml[2 * ((sp + 2) * GS + g)], p2, s2);
      s3 = fmaf(cml[2 * ((sp + 3) * GS + g)], p3, s3);
    }
    for (; sp < a.ns; ++sp)
      s0 = fmaf(cml[2 * (sp * GS + g)],
                __hip_atomic_load(Pacc + (sp * GS + g) * D + d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), s0);
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
  if (tid == 0) __hip_atomic_store(a.counters + pairq, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, int GS, int SP, int KF, int VF>
int launch_one(const DecodeArgs &a, int64_t n_wg, hipStream_t stream) {
  hipLaunchKernelGGL((decode_kernel<D, GS, SP, KF, VF>), dim3((unsigned)n_wg), dim3(64 * kDecodeWaves), 0, stream,
                     a);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

template <int D, int GS, int KF, int VF>
int launch_sp(int SP, const DecodeArgs &a, int64_t n_wg, hipStream_t stream) {
  switch (SP) {
    case 2: return launch_one<D, GS, 2, KF, VF>(a, n_wg, stream);
    case 4: return launch_one<D, GS, 4, KF, VF>(a, n_wg, stream);
    case 8: return launch_one<D, GS, 8, KF, VF>(a, n_wg, stream);
    case 16: return launch_one<D, GS, 16, KF, VF>(a, n_wg, stream);
    default: return -1;
  }
}

template <int D, int KF, int VF>
int launch_gs(int GS, int SP, const DecodeArgs &a, int64_t n_wg, hipStream_t stream) {
  switch (GS) {
    case 1: return launch_sp<D, 1, KF, VF>(SP, a, n_wg, stream);
    case 2: return launch_sp<D, 2, KF, VF>(SP, a, n_wg, stream);
    case 4: return launch_sp<D, 4, KF, VF>(SP, a, n_wg, stream);
    case 8: return launch_sp<D, 8, KF, VF>(SP, a, n_wg, stream);
    default: return -1;
  }
}

template <int KF, int VF>
int launch_fmt(int D, int GS, int SP, const DecodeArgs &a, int64_t n_wg, hipStream_t stream) {
  switch (D) {
    case 64: return launch_gs<64, KF, VF>(GS, SP, a, n_wg, stream);
    case 128: return launch_gs<128, KF, VF>(GS, SP, a, n_wg, stream);
    case 256: return launch_gs<256, KF, VF>(GS, SP, a, n_wg, stream);
    default: return -1;
  }
}

}  // namespace dec
}  // namespace cdattn
