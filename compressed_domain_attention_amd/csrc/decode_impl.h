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
// all GS query heads of the group (G rounded up to 1, 2, 4 or 8, eight at a
// time beyond that), so each coefficient byte is read from HBM once per
// group.  kDecodeWaves waves per workgroup, one workgroup per CU.
//  * Tiles of TR coefficient rows (about 8 KB of K+V) stream through
//    registers with 16-byte buffer loads; a wave requests its next tile's K
//    rows as soon as its K phase is done and the V rows after the V phase.
//    Loads past a tile's end return zeros, so edges need no branches.
//  * int8 K rows: s = codes . q on v_mfma_i32_16x16x64_i8, the bf16 query
//    split into three signed-byte digits of a 22-bit fixed-point value per
//    head (exact int32 sums, recombined in fp32).  bf16 / fp32 K rows: fp16
//    query pairs against the rows on the VALU.
//  * Logits: z = A s and w = p A on v_mfma_f32_16x16x4_f32 (items = (block,
//    head) columns), base-2 online softmax with log2(e) folded into the
//    scale, running max per head.
//  * int8 V rows: the tile goes to LDS (16-byte chunks XOR-swizzled by row),
//    ds_read_b64_tr_b8 hands out the B operand of v_mfma_i32_16x16x32_i8,
//    and the weights w * vscale per head and 32-row chunk become three
//    signed-byte digits of a 22-bit fixed-point value (A operand).  bf16 V
//    rows: ds_read_b64_tr_b16 and v_mfma_f32_16x16x32_bf16, each weight as
//    three bf16 terms (products exact in fp32).  fp32 V rows: fp32 FMAs on
//    the VALU.
//  * The raw tail (fewer than R tokens, plus a fused new token) runs on the
//    VALU paths in one wave of the last split, before that wave's tiles.
//  * Waves merge in LDS in a fixed order; the workgroup publishes its
//    partial with device-scope stores, waits for them, and bumps a per-(b,
//    h, group) counter; the last workgroup to arrive combines all splits
//    with one round of system-scope loads and writes the output (no second
//    launch, and no L2 write-back or invalidate per workgroup).  A split
//    that is alone writes the output directly.
#pragma once

#include <math.h>

#include <type_traits>

#include "basis_dev.h"
#include "internal.h"

namespace cdattn {
namespace dec {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// op(v[l], v[l ^ 16]) and op(v[l], v[l ^ 32]) through the gfx950 row-pair
// and half-wave swaps (no LDS): with both operands v, the swap returns the
// lane's own value and its partner's, in an order that depends on the lane,
// so op must be commutative (it is: max, or an fp32 sum of two terms).
template <typename Op>
__device__ __forceinline__ float xop16(float v, Op op) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
template <typename Op>
__device__ __forceinline__ float xop32(float v, Op op) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Sum / max over aligned groups of L consecutive lanes (every lane gets it).
template <int L, bool MAX>
__device__ __forceinline__ float group_red(float v) {
  auto op = [](float x, float y) { return MAX ? fmaxf(x, y) : x + y; };
  if constexpr (L >= 2) v = op(v, dpp<0xB1>(v));    // quad_perm [1,0,3,2]
  if constexpr (L >= 4) v = op(v, dpp<0x4E>(v));    // quad_perm [2,3,0,1]
  if constexpr (L >= 8) v = op(v, dpp<0x141>(v));   // row_half_mirror
  if constexpr (L >= 16) v = op(v, dpp<0x140>(v));  // row_mirror
  if constexpr (L >= 32) v = xop16(v, op);
  if constexpr (L >= 64) v = xop32(v, op);
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
  if constexpr (L <= 16) v = xop16(v, op);
  if constexpr (L <= 32) v = xop32(v, op);
  return v;
}

// Maximum over lanes l and l ^ 32 (l ^ 16): the gfx950 half-wave (row pair)
// swaps exchange the two halves, so max(copy, swapped copy) is the pair max.
__device__ __forceinline__ uint32_t umax_x32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max(r[0], r[1]);
}
__device__ __forceinline__ uint32_t umax_x16(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return max(r[0], r[1]);
}

__device__ __forceinline__ float readlane(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

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

constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }

template <int D, int GS, int KF, int VF>
struct Cfg {
  static constexpr int W = kDecodeWaves;
  static constexpr int NBUF = 1;                     // register buffers (tiles in flight) per wave
  static constexpr int EBK = ebytes(KF), EBV = ebytes(VF);
  static constexpr int TR = decode_tile_rows(D, KF, VF);   // rows per tile (K+V ~ 8 KB)
  static constexpr int SWR = cmax(cdiv(TR, 32) * 32, kMaxR);   // rows of the per-head scratch
  static constexpr bool KM = KF == I8;                  // key rows through int8 MFMA
  static constexpr bool VM = VF == I8 || VF == BF16;   // value rows through MFMA (int8 or bf16)
  static constexpr int RBV = D * EBV;                   // bytes of a value row
  // VALU key path: lane = 16 consecutive elements of one row
  static constexpr int LK = D / 16, RK = 64 / LK, KSTEPS = cdiv(TR, RK), KQ = EBK;
  // MFMA key path: 16-row groups x 64-element k steps; N blocks of 4 heads x 4 limb slots
  static constexpr int RG = cdiv(TR, 16), KK = D / 64, NBN = cdiv(GS, 4);
  // VALU value path: lane = EV consecutive elements of one row
  static constexpr int EV = cmin(16, 64 / GS), LV = D / EV, RV = 64 / LV;
  static constexpr int VSTEPS = cdiv(TR, RV), VDW = EV * EBV / 4;
  // MFMA value path: tile staged in LDS; 32-row chunks; M blocks of 4 heads; N blocks of 16 columns
  static constexpr int VQ = cdiv(TR * D * EBV, 1024), CH = SWR / 32, MB = cdiv(GS, 4), NBV = D / 16;
};

// ---------------------------------------------------------------- buffers --
template <int D, int GS, int KF, int VF, bool M = Cfg<D, GS, KF, VF>::KM>
struct KBuf {                 // VALU layout (bf16 / fp32 rows)
  using C = Cfg<D, GS, KF, VF>;
  uint4 k[C::KSTEPS][C::KQ];
};
template <int D, int GS, int KF, int VF>
struct KBuf<D, GS, KF, VF, true> {   // MFMA layout: row 16*rg + lane%16, bytes 64*kk + 16*(lane/16) ..
  using C = Cfg<D, GS, KF, VF>;
  uint4 k[C::RG][C::KK];
  float ks[C::RG];            // scale of row 16*rg + lane%16
};
template <int D, int GS, int KF, int VF, bool M = Cfg<D, GS, KF, VF>::VM>
struct VBuf {                 // VALU layout (bf16 / fp32 rows)
  using C = Cfg<D, GS, KF, VF>;
  uint32_t v[C::VSTEPS][C::VDW];
};
template <int D, int GS, int KF, int VF>
struct VBuf<D, GS, KF, VF, true> {   // contiguous 16-byte chunks, copied to LDS before use
  using C = Cfg<D, GS, KF, VF>;
  uint4 v[C::VQ];
  float vs;                   // scale of row `lane` of the tile
};
template <int D, int GS, int KF, int VF>
struct TileBuf {
  KBuf<D, GS, KF, VF> k;
  VBuf<D, GS, KF, VF> v;
};

// One tile of coefficient rows: its K and V rows and scales, its row count,
// and the head_dim dm of the rows in memory (their pitch; the kernel's
// compute width D is dm rounded up to 64, 128 or 256).
struct TileRef {
  const char *k;
  const char *v;
  const float *ks;
  const float *vs;
  int nrows;
  int dm;
};

#ifdef CDATTN_TIMELINE
constexpr bool kTimeline = true;    // measurement builds: per-wave phase stamps
#else
constexpr bool kTimeline = false;
#endif

constexpr uint32_t kOutOfRange = 0x40000000u;   // a buffer offset past every range: the load reads zeros

template <int D, int GS, int KF, int VF>
__device__ __forceinline__ void issue_k(TileBuf<D, GS, KF, VF> &B, const TileRef &T, int lane) {
  using C = Cfg<D, GS, KF, VF>;
  const int dm = T.dm;
  const rsrc_t rk = make_rsrc(T.k, (uint32_t)T.nrows * dm * C::EBK);
  if constexpr (C::KM) {
    // columns past dm read the next row's codes (or zeros past the tile):
    // they meet zero query digits
    const uint32_t vk = (uint32_t)((lane % 16) * dm + 16 * (lane / 16));
#pragma unroll
    for (int rg = 0; rg < C::RG; ++rg)
#pragma unroll
      for (int kk = 0; kk < C::KK; ++kk) B.k.k[rg][kk] = bload128(rk, vk + 64 * kk, rg * 16 * dm);
    const rsrc_t rs = make_rsrc(T.ks, (uint32_t)T.nrows * 4);
#pragma unroll
    for (int rg = 0; rg < C::RG; ++rg) B.k.ks[rg] = bloadf(rs, 4 * (lane % 16), 64 * rg);
  } else {
    // 16 columns per lane in KQ loads of 16 / KQ columns; loads past dm read zeros
    const int rrk = lane / C::LK, ck = lane % C::LK;
    const uint32_t vk = (uint32_t)(rrk * dm + ck * 16) * C::EBK;
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s)
#pragma unroll
      for (int k = 0; k < C::KQ; ++k)
        B.k.k[s][k] = bload128(rk, ck * 16 + k * (16 / C::KQ) < dm ? vk + 16 * k : kOutOfRange, s * C::RK * dm * C::EBK);
  }
}

template <int D, int GS, int KF, int VF>
__device__ __forceinline__ void issue_v(TileBuf<D, GS, KF, VF> &B, const TileRef &T, int lane) {
  using C = Cfg<D, GS, KF, VF>;
  const int dm = T.dm;
  const rsrc_t rv = make_rsrc(T.v, (uint32_t)T.nrows * dm * C::EBV);
  if constexpr (C::VM) {
    // chunk c of a lane: 16-byte column chunk lane % NCP of tile row
    // lane / NCP + c * 64 / NCP (NCP chunks per row at the compute width;
    // with dm == D that is byte 16 * (lane + 64 c) of the tile).  Chunks past
    // the row's dm columns read zeros; an int8 chunk that straddles dm brings
    // 8 bytes of the next row into columns past dm, which are never output.
    constexpr int NCP = C::RBV / 16;
    const uint32_t vbase = 16 * (lane % NCP) < dm * C::EBV
                               ? (uint32_t)((lane / NCP) * dm * C::EBV + 16 * (lane % NCP))
                               : kOutOfRange;
#pragma unroll
    for (int c = 0; c < C::VQ; ++c) B.v.v[c] = bload128(rv, vbase, c * (64 / NCP) * dm * C::EBV);
    if constexpr (VF == I8) B.v.vs = bloadf(make_rsrc(T.vs, (uint32_t)T.nrows * 4), 4 * lane, 0);
  } else {
    const int rrv = lane / C::LV, cv = lane % C::LV;
    const uint32_t vv = (uint32_t)(rrv * dm + cv * C::EV) * C::EBV;
#pragma unroll
    for (int s = 0; s < C::VSTEPS; ++s) {
      if constexpr (C::VDW % 4 == 0) {
#pragma unroll
        for (int k = 0; k < C::VDW / 4; ++k) {
          const uint4 t = bload128(rv, cv * C::EV + k * (16 / C::EBV) < dm ? vv + 16 * k : kOutOfRange,
                                   s * C::RV * dm * C::EBV);
          B.v.v[s][4 * k] = t.x; B.v.v[s][4 * k + 1] = t.y; B.v.v[s][4 * k + 2] = t.z; B.v.v[s][4 * k + 3] = t.w;
        }
      } else {
        const uint2 t = bload64(rv, cv * C::EV < dm ? vv : kOutOfRange, s * C::RV * dm * C::EBV);
        B.v.v[s][0] = t.x; B.v.v[s][1] = t.y;
      }
    }
  }
}

template <int D, int GS, int KF, int VF>
__device__ __forceinline__ void issue(TileBuf<D, GS, KF, VF> &B, const TileRef &T, int lane) {
  issue_k(B, T, lane);
  issue_v(B, T, lane);
}

// --------------------------------------------------------- int8 digits --
// A value x in [-2^22, 2^22] as balanced base-256 digits x = d0 + 256 d1 +
// 65536 d2 (d0, d1 in [-128, 127], d2 in [-64, 64]), so int8 x int8 products
// summed in int32 reproduce x exactly.  With u = x + 0x808080 (positive),
// digit k is byte k of u minus 128; as an int8 bit pattern that is byte k of
// u with its top bit flipped.  biased() returns u; byte 3 (digit 3) is a
// don't-care slot, multiplied by zero wherever it is used.
__device__ __forceinline__ uint32_t biased(float x) { return (uint32_t)((int)__builtin_rintf(x) + 0x808080); }

// Bytes `which` of four biased values, packed and turned into int8 digits.
__device__ __forceinline__ uint32_t pack_digits(uint32_t u0, uint32_t u1, uint32_t u2, uint32_t u3, int which) {
  const uint32_t sh = 8u * (uint32_t)which;
  const uint32_t p = __builtin_amdgcn_ubfe(u0, sh, 8) | (__builtin_amdgcn_ubfe(u1, sh, 8) << 8) |
                     (__builtin_amdgcn_ubfe(u2, sh, 8) << 16) | (__builtin_amdgcn_ubfe(u3, sh, 8) << 24);
  return p ^ 0x80808080u;
}

typedef int v4i __attribute__((ext_vector_type(4)));

// ------------------------------------------------------ K phase (MFMA) --
// Query of the key MFMA: A operand of v_mfma_i32_16x16x64_i8 for k step kk
// and block nb: row n = lane % 16 holds head 4*nb + n/4, digit n % 4 of the
// query scaled to 22-bit integers; the k bytes are the same head_dim
// elements the codes of this lane hold.  cqq = scale * log2(e) / up for the
// output head of the MFMA at this lane, 4*nb + lane/16.  Every wave converts
// its own copy: the raw loads are issued before the first tile's, the
// conversion runs once they have landed.
template <int D, int GS, bool FULL>
struct QRegMfma {
  static constexpr int KK = D / 64, NBN = cdiv(GS, 4);
  uint4 raw[NBN][KK][2];
  // Plain global loads (the lanes read different heads; a buffer resource
  // per lane would have to be made uniform one head at a time), issued
  // unconditionally so that no wait is needed until the conversion.  Rows
  // narrower than D (FULL false): a half of 8 columns at or past a.Dm (a
  // multiple of 8) reads column 0 instead, and the conversion takes it as
  // zero.
  // Heads g >= gv of the group (past the kv head's query heads) read head 0.
  __device__ __forceinline__ void load(const DecodeArgs &a, int b, int hq0, int gv, int lane) {
    const int n = lane % 16, G = lane / 16;
#pragma unroll
    for (int nb = 0; nb < NBN; ++nb) {
      const int g = 4 * nb + n / 4;
      const int gl = g < gv ? g : 0;   // columns of absent heads read a live one and are zeroed below
      const uint4 *qh = reinterpret_cast<const uint4 *>(a.q + (int64_t)b * a.q_sb + (int64_t)(hq0 + gl) * a.q_sh);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int c = 64 * kk + 16 * G + 8 * hf;
          raw[nb][kk][hf] = qh[FULL || c < a.Dm ? c / 8 : 0];
        }
    }
  }
  __device__ __forceinline__ void convert(const DecodeArgs &a, int lane, uint4 (&qB)[KK][NBN],
                                          float (&cqq)[NBN]) const {
    const int n = lane % 16, which = n % 4, G = lane / 16;
#pragma unroll
    for (int nb = 0; nb < NBN; ++nb) {
      const bool live = 4 * nb + n / 4 < GS;
      float qf[KK][16];
      float amax = 0.0f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const uint32_t wv[8] = {raw[nb][kk][0].x, raw[nb][kk][0].y, raw[nb][kk][0].z, raw[nb][kk][0].w,
                                raw[nb][kk][1].x, raw[nb][kk][1].y, raw[nb][kk][1].z, raw[nb][kk][1].w};
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const bool in = live && (FULL || 64 * kk + 16 * G + 8 * (t / 4) < a.Dm);
          qf[kk][2 * t] = in ? bf16lo(wv[t]) : 0.0f;
          qf[kk][2 * t + 1] = in ? bf16hi(wv[t]) : 0.0f;
          amax = fmaxf(amax, fmaxf(fabsf(qf[kk][2 * t]), fabsf(qf[kk][2 * t + 1])));
        }
      }
      amax = xop16(amax, [](float x, float y) { return fmaxf(x, y); });
      amax = xop32(amax, [](float x, float y) { return fmaxf(x, y); });
      int E = 0;
      if (amax > 0.0f) frexpf(amax, &E);
      const float up = ldexpf(1.0f, 22 - E);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        uint32_t u[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) u[e] = biased(qf[kk][e] * up);
        qB[kk][nb] = make_uint4(pack_digits(u[0], u[1], u[2], u[3], which), pack_digits(u[4], u[5], u[6], u[7], which),
                                pack_digits(u[8], u[9], u[10], u[11], which),
                                pack_digits(u[12], u[13], u[14], u[15], which));
      }
      // lane 4*(lane/16) holds head 4*nb + lane/16 in its row group
      cqq[nb] = __shfl(a.qk_scale * ldexpf(1.0f, E - 22), 4 * (lane / 16), 64);
    }
  }
};

// s[g][row] = cqq[g] * kscale[row] * sum_d code[row][d] * qint[g][d] for the
// tile's rows.  The query digits are the A operand (row 4*head + digit) and
// the codes the B operand, so lane l receives the three digit sums of head
// 4*nb + l/16 and row 16*rg + l%16 in its own registers; the int32 sums are
// exact and recombined in fp32.  Absent heads store to the junk slots.
template <int D, int GS, int SWR, int KF, int VF>
__device__ __forceinline__ void kcompute_mfma(const KBuf<D, GS, KF, VF, true> &kb, int lane,
                                              const uint4 (&qB)[D / 64][cdiv(GS, 4)], const float (&cqq)[cdiv(GS, 4)],
                                              float *sw) {
  using C = Cfg<D, GS, KF, VF>;
#pragma unroll
  for (int rg = 0; rg < C::RG; ++rg) {
#pragma unroll
    for (int nb = 0; nb < C::NBN; ++nb) {
      v4i acc = {0, 0, 0, 0};
#pragma unroll
      for (int kk = 0; kk < C::KK; ++kk)
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, qB[kk][nb]),
                                                     __builtin_bit_cast(v4i, kb.k[rg][kk]), acc, 0, 0, 0);
      const float sv = ((float)acc[0] + 256.0f * (float)acc[1]) + 65536.0f * (float)acc[2];
      const int g = 4 * nb + lane / 16;
      sw[g < GS ? g * SWR + 16 * rg + lane % 16 : GS * SWR + lane] = sv * kb.ks[rg] * cqq[nb];
    }
  }
}

// ------------------------------------------------------ V phase (MFMA) --
// The tile's value rows (RB bytes each) go to LDS row-major with 16-byte
// chunks XOR swizzled by row, so the transpose reads below hit distinct banks.
template <int RB>
__device__ __forceinline__ int vlds_off(int row, int chunk16) {
  constexpr int NC = RB / 16, SW = NC < 8 ? NC : 8;
  return row * RB + ((chunk16 ^ (row % SW)) * 16);
}

// (x, y) rounded to bf16 (ties to even, v_cvt_pk_bf16_f32), x in the low half.
__device__ __forceinline__ uint32_t pk_bf16(float x, float y) {
  typedef float f2v __attribute__((ext_vector_type(2)));
  typedef __bf16 b2v __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v){x, y}, b2v));
}

// bf16 value rows (no scales): acc[mb][nb] += sum over the tile's rows of
// w[g][row] * v[row][col] on v_mfma_f32_16x16x32_bf16.  Each weight is split
// into three bf16 terms hi + mid + lo (each the rounded remainder of the one
// before, together the fp32 weight to its last bits); A row m = 4 * head +
// term (term 3 is zero), so one MFMA forms the three partial sums of a head,
// each product exact in fp32, and the lane adds them.  The values come from
// LDS through ds_read_b64_tr_b16, which hands lane i of a 16-lane group
// element (i % 4) of the 8 bytes addressed by lane 4j + i/4, j = 0..3: with
// lane k pointing at row r + k/4, columns 4*(k%4) .. of the block, lane i
// receives column i of rows r .. r+3; two reads give the 8 rows of the B
// operand.  Rows past the staged tile are zero (cleared once), rows past
// nrows have zero weight.
template <int D, int GS, int SWR, int KF, int VF>
__device__ __forceinline__ void vcompute_mfma_bf16(int nrows, int lane, const float *sw, const char *vl,
                                                   float (&acc)[cdiv(GS, 4)][D / 16]) {
  using C = Cfg<D, GS, KF, VF>;
  typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef short v8s __attribute__((ext_vector_type(8)));
  typedef float f4v __attribute__((ext_vector_type(4)));
  const int m = lane % 16, G = lane / 16, k = lane % 16;
  const int term = m % 4;
#pragma unroll
  for (int ch = 0; ch < C::CH; ++ch) {
    const int r0 = 32 * ch + 8 * G;
    v8bf A[C::MB];
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
      const int g = 4 * mb + m / 4;
      const float *wp = sw + (g < GS ? g : 0) * SWR + r0;
      const float4 wa = *reinterpret_cast<const float4 *>(wp);
      const float4 wb = *reinterpret_cast<const float4 *>(wp + 4);
      const float wr[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
      // pairs of weights: three packed roundings (hi, mid, lo), each of the
      // remainder left by the ones before; the lane keeps its term (term 3: zero)
      uint32_t a[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float w0 = (g < GS && r0 + 2 * p < nrows) ? wr[2 * p] : 0.0f;
        const float w1 = (g < GS && r0 + 2 * p + 1 < nrows) ? wr[2 * p + 1] : 0.0f;
        const uint32_t t0 = pk_bf16(w0, w1);
        const float x0 = w0 - __uint_as_float(t0 << 16), x1 = w1 - __uint_as_float(t0 & 0xFFFF0000u);
        const uint32_t t1 = pk_bf16(x0, x1);
        const float y0 = x0 - __uint_as_float(t1 << 16), y1 = x1 - __uint_as_float(t1 & 0xFFFF0000u);
        const uint32_t t2 = pk_bf16(y0, y1);
        a[p] = term == 0 ? t0 : (term == 1 ? t1 : (term == 2 ? t2 : 0u));
      }
      A[mb] = __builtin_bit_cast(v8bf, a);
    }
    const int trow = r0 + k / 4;
#pragma unroll
    for (int nb = 0; nb < C::NBV; ++nb) {
      const int cb = 2 * nb + (k % 4) / 2;   // 16-byte chunk of columns 16 nb + 4 (k % 4) ..
      const v4s b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s *)(vl + vlds_off<C::RBV>(trow, cb) + 8 * (k % 2)));
      const v4s b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s *)(vl + vlds_off<C::RBV>(trow + 4, cb) + 8 * (k % 2)));
      const v8s bb = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
      const v8bf B = __builtin_bit_cast(v8bf, bb);
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        const f4v z = {0.0f, 0.0f, 0.0f, 0.0f};
        const f4v c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mb], B, z, 0, 0, 0);
        acc[mb][nb] += (c[0] + c[1]) + c[2];
      }
    }
  }
}

// acc[mb][nb] (lane: head 4*mb + lane/16, column 16*nb + lane%16) +=
//   sum over the tile's rows of w[g][row] * vscale[row] * code[row][col].
// Per 32-row chunk and M block: the weights of 4 heads become 22-bit integers
// (scale per head and chunk) split in three signed bytes, the A operand of
// v_mfma_i32_16x16x32_i8 (row m = head*4 + digit); the value codes come from
// LDS through ds_read_b64_tr_b8, which hands lane i of a 16-lane group byte
// (i % 8) of the 8 bytes addressed by lane 2j + i/8, j = 0..7: with lane k
// of group G pointing at row 8G + k/2, columns 8*(k%2) .. of the block, lane
// i receives column i of rows 8G .. 8G+7, the B operand of the MFMA.
template <int D, int GS, int SWR, int KF, int VF>
__device__ __forceinline__ void vcompute_mfma(const VBuf<D, GS, KF, VF, true> &vb, int nrows, int lane,
                                              const float *sw, char *vl, float *svs,
                                              float (&acc)[cdiv(GS, 4)][D / 16]) {
  using C = Cfg<D, GS, KF, VF>;
#pragma unroll
  for (int c = 0; c < C::VQ; ++c) {
    const int q = lane + 64 * c;            // 16-byte chunk of the tile
    const int row = q / (C::RBV / 16), ch16 = q % (C::RBV / 16);
    if (row < SWR) *reinterpret_cast<uint4 *>(vl + vlds_off<C::RBV>(row, ch16)) = vb.v[c];
  }
  if constexpr (VF == I8) svs[lane] = vb.vs;
  wave_lds_sync();
  const int m = lane % 16, G = lane / 16;
  const int which = m % 4;
  if constexpr (VF == BF16) {
    vcompute_mfma_bf16<D, GS, SWR, KF, VF>(nrows, lane, sw, vl, acc);
    wave_lds_sync();
    return;
  }
#pragma unroll
  for (int ch = 0; ch < C::CH; ++ch) {
    const float4 vs0 = *reinterpret_cast<const float4 *>(svs + 32 * ch + 8 * G);
    const float4 vs1 = *reinterpret_cast<const float4 *>(svs + 32 * ch + 8 * G + 4);
    const float vsj[8] = {vs0.x, vs0.y, vs0.z, vs0.w, vs1.x, vs1.y, vs1.z, vs1.w};
    const int r0 = 32 * ch + 8 * G;
    // the B operands of every N block first: their LDS reads overlap the
    // weight conversion, and the MFMAs below then issue back to back
    typedef int v2i __attribute__((ext_vector_type(2)));
    v2i bt[C::NBV];
    {
      const int k = lane % 16;
      const int trow = 32 * ch + 8 * G + k / 2;
#pragma unroll
      for (int nb = 0; nb < C::NBV; ++nb)
        bt[nb] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) v2i *)(vl + vlds_off<C::RBV>(trow, nb) + 8 * (k % 2)));
    }
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
      const int g = 4 * mb + m / 4;
      // the lane's 8 weights: two aligned 16-byte reads (absent heads read
      // head 0), rows past the tile's end and absent heads selected to zero
      const float *wp = sw + (g < GS ? g : 0) * SWR + r0;
      const float4 wa = *reinterpret_cast<const float4 *>(wp);
      const float4 wb = *reinterpret_cast<const float4 *>(wp + 4);
      const float wr[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
      float w[8];
      uint32_t ubits = 0;   // max |w| as bits: non-negative floats order like their bit patterns
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bool ok = g < GS && r0 + j < nrows;
        w[j] = ok ? wr[j] * vsj[j] : 0.0f;
        ubits = max(ubits, __float_as_uint(fabsf(w[j])));
      }
      ubits = umax_x16(umax_x32(ubits));
      const float amax = __uint_as_float(ubits);
      int E = 0;
      if (amax > 0.0f) frexpf(amax, &E);
      const float up = ldexpf(1.0f, 22 - E);
      uint32_t u[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) u[j] = biased(w[j] * up);
      const long A = (long)pack_digits(u[0], u[1], u[2], u[3], which) |
                     ((long)pack_digits(u[4], u[5], u[6], u[7], which) << 32);
      // per-head scale of this chunk for the output layout (head = 4*mb + lane/16)
      const float down = ldexpf(1.0f, E - 22);
      const float d0 = readlane(down, 0), d1 = readlane(down, 4), d2 = readlane(down, 8), d3 = readlane(down, 12);
      const float dn = G == 0 ? d0 : (G == 1 ? d1 : (G == 2 ? d2 : d3));
      v4i c[C::NBV];
#pragma unroll
      for (int nb = 0; nb < C::NBV; ++nb) {
        const v4i z = {0, 0, 0, 0};
        c[nb] = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, __builtin_bit_cast(long, bt[nb]), z, 0, 0, 0);
      }
#pragma unroll
      for (int nb = 0; nb < C::NBV; ++nb)
        acc[mb][nb] = fmaf(dn, ((float)c[nb][0] + 256.0f * (float)c[nb][1]) + 65536.0f * (float)c[nb][2], acc[mb][nb]);
    }
  }
  wave_lds_sync();
}

template <int GS, int MBK, int NBK>
__device__ __forceinline__ void rescale_mfma(float (&acc)[MBK][NBK], const float (&alpha)[GS], int lane) {
  bool moved = false;
#pragma unroll
  for (int g = 0; g < GS; ++g) moved |= alpha[g] != 1.0f;
  if (!moved) return;
  const int G = lane / 16;
#pragma unroll
  for (int mb = 0; mb < MBK; ++mb) {
    float al = 1.0f;
#pragma unroll
    for (int h = 0; h < 4; ++h)
      if (4 * mb + h < GS && G == h) al = alpha[4 * mb + h];
#pragma unroll
    for (int nb = 0; nb < NBK; ++nb) acc[mb][nb] *= al;
  }
}

// ------------------------------------------------------- VALU query setup --
// fp16 pairs of the lane's 16 key elements (lane % (D/16) picks them),
// pre-scaled per head by a power of two into fp16 range; loads issued first,
// converted once other loads are in flight.
template <int D, int GS, bool FULL>
struct QRegValu {
  static constexpr int LK = D / 16;
  uint4 raw[GS][2];
  // Unconditional loads (no wait before the conversion).  Rows narrower than
  // D (FULL false): a half of 8 columns at or past a.Dm (a multiple of 8)
  // reads column 0 instead, and the conversion takes it as zero.
  // Heads g >= gv of the group (past the kv head's query heads) read head 0.
  __device__ __forceinline__ void load(const DecodeArgs &a, int b, int hq0, int gv, int lane) {
#pragma unroll
    for (int g = 0; g < GS; ++g) {
      const int gl = g < gv ? g : 0;
      const uint4 *qh = reinterpret_cast<const uint4 *>(a.q + (int64_t)b * a.q_sb + (int64_t)(hq0 + gl) * a.q_sh);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int c = (lane % LK) * 16 + 8 * hf;
        raw[g][hf] = qh[FULL || c < a.Dm ? c / 8 : 0];
      }
    }
  }
  __device__ __forceinline__ void convert(const DecodeArgs &a, int lane, h2 (&qh)[GS][8], float (&cq)[GS]) const {
#pragma unroll
    for (int g = 0; g < GS; ++g) {
      const uint32_t wv[8] = {raw[g][0].x, raw[g][0].y, raw[g][0].z, raw[g][0].w,
                              raw[g][1].x, raw[g][1].y, raw[g][1].z, raw[g][1].w};
      float qf[16];
      float amax = 0.0f;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const bool in = FULL || (lane % LK) * 16 + 8 * (t / 4) < a.Dm;
        qf[2 * t] = in ? bf16lo(wv[t]) : 0.0f;
        qf[2 * t + 1] = in ? bf16hi(wv[t]) : 0.0f;
        amax = fmaxf(amax, fmaxf(fabsf(qf[2 * t]), fabsf(qf[2 * t + 1])));
      }
      amax = group_red<LK, true>(amax);
      int E = 0;
      if (amax > 0.0f) frexpf(amax, &E);
      const float up = ldexpf(1.0f, 15 - E);
#pragma unroll
      for (int t = 0; t < 8; ++t) qh[g][t] = h2{(_Float16)(qf[2 * t] * up), (_Float16)(qf[2 * t + 1] * up)};
      cq[g] = a.qk_scale * ldexpf(1.0f, E - 15);
    }
  }
};
// ------------------------------------------------------- K phase (VALU) --
// bf16 / fp32 key rows and the raw tail.
// s[g][row] = cq[g] * sum_d k[row][d] * q[g][d]; 16 elements per lane held in
// F's bytes (KQ uint4), the query in pre-scaled fp16 pairs.
template <int D, int GS, int SWR, int F, int STEPS, int KQ>
__device__ __forceinline__ void kcompute(const uint4 (&kb)[STEPS][KQ], int nrows, int lane, h2 (&qh)[GS][8],
                                         const float (&cq)[GS], float *sw, int row_base = 0) {
  static_assert(F != I8, "int8 key rows take the MFMA path");
  constexpr int LK = D / 16, RK = 64 / LK;
  const int rr = lane / LK, c = lane % LK;
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    if (row_base + s * RK >= nrows) break;
    const int row = row_base + s * RK + rr;
    float dot[GS];
#pragma unroll
    for (int g = 0; g < GS; ++g) dot[g] = 0.0f;
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
#pragma unroll
    for (int g = 0; g < GS; ++g) dot[g] = group_red<LK, false>(dot[g]);
    if (c == 0 && row < nrows) {
#pragma unroll
      for (int g = 0; g < GS; ++g) sw[g * SWR + row] = dot[g] * cq[g];
    }
  }
}

// ------------------------------------------------------- V phase (VALU) --
// bf16 / fp32 value rows and the raw tail.
// acc[g][e] += sum over rows of w[g][row] * v[row][c*EV + e].
// Rows past nrows hold zero data (buffer range) and finite stale weights.
template <int D, int GS, int SWR, int F, int STEPS, int VDW, int EV>
__device__ __forceinline__ void vcompute(const uint32_t (&vb)[STEPS][VDW], int nrows, int lane, const float *sw,
                                         float (&acc)[GS][EV], int row_base = 0) {
  static_assert(F != I8, "int8 value rows take the MFMA path");
  constexpr int LV = D / EV, RV = 64 / LV;
  const int rr = lane / LV;
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    if (row_base + s * RV >= nrows) break;
    const int row = row_base + s * RV + rr;
    float w[GS];
#pragma unroll
    for (int g = 0; g < GS; ++g) w[g] = sw[g * SWR + row];
    float v[EV];
    if constexpr (F == BF16) {
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
// Per tile, with s = the K-phase scores in sw (head-major, row n*S + j of
// block n): z = A s per (block, head) item, the running max per head,
// p = 2^(z - max), l += sum p and the value weights w = p A, written back
// over s.  Both small products run on v_mfma_f32_16x16x4_f32 (lane l holds
// A[l%16][l/16] and B[l/16][l%16]; result register i of lane l is
// D[4(l/16)+i][l%16]): items (block n, head g) are the 16 columns of a
// group, item it = n*GS + g, so the head of a lane is fixed: (l%16) % GS.
//   z:  M = 16 tokens of a block, K = 4 coefficients per step, N = items.
//   w:  M = items, K = 4 tokens per step, N = coefficients; step kk takes
//       token 4(l/16) + kk from the lane that computed it, so p never moves.
// Tokens past R and items past the tile's blocks are masked.  A first pass
// takes the max, a second recomputes z (MFMA is cheap) and forms p and w.
typedef float v4f __attribute__((ext_vector_type(4)));

template <int SP>
struct Basis {
  static constexpr int SK = SP < 4 ? 1 : SP / 4;   // 4-coefficient steps
  float az[2][SK];   // A operand of z, token tile rt: A[16 rt + l%16][4 kk + l/16]
  float bw[2][4];    // B operand of w, token tile rt: A[16 rt + 4 (l/16) + kk][l%16]
  float bwh[2][4];   // SP > 16: the same for coefficients 16 .. 31, A[..][16 + l%16]
  int rt_n;          // token tiles of 16: 1 if R <= 16 else 2
  // SP = 2 with R <= 8: two items per MFMA column (item half h = rows 8h ..
  // of z, coefficients 2h .. of its B operand, columns S h .. of w):
  // A operand of z, A'[l%16][l/16]; B operand of w, B'[l/16][l%16] per step
  float azp;
  float bwp[4];
  // Operand registers from the workgroup's copy sA of the synthesis basis
  // (entry r * SP + j, zero past row R and column S).
  __device__ __forceinline__ void load(const float *sA, int R, int S, int lane) {
    const int lo = lane % 16, hi = lane / 16;
    rt_n = R > 16 ? 2 : 1;
    if constexpr (SP == 2) {
      const int h = lo / 8, t = lo % 8, j = hi - 2 * h;
      azp = (hi / 2 == h && t < R && j >= 0 && j < S) ? sA[t * SP + j] : 0.0f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int hb = hi / 2, tb = 4 * (hi % 2) + kk, jb = lo - S * hb;
        bwp[kk] = (tb < R && jb >= 0 && jb < S) ? sA[tb * SP + jb] : 0.0f;
      }
    }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
      for (int kk = 0; kk < SK; ++kk) {
        const int r = 16 * rt + lo, j = 4 * kk + hi;
        az[rt][kk] = (r < R && j < S) ? sA[r * SP + j] : 0.0f;
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int r = 16 * rt + 4 * hi + kk, j = lo;
        bw[rt][kk] = (r < R && j < S) ? sA[r * SP + j] : 0.0f;
        if constexpr (SP > 16) bwh[rt][kk] = (r < R && 16 + j < S) ? sA[r * SP + 16 + j] : 0.0f;
      }
    }
  }
  // every token its own block (the raw tail): R = S = 1, A = [1]
  __device__ __forceinline__ void unit(int lane) {
    rt_n = 1;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
      for (int kk = 0; kk < SK; ++kk) az[rt][kk] = (rt == 0 && kk == 0 && lane == 0) ? 1.0f : 0.0f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        bw[rt][kk] = (rt == 0 && kk == 0 && lane == 0) ? 1.0f : 0.0f;
        bwh[rt][kk] = 0.0f;
      }
    }
  }
};

template <int GS, int SP, int SWR>
__device__ __forceinline__ void logits_any(const Basis<SP> &A, float *sw, int nb, int R, int S, int lane,
                                       float (&m_u)[GS], float &m_lane, float &l_lane, float (&alpha)[GS]) {
  constexpr int SK = Basis<SP>::SK;
  const int col = lane % 16, hi = lane / 16;
  const int g = col % GS;
  const int items = nb * GS;
  const int ngroups = (items + 15) / 16;
  auto zgroup = [&](int ig, int rt) {
    const int it = ig * 16 + col;
    const bool ok = it < items;
    const int base = g * SWR + (it / GS) * S;
    v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < SK; ++kk) {
      const int j = 4 * kk + hi;
      const bool live = ok && j < S;
      const float sv = sw[live ? base + j : 0];
      z = __builtin_amdgcn_mfma_f32_16x16x4f32(A.az[rt][kk], live ? sv : 0.0f, z, 0, 0, 0);
    }
    return z;
  };
  // First pass: the lane's max.  The running max is only moved when some
  // logit exceeds it by more than kSlack (base 2): otherwise p <= 2^kSlack,
  // harmless in fp32, and neither the head reduction nor a rescale is needed.
  constexpr float kSlack = 8.0f;
  float mx = -INFINITY;
#pragma unroll 2
  for (int ig = 0; ig < ngroups; ++ig) {
    const bool ok = ig * 16 + col < items;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      if (rt < A.rt_n) {
        const v4f z = zgroup(ig, rt);
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = (ok && 16 * rt + 4 * hi + i < R) ? fmaxf(mx, z[i]) : mx;
      }
    }
  }
  float m_new = m_lane, a_lane = 1.0f;
  if (__builtin_amdgcn_ballot_w64(mx > m_lane + kSlack) != 0) {
    mx = strided<GS, true>(mx);
    m_new = fmaxf(m_lane, mx);
    a_lane = m_new == m_lane ? 1.0f : __builtin_amdgcn_exp2f(m_lane - m_new);
#pragma unroll
    for (int gg = 0; gg < GS; ++gg) m_u[gg] = readlane(m_new, gg);
  }
#pragma unroll
  for (int gg = 0; gg < GS; ++gg) alpha[gg] = readlane(a_lane, gg);
  m_lane = m_new;
  float lsum = 0.0f;
#pragma unroll 2
  for (int ig = 0; ig < ngroups; ++ig) {
    const bool ok = ig * 16 + col < items;
    v4f w = {0.0f, 0.0f, 0.0f, 0.0f}, wh = w;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      if (rt < A.rt_n) {
        const v4f z = zgroup(ig, rt);
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[i] = (ok && 16 * rt + 4 * hi + i < R) ? __builtin_amdgcn_exp2f(z[i] - m_new) : 0.0f;
          lsum += p[i];
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) w = __builtin_amdgcn_mfma_f32_16x16x4f32(p[kk], A.bw[rt][kk], w, 0, 0, 0);
        if constexpr (SP > 16) {
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) wh = __builtin_amdgcn_mfma_f32_16x16x4f32(p[kk], A.bwh[rt][kk], wh, 0, 0, 0);
        }
      }
    }
    // lane (hi, j = col) holds w of items ig*16 + 4 hi + i, coefficient j
    // (and coefficient 16 + j in wh)
    if (col < S) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int it = ig * 16 + 4 * hi + i;
        if (it < items) sw[(it % GS) * SWR + (it / GS) * S + col] = w[i];
      }
    }
    if constexpr (SP > 16) {
      if (16 + col < S) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int it = ig * 16 + 4 * hi + i;
          if (it < items) sw[(it % GS) * SWR + (it / GS) * S + 16 + col] = wh[i];
        }
      }
    }
  }
  l_lane = l_lane * a_lane + lsum;
}

// Tile version: at most NG groups (a compile-time bound for the tile's
// blocks), one token tile (R <= 16).  z is computed once and kept in
// registers between the max and the exponentials; the four w products of a
// group go to independent accumulators.  Other shapes take logits_any.
template <int GS, int SP, int SWR, int NG>
__device__ __forceinline__ void logits(const Basis<SP> &A, float *sw, int nb, int R, int S, int lane,
                                       float (&m_u)[GS], float &m_lane, float &l_lane, float (&alpha)[GS]) {
  constexpr int SK = Basis<SP>::SK;
  const int items = nb * GS;
  const int ngroups = (items + 15) / 16;
  if (A.rt_n != 1 || ngroups > NG) {
    logits_any<GS, SP, SWR>(A, sw, nb, R, S, lane, m_u, m_lane, l_lane, alpha);
    return;
  }
  const int col = lane % 16, hi = lane / 16;
  const int g = col % GS;
  constexpr float kSlack = 8.0f;
  v4f z[NG];
  float mx = -INFINITY;
#pragma unroll
  for (int ig = 0; ig < NG; ++ig) {
    if (ig < ngroups) {
      const int it = ig * 16 + col;
      const bool ok = it < items;
      const int base = g * SWR + (it / GS) * S;
      v4f zz = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < SK; ++kk) {
        const int j = 4 * kk + hi;
        const bool live = ok && j < S;
        const float sv = sw[live ? base + j : 0];
        zz = __builtin_amdgcn_mfma_f32_16x16x4f32(A.az[0][kk], live ? sv : 0.0f, zz, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool v = ok && 4 * hi + i < R;
        zz[i] = v ? zz[i] : -INFINITY;
        mx = fmaxf(mx, zz[i]);
      }
      z[ig] = zz;
    }
  }
  float m_new = m_lane, a_lane = 1.0f;
  if (__builtin_amdgcn_ballot_w64(mx > m_lane + kSlack) != 0) {
    mx = strided<GS, true>(mx);
    m_new = fmaxf(m_lane, mx);
    a_lane = m_new == m_lane ? 1.0f : __builtin_amdgcn_exp2f(m_lane - m_new);
#pragma unroll
    for (int gg = 0; gg < GS; ++gg) {
      m_u[gg] = readlane(m_new, gg);
      alpha[gg] = readlane(a_lane, gg);
    }
  } else {
#pragma unroll
    for (int gg = 0; gg < GS; ++gg) alpha[gg] = 1.0f;
  }
  m_lane = m_new;
  float lsum = 0.0f;
#pragma unroll
  for (int ig = 0; ig < NG; ++ig) {
    if (ig < ngroups) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = __builtin_amdgcn_exp2f(z[ig][i] - m_new);   // masked tokens: exp2(-inf) = 0
        lsum += p[i];
      }
      v4f w0 = {0.0f, 0.0f, 0.0f, 0.0f}, w1 = w0, w2 = w0, w3 = w0;
      w0 = __builtin_amdgcn_mfma_f32_16x16x4f32(p[0], A.bw[0][0], w0, 0, 0, 0);
      w1 = __builtin_amdgcn_mfma_f32_16x16x4f32(p[1], A.bw[0][1], w1, 0, 0, 0);
      w2 = __builtin_amdgcn_mfma_f32_16x16x4f32(p[2], A.bw[0][2], w2, 0, 0, 0);
      w3 = __builtin_amdgcn_mfma_f32_16x16x4f32(p[3], A.bw[0][3], w3, 0, 0, 0);
      // lane (hi, j = col) holds w of items ig*16 + 4 hi + i, coefficient j;
      // lanes without a live (item, coefficient) store to the junk slots
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int it = ig * 16 + 4 * hi + i;
        const bool ok = col < S && it < items;
        sw[ok ? (it % GS) * SWR + (it / GS) * S + col : GS * SWR + lane] = (w0[i] + w1[i]) + (w2[i] + w3[i]);
      }
      if constexpr (SP > 16) {
        // coefficients 16 .. 31
        w0 = w1 = w2 = w3 = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        w0 = __builtin_amdgcn_mfma_f32_16x16x4f32(p[0], A.bwh[0][0], w0, 0, 0, 0);
        w1 = __builtin_amdgcn_mfma_f32_16x16x4f32(p[1], A.bwh[0][1], w1, 0, 0, 0);
        w2 = __builtin_amdgcn_mfma_f32_16x16x4f32(p[2], A.bwh[0][2], w2, 0, 0, 0);
        w3 = __builtin_amdgcn_mfma_f32_16x16x4f32(p[3], A.bwh[0][3], w3, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int it = ig * 16 + 4 * hi + i;
          const bool ok = 16 + col < S && it < items;
          sw[ok ? (it % GS) * SWR + (it / GS) * S + 16 + col : GS * SWR + lane] = (w0[i] + w1[i]) + (w2[i] + w3[i]);
        }
      }
    }
  }
  l_lane = l_lane * a_lane + lsum;
}

// Tile version for SP = 2 and R <= 8: two (block, head) items per MFMA
// column, so a group holds 32 items and both products run on half as many
// groups.  Column n of group ig holds items ig*32 + n and ig*32 + 16 + n (the
// same head); lane (hi, col) gives coefficient hi % 2 of item half hi / 2 and
// receives z rows 4 hi .. 4 hi + 3, tokens 4 (hi % 2) .. of that item half;
// w comes out with item half h in columns S h .. S h + S - 1.  Other shapes
// (S = 1 tiles with more groups, R > 8) take logits / logits_any.
template <int GS, int SWR, int NGP>
__device__ __forceinline__ bool logits_packed(const Basis<2> &A, float *sw, int nb, int R, int S, int lane,
                                              float (&m_u)[GS], float &m_lane, float &l_lane, float (&alpha)[GS]) {
  const int items = nb * GS;
  const int ngroups = (items + 31) / 32;
  if (R > 8 || ngroups > NGP) return false;
  const int col = lane % 16, hi = lane / 16;
  const int g = col % GS, hh = hi / 2, jb = hi % 2;
  constexpr float kSlack = 8.0f;
  v4f z[NGP];
  float mx = -INFINITY;
#pragma unroll
  for (int ig = 0; ig < NGP; ++ig) {
    if (ig < ngroups) {
      const int it = ig * 32 + 16 * hh + col;
      const bool live = it < items && jb < S;
      const float sv = sw[live ? g * SWR + (it / GS) * S + jb : 0];
      v4f zz = {0.0f, 0.0f, 0.0f, 0.0f};
      zz = __builtin_amdgcn_mfma_f32_16x16x4f32(A.azp, live ? sv : 0.0f, zz, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool v = it < items && 4 * jb + i < R;
        zz[i] = v ? zz[i] : -INFINITY;
        mx = fmaxf(mx, zz[i]);
      }
      z[ig] = zz;
    }
  }
  float m_new = m_lane, a_lane = 1.0f;
  if (__builtin_amdgcn_ballot_w64(mx > m_lane + kSlack) != 0) {
    mx = strided<GS, true>(mx);
    m_new = fmaxf(m_lane, mx);
    a_lane = m_new == m_lane ? 1.0f : __builtin_amdgcn_exp2f(m_lane - m_new);
#pragma unroll
    for (int gg = 0; gg < GS; ++gg) {
      m_u[gg] = readlane(m_new, gg);
      alpha[gg] = readlane(a_lane, gg);
    }
  } else {
#pragma unroll
    for (int gg = 0; gg < GS; ++gg) alpha[gg] = 1.0f;
  }
  m_lane = m_new;
  float lsum = 0.0f;
  // output column col: item half hs = col / S (col < 2 S), coefficient col - S hs
  const int hs = col < S ? 0 : 1, jo = col - S * hs;
#pragma unroll
  for (int ig = 0; ig < NGP; ++ig) {
    if (ig < ngroups) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = __builtin_amdgcn_exp2f(z[ig][i] - m_new);   // masked tokens: exp2(-inf) = 0
        lsum += p[i];
      }
      v4f w0 = {0.0f, 0.0f, 0.0f, 0.0f}, w1 = w0, w2 = w0, w3 = w0;
      w0 = __builtin_amdgcn_mfma_f32_16x16x4f32(p[0], A.bwp[0], w0, 0, 0, 0);
      w1 = __builtin_amdgcn_mfma_f32_16x16x4f32(p[1], A.bwp[1], w1, 0, 0, 0);
      w2 = __builtin_amdgcn_mfma_f32_16x16x4f32(p[2], A.bwp[2], w2, 0, 0, 0);
      w3 = __builtin_amdgcn_mfma_f32_16x16x4f32(p[3], A.bwp[3], w3, 0, 0, 0);
      // lane (hi, col) holds w of item columns 4 hi + i, slot col; lanes
      // without a live (item, coefficient) store to the junk slots
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int it = ig * 32 + 16 * hs + 4 * hi + i;
        const bool ok = col < 2 * S && it < items;
        sw[ok ? (it % GS) * SWR + (it / GS) * S + jo : GS * SWR + lane] = (w0[i] + w1[i]) + (w2[i] + w3[i]);
      }
    }
  }
  l_lane = l_lane * a_lane + lsum;
  return true;
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


// ---------------------------------------------------------------- phases --
template <int D, int GS, int KF, int VF>
struct Acc {
  using C = Cfg<D, GS, KF, VF>;
  float v[C::VM ? 1 : GS][C::VM ? 1 : C::EV];     // VALU value path: [head][lane's EV columns]
  float m[C::VM ? C::MB : 1][C::VM ? C::NBV : 1];  // MFMA value path: head 4*mb + lane/16, column 16*nb + lane%16
};

template <int D, int GS>
struct Query {
  h2 qh[GS][8];                          // VALU key path
  float cq[GS];
  uint4 qB[D / 64][cdiv(GS, 4)];         // MFMA key path
  float cqq[cdiv(GS, 4)];
};

// Per-wave LDS: scores / weights (head-major) and junk slots for masked
// stores, the tile's V row scales, and the int8 value tile of the MFMA path.
template <int D, int GS, int KF, int VF>
struct WaveLds {
  using C = Cfg<D, GS, KF, VF>;
  static constexpr int SW_BYTES = C::SWR * GS * 4 + 64 * 4;
  static constexpr int SC_BYTES = 64 * 4;
  static constexpr int VT_BYTES = C::VM ? C::SWR * C::RBV : 0;
  static constexpr int BYTES = SW_BYTES + SC_BYTES + VT_BYTES;
  float *sw;
  float *svs;
  char *vl;
  __device__ __forceinline__ WaveLds(char *base) {
    sw = reinterpret_cast<float *>(base);
    svs = reinterpret_cast<float *>(base + SW_BYTES);
    vl = base + SW_BYTES + SC_BYTES;
  }
};

template <int D, int GS, int SP, int KF, int VF>
__device__ __forceinline__ void process_k(const TileBuf<D, GS, KF, VF> &B, int nrows, int lane, Query<D, GS> &Q,
                                          const WaveLds<D, GS, KF, VF> &L) {
  using C = Cfg<D, GS, KF, VF>;
  if constexpr (C::KM) {
    kcompute_mfma<D, GS, C::SWR, KF, VF>(B.k, lane, Q.qB, Q.cqq, L.sw);
  } else {
    kcompute<D, GS, C::SWR, KF, C::KSTEPS, C::KQ>(B.k.k, nrows, lane, Q.qh, Q.cq, L.sw);
  }
  wave_lds_sync();
}

template <int D, int GS, int SP, int KF, int VF>
__device__ __forceinline__ void process_lv(const TileBuf<D, GS, KF, VF> &B, int nrows, int S, int R, int lane,
                                           const Basis<SP> &bas, const WaveLds<D, GS, KF, VF> &L, float (&m_u)[GS],
                                           float &m_lane, float &l_lane, Acc<D, GS, KF, VF> &acc) {
  using C = Cfg<D, GS, KF, VF>;
  float alpha[GS];
  // groups of 16 (block, head) items in a tile, bounded by the fewest kept
  // rows a padded keep count SP allows: SP / 2 + 1, and 2 for SP = 2 (a
  // tile with S = 1 has more groups and takes logits_any)
  constexpr int kSmin = SP == 2 ? 2 : SP / 2 + 1;
  constexpr int NG = cmax(1, cdiv((C::TR / kSmin) * GS, 16));
  bool done = false;
  // eight-head groups pack only with int8 keys and values: other row formats
  // leave no registers for it (their tile loops would reach scratch)
  if constexpr (SP == 2 && (GS <= 4 || (KF == I8 && VF == I8)))
    done = logits_packed<GS, C::SWR, cdiv(NG, 2)>(bas, L.sw, nrows / S, R, S, lane, m_u, m_lane, l_lane, alpha);
  if (!done) logits<GS, SP, C::SWR, NG>(bas, L.sw, nrows / S, R, S, lane, m_u, m_lane, l_lane, alpha);
  if constexpr (C::VM)
    rescale_mfma<GS>(acc.m, alpha, lane);
  else
    rescale(acc.v, alpha);
  wave_lds_sync();
  if constexpr (C::VM)
    vcompute_mfma<D, GS, C::SWR, KF, VF>(B.v, nrows, lane, L.sw, L.vl, L.svs, acc.m);
  else
    vcompute<D, GS, C::SWR, VF, C::VSTEPS, C::VDW, C::EV>(B.v.v, nrows, lane, L.sw, acc.v);
  wave_lds_sync();
}

// The raw tail (< R tokens of bf16 / fp32) in one wave, one load step at a
// time so it needs few registers.  Every token is a block with R = S = 1.
// acc (VALU layout) is rescaled here; alpha is returned for other
// accumulators of the same heads.
// A fused new token (t_new >= 0) is tail row t_new: its key and value rows
// are read from kn / vn (rows past the old tail read zeros from the tail,
// every other row reads zeros from the new token), and with store_new the
// lanes holding it also write it to tail slot t_new.
// issue() requests the first chunk of rows (and the new token) and returns;
// compute() waits for them, so the caller can request other data in between.
template <int D, int GS, int SP, int SWR, int RAWK, int RAWV, int EV>
struct TailPass {
  static constexpr int LK = D / 16, RK = 64 / LK, EBK = ebytes(RAWK), EBV = ebytes(RAWV);
  static constexpr int LV = D / EV, RV = 64 / LV, VDW = EV * EBV / 4;
  static_assert(kMaxR % RV == 0 && kMaxR % RK == 0, "tail steps must tile the tail rows");
  // Up to PK key and PV value load steps (about 16 registers of data each,
  // 8 with eight heads per group) are requested together (rows past the tail
  // read zeros), so the first chunk of both costs one round trip.
  static constexpr int BUDGET = GS >= 8 ? 8 : 16;
  static constexpr int PK = cmin(kMaxR / RK, cmax(1, BUDGET / (4 * EBK))), PV = cmin(kMaxR / RV, cmax(1, BUDGET / VDW));
  static constexpr uint32_t kOut = kOutOfRange;
  // 16-byte loads per row step: EBK for a key row's 16 columns, NVL for a
  // value row's EV columns
  static constexpr int NVL = VDW % 4 == 0 ? VDW / 4 : 1;
  const void *kt, *vt;
  int nt, t_new, rrk, ck, rrv, cv, dm;
  rsrc_t rk, rv;
  // per load: the lane's offset, or kOut for columns at or past dm
  uint32_t offk[EBK], offv[NVL];
  // The new token's rows, held by the lanes whose row in a step it is
  // (zeros in every other lane), merged into its step's registers below.
  uint4 knw[EBK];
  uint32_t vnw[VDW];
  uint4 kb[PK][EBK];
  uint32_t vb[PV][VDW];

  __device__ __forceinline__ void load_k(int r00) {
#pragma unroll
    for (int s = 0; s < PK; ++s)
#pragma unroll
      for (int k = 0; k < EBK; ++k) kb[s][k] = bload128(rk, offk[k], (r00 + s * RK) * dm * EBK);
  }
  __device__ __forceinline__ void load_v(int r00) {
#pragma unroll
    for (int s = 0; s < PV; ++s) {
      if constexpr (VDW % 4 == 0) {
#pragma unroll
        for (int k = 0; k < VDW / 4; ++k) {
          const uint4 t = bload128(rv, offv[k], (r00 + s * RV) * dm * EBV);
          vb[s][4 * k] = t.x; vb[s][4 * k + 1] = t.y; vb[s][4 * k + 2] = t.z; vb[s][4 * k + 3] = t.w;
        }
      } else if constexpr (VDW == 2) {
        const uint2 t = bload64(rv, offv[0], (r00 + s * RV) * dm * EBV);
        vb[s][0] = t.x; vb[s][1] = t.y;
      } else {
        static_assert(VDW == 1, "value words per lane: 1, 2 or a multiple of 4");
        vb[s][0] = __builtin_bit_cast(uint32_t, bloadf(rv, offv[0], (r00 + s * RV) * dm * EBV));
      }
    }
  }
  // OR the new token into the step that holds its row (its lanes read zeros
  // from the slab).  Every step takes an OR with the token or with zero, so
  // no step is picked by a computed index (which would put the rows in
  // scratch memory).
  __device__ __forceinline__ void merge_k(int r00) {
#pragma unroll
    for (int s = 0; s < PK; ++s) {
      const bool hit = t_new >= r00 + s * RK && t_new < r00 + (s + 1) * RK;
#pragma unroll
      for (int k = 0; k < EBK; ++k)
        kb[s][k] = make_uint4(kb[s][k].x | (hit ? knw[k].x : 0u), kb[s][k].y | (hit ? knw[k].y : 0u),
                              kb[s][k].z | (hit ? knw[k].z : 0u), kb[s][k].w | (hit ? knw[k].w : 0u));
    }
  }
  __device__ __forceinline__ void merge_v(int r00) {
#pragma unroll
    for (int s = 0; s < PV; ++s) {
      const bool hit = t_new >= r00 + s * RV && t_new < r00 + (s + 1) * RV;
#pragma unroll
      for (int k = 0; k < VDW; ++k) vb[s][k] |= hit ? vnw[k] : 0u;
    }
  }

  __device__ __forceinline__ void issue(const void *kt_, const void *vt_, int nt_, const void *kn, const void *vn,
                                        int t_new_, int dm_, int lane) {
    kt = kt_;
    vt = vt_;
    nt = nt_;
    t_new = t_new_;
    dm = dm_;
    const int t_old = t_new >= 0 ? t_new : nt;   // rows held by the tail slab
    rk = make_rsrc(kt, (uint32_t)t_old * dm * EBK);
    rv = make_rsrc(vt, (uint32_t)t_old * dm * EBV);
    rrk = lane / LK;
    ck = lane % LK;
    rrv = lane / LV;
    cv = lane % LV;
#pragma unroll
    for (int k = 0; k < EBK; ++k)
      offk[k] = ck * 16 + k * (16 / EBK) < dm ? (uint32_t)(rrk * dm + ck * 16) * EBK + 16 * k : kOut;
#pragma unroll
    for (int k = 0; k < NVL; ++k)
      offv[k] = cv * EV + k * (16 / EBV) < dm ? (uint32_t)(rrv * dm + cv * EV) * EBV + 16 * k : kOut;
    {
      // the new token's range ends at its dm columns: columns past it read zeros
      const rsrc_t rkn = make_rsrc(kn, t_new >= 0 ? (uint32_t)(dm * EBK) : 0u);
      const rsrc_t rvn = make_rsrc(vn, t_new >= 0 ? (uint32_t)(dm * EBV) : 0u);
      const uint32_t onk = t_new >= 0 && rrk == t_new % RK ? (uint32_t)(ck * 16) * EBK : kOut;
      const uint32_t onv = t_new >= 0 && rrv == t_new % RV ? (uint32_t)(cv * EV) * EBV : kOut;
#pragma unroll
      for (int k = 0; k < EBK; ++k) knw[k] = bload128(rkn, onk + 16 * k, 0);
      if constexpr (VDW % 4 == 0) {
#pragma unroll
        for (int k = 0; k < VDW / 4; ++k) {
          const uint4 t = bload128(rvn, onv + 16 * k, 0);
          vnw[4 * k] = t.x; vnw[4 * k + 1] = t.y; vnw[4 * k + 2] = t.z; vnw[4 * k + 3] = t.w;
        }
      } else if constexpr (VDW == 2) {
        const uint2 t = bload64(rvn, onv, 0);
        vnw[0] = t.x; vnw[1] = t.y;
      } else {
        vnw[0] = __builtin_bit_cast(uint32_t, bloadf(rvn, onv, 0));
      }
    }
    load_k(0);
    load_v(0);
  }

  template <typename Prep>
  __device__ __forceinline__ void compute(bool store_new, int lane, h2 (&qh)[GS][8], const float (&cq)[GS], float *sw,
                                          float (&m_u)[GS], float &m_lane, float &l_lane, float (&acc)[GS][EV],
                                          float (&alpha)[GS], Prep &&prep) {
    merge_k(0);
    // the new token's rows into tail slot t_new (the lanes that hold it;
    // columns below dm only)
    if (store_new) {
      if (rrk == t_new % RK) {
#pragma unroll
        for (int k = 0; k < EBK; ++k)
          if (ck * 16 + k * (16 / EBK) < dm)
            *reinterpret_cast<uint4 *>(static_cast<char *>(const_cast<void *>(kt)) +
                                       (size_t)(t_new * dm + ck * 16) * EBK + 16 * k) = knw[k];
      }
      if (rrv == t_new % RV) {
        uint32_t *dst = reinterpret_cast<uint32_t *>(static_cast<char *>(const_cast<void *>(vt)) +
                                                     (size_t)(t_new * dm + cv * EV) * EBV);
#pragma unroll
        for (int k = 0; k < VDW; ++k)
          if (cv * EV + (4 * (k / 4)) * (4 / EBV) < dm) dst[k] = vnw[k];
      }
    }
    prep();   // the query in the VALU layout, its loads issued before the tail's
    kcompute<D, GS, SWR, RAWK, PK, EBK>(kb, nt, lane, qh, cq, sw, 0);
    for (int r00 = PK * RK; r00 < nt; r00 += PK * RK) {
      load_k(r00);
      merge_k(r00);
      kcompute<D, GS, SWR, RAWK, PK, EBK>(kb, nt, lane, qh, cq, sw, r00);
    }
    wave_lds_sync();
    Basis<SP> unit;
    unit.unit(lane);
    logits_any<GS, SP, SWR>(unit, sw, nt, 1, 1, lane, m_u, m_lane, l_lane, alpha);
    rescale(acc, alpha);
    wave_lds_sync();
    merge_v(0);
    vcompute<D, GS, SWR, RAWV, PV, VDW, EV>(vb, nt, lane, sw, acc, 0);
    for (int r00 = PV * RV; r00 < nt; r00 += PV * RV) {
      load_v(r00);
      merge_v(r00);
      vcompute<D, GS, SWR, RAWV, PV, VDW, EV>(vb, nt, lane, sw, acc, r00);
    }
    wave_lds_sync();
  }
};

template <int D, int GS, int SP, int SWR, int RAWK, int RAWV, int EV, typename Prep>
__device__ __forceinline__ void tail_pass(const void *kt, const void *vt, int nt, const void *kn, const void *vn,
                                          int t_new, int dm, bool store_new, int lane, h2 (&qh)[GS][8],
                                          const float (&cq)[GS], float *sw, float (&m_u)[GS], float &m_lane,
                                          float &l_lane, float (&acc)[GS][EV], float (&alpha)[GS], Prep &&prep) {
  TailPass<D, GS, SP, SWR, RAWK, RAWV, EV> tp;
  tp.issue(kt, vt, nt, kn, vn, t_new, dm, lane);
  tp.compute(store_new, lane, qh, cq, sw, m_u, m_lane, l_lane, acc, alpha, prep);
}

// The first tiles' addresses come as separate leading arguments (row counts
// in 32 bits) so that they can be preloaded into scalar registers at wave
// launch; everything else is in `a`.
//
// FULL: the rows' head_dim a.Dm equals the compute width D (the row pitch is
// a constant and no column needs masking); otherwise a.Dm < D, a multiple of 8.
template <int D, int GS, int SP, int KF, int VF, bool FULL>
__global__ __launch_bounds__(64 * kDecodeWaves) void decode_kernel(const char *krows, const char *vrows,
                                                                   const float *kscales, const float *vscales,
                                                                   int32_t k_bh_rows, int32_t v_bh_rows,
                                                                   int32_t chunk_rows, int32_t n_rows,
                                                                   int32_t tile_rows, DecodeArgs a) {
  using C = Cfg<D, GS, KF, VF>;
  using WL = WaveLds<D, GS, KF, VF>;
  constexpr int W = C::W, EV = C::EV, SWR = C::SWR, NT = 64 * W;
  static_assert(C::TR <= 64, "one scale per lane and tile");
  static_assert(C::TR <= SWR && C::KSTEPS * C::RK <= SWR && C::VSTEPS * C::RV <= SWR, "tile exceeds scratch");
  static_assert(!C::KM || C::RG * 16 <= SWR, "key MFMA rows exceed scratch");
  static_assert(!C::VM || (C::CH * 32 == SWR && C::VQ * 1024 <= SWR * C::RBV), "value tile exceeds scratch");
  constexpr int MERGE_BYTES = (W * GS * D + W * GS * 2) * 4;
  constexpr int COMBINE_BYTES = (4 * NT + kMaxSplits * GS + GS) * 4;
  constexpr int LDS_BYTES = cmax(W * WL::BYTES, cmax(MERGE_BYTES, COMBINE_BYTES));
  __shared__ __attribute__((aligned(16))) char lds_raw[LDS_BYTES];
  __shared__ __attribute__((aligned(16))) float sA[kMaxR * SP];
  __shared__ int last_flag;
  static_assert(GS <= 8, "one tail max per head");
  __shared__ float tail_m[8];   // the tail wave's running max per head right after the tail (MFMA value path)
  float *lds = reinterpret_cast<float *>(lds_raw);

  // Measurement builds only: the 100 MHz clock at the end of each phase,
  // 0 start, 1 query converted, 2 raw tail done, 3 tile loop done, 4 waves
  // merged, 5 partial published, 6 arrival counted, 7 output written.
  unsigned long long tl[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  auto stamp = [&](int i) {
    if constexpr (kTimeline) tl[i] = __builtin_amdgcn_s_memrealtime();
  };
  stamp(0);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: tile addresses live in SGPRs
  auto tl_store = [&]() {
#ifdef CDATTN_TIMELINE
    const int64_t wg = blockIdx.x + (int64_t)gridDim.x * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
    const int64_t w0 = (wg * W + wave) * 8;
    if (lane == 0 && a.timeline != nullptr && w0 + 8 <= a.timeline_words) {
#pragma unroll
      for (int i = 0; i < 8; ++i) a.timeline[w0 + i] = tl[i];
    }
#endif
  };
  // grid: x = split, y = query group, z = batch row * kv heads + kv head
  const int split = blockIdx.x;
  const int qg = blockIdx.y;
  const int64_t bh = blockIdx.z;
  const int h = (int)(blockIdx.z % (unsigned)a.H);
  const int b = (int)(blockIdx.z / (unsigned)a.H);
  const int64_t pairq = bh * a.NQG + qg;
  const int hq0 = h * a.G + qg * GS;
  // query heads of this group: GS, or fewer in the last group when GS does
  // not divide the kv head's G query heads (the others are computed on head
  // 0's query and never stored)
  const int gv = a.G - qg * GS < GS ? a.G - qg * GS : GS;
  const int R = a.R, S = a.S;
  const int dm = FULL ? D : a.Dm;   // head_dim in memory (D is the compute width)

  const WL L(lds_raw + wave * WL::BYTES);
  Basis<SP> bas;
  Query<D, GS> Q;
  Acc<D, GS, KF, VF> acc;
  float m_u[GS];
#pragma unroll
  for (int g = 0; g < GS; ++g) m_u[g] = -INFINITY;
  if constexpr (C::VM) {
#pragma unroll
    for (int i = 0; i < C::MB; ++i)
#pragma unroll
      for (int j = 0; j < C::NBV; ++j) acc.m[i][j] = 0.0f;
  } else {
#pragma unroll
    for (int g = 0; g < GS; ++g)
#pragma unroll
      for (int e = 0; e < EV; ++e) acc.v[g][e] = 0.0f;
  }
  float m_lane = -INFINITY, l_lane = 0.0f;   // running max and sum of this lane's head, (lane % 16) % GS

  // ---- this wave's tiles: t = wave, wave + W, ... of the split; a tile is
  // tile_rows = (TR / S) * S rows (whole blocks), a split chunk_rows rows.
  // With a raw tail and several splits the ranges shift by one tile: the
  // first split (dispatched first) takes one tile more and the last split,
  // whose wave with the fewest tiles runs the tail, one tile fewer.
  const int64_t shift = (a.n_tail + a.fuse_new > 0 && a.ns > 1) ? tile_rows : 0;
  const int64_t r0s = split == 0 ? 0 : (int64_t)split * chunk_rows + shift;
  const int64_t r1e = (int64_t)(split + 1) * chunk_rows + shift;
  const int64_t r1s = r1e < n_rows ? r1e : n_rows;
  const int nrs = r1s > r0s ? (int)(r1s - r0s) : 0;
  const int ntiles = (nrs + tile_rows - 1) / tile_rows;
  // The split's first rows (tile t of the split starts t * tile_rows rows
  // later), computed once so that few uniform values stay live in the loop.
  // Tiles past the split's end are empty (zero rows): their loads are out of
  // range and return zeros without touching memory, so every buffer is
  // re-requested unconditionally and the number of loads in flight is the
  // same on every path (the compiler's wait counts stay exact).
  const int64_t k0 = bh * k_bh_rows + r0s, v0 = bh * v_bh_rows + r0s;
  const char *kw = krows + k0 * dm * C::EBK;
  const char *vw = vrows + v0 * dm * C::EBV;
  const float *ksw = KF == I8 ? kscales + k0 : nullptr;
  const float *vsw = VF == I8 ? vscales + v0 : nullptr;
  const int kstep = tile_rows * dm * C::EBK, vstep = tile_rows * dm * C::EBV;   // bytes per tile
  auto tile_ref = [&](int t) {
    TileRef T;
    const int row0 = t * tile_rows;   // within the split
    const int left = nrs - row0;
    T.k = kw + (int64_t)t * kstep;
    T.v = vw + (int64_t)t * vstep;
    T.ks = KF == I8 ? ksw + row0 : nullptr;
    T.vs = VF == I8 ? vsw + row0 : nullptr;
    T.nrows = left < 0 ? 0 : (left < tile_rows ? left : tile_rows);
    T.dm = dm;
    return T;
  };

  // The synthesis basis from the table: A[r][j] = M[j][r] (the values the
  // encoder and the view use), or PNG mode's cumulative sum [j <= r], entry
  // r * SP + j of the workgroup's copy sA.  Only the threads that own an
  // entry inside the R x S matrix read the table (a few cache lines, once per
  // workgroup: every thread, or every lane reading its own operand entries,
  // would queue many more requests on those lines at launch), and they do it
  // before any other load (loads return in order).
  constexpr int NAU = (kMaxR * SP + NT - 1) / NT;
  float a_pre[NAU];
#pragma unroll
  for (int u = 0; u < NAU; ++u) {
    const int i = tid + u * NT, r = i / SP, j = i % SP;
    a_pre[u] = r < R && j < S ? synthesis_entry(a.png, R, r, j) : 0.0f;
  }
  // Tiles stream through NBUF register buffers per wave.  The query loads
  // are issued before the first tile's, and the set-up work (basis, query
  // conversion) runs while the tile is in flight.
  using QR = typename std::conditional<C::KM, QRegMfma<D, GS, FULL>, QRegValu<D, GS, FULL>>::type;
  QR qr;
  qr.load(a, b, hq0, gv, lane);
  // NBUF register buffers per wave: the first NBUF tiles are requested at once
  TileBuf<D, GS, KF, VF> bufs[C::NBUF];
#pragma unroll
  for (int i = 0; i < C::NBUF; ++i) issue(bufs[i], tile_ref(wave + i * W), lane);
  // weights of rows past a tile's end multiply zero data: keep them finite
  for (int i = lane; i < SWR * GS; i += 64) L.sw[i] = 0.0f;
  // bf16 value rows past the staged tile meet zero weights: keep them zero (not NaN)
  if constexpr (C::VM && VF == BF16)
    for (int i = lane; i < SWR * C::RBV / 16; i += 64) reinterpret_cast<uint4 *>(L.vl)[i] = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int u = 0; u < NAU; ++u)
    if (tid + u * NT < kMaxR * SP) sA[tid + u * NT] = a_pre[u];
  __syncthreads();
  bas.load(sA, R, S, lane);
  if constexpr (C::KM)
    qr.convert(a, lane, Q.qB, Q.cqq);
  else
    qr.convert(a, lane, Q.qh, Q.cq);
  stamp(1);
  // ---- the raw tail: one wave of the last split (the one with the fewest
  // tiles; with the shifted ranges the split has a tile fewer), on the VALU
  // paths, before that wave's tiles (its first tiles are already requested):
  // the wave with a tile fewer spends the difference on the tail while the
  // others stream.  The tail's softmax state and sums are where the tiles'
  // online softmax starts.
  const bool tail_wave = a.n_tail + a.fuse_new > 0 && split == a.ns - 1 && wave == ntiles % W;
  // tail accumulator beside the MFMA layout: ET columns per lane, few registers
  constexpr int ET = C::VM ? cmax(D / 64, 16 / GS) : 1, LT = D / ET;
  float acct[C::VM ? GS : 1][ET];
#pragma unroll
  for (int g = 0; g < (C::VM ? GS : 1); ++g)
#pragma unroll
    for (int e = 0; e < ET; ++e) acct[g][e] = 0.0f;
  auto run_tail = [&]() {
    // MFMA key path: the VALU-layout query is loaded here and converted once
    // the tail's own loads are in flight
    QRegValu<D, GS, FULL> qv;
    if constexpr (C::KM) qv.load(a, b, hq0, gv, lane);
    auto prep = [&]() {
      if constexpr (C::KM) qv.convert(a, lane, Q.qh, Q.cq);
    };
    const int nt = a.n_tail + a.fuse_new;
    const int ebk = a.kraw == BF16 ? 2 : 4, ebv = a.vraw == BF16 ? 2 : 4;
    const char *kt = static_cast<const char *>(a.ktail) + bh * (int64_t)R * dm * ebk;
    const char *vt = static_cast<const char *>(a.vtail) + bh * (int64_t)R * dm * ebv;
    // a fused new token: row n_tail of the tail, stored to its slot by query group 0
    const int t_new = a.fuse_new ? a.n_tail : -1;
    const bool store_new = a.fuse_new && qg == 0;
    const char *kn = a.fuse_new ? static_cast<const char *>(a.knew) + (b * a.kn_sb + (int64_t)h * a.kn_sh) * ebk : kt;
    const char *vn = a.fuse_new ? static_cast<const char *>(a.vnew) + (b * a.vn_sb + (int64_t)h * a.vn_sh) * ebv : vt;
    float alpha[GS];
    auto run = [&](auto &tacc) {
      constexpr int E = sizeof(tacc[0]) / sizeof(float);
      if (a.kraw == BF16 && a.vraw == BF16)
        tail_pass<D, GS, SP, SWR, BF16, BF16, E>(kt, vt, nt, kn, vn, t_new, dm, store_new, lane, Q.qh, Q.cq, L.sw, m_u,
                                                 m_lane, l_lane, tacc, alpha, prep);
      else if (a.kraw == F32 && a.vraw == F32)
        tail_pass<D, GS, SP, SWR, F32, F32, E>(kt, vt, nt, kn, vn, t_new, dm, store_new, lane, Q.qh, Q.cq, L.sw, m_u,
                                               m_lane, l_lane, tacc, alpha, prep);
      else if (a.kraw == BF16)
        tail_pass<D, GS, SP, SWR, BF16, F32, E>(kt, vt, nt, kn, vn, t_new, dm, store_new, lane, Q.qh, Q.cq, L.sw, m_u,
                                                m_lane, l_lane, tacc, alpha, prep);
      else
        tail_pass<D, GS, SP, SWR, F32, BF16, E>(kt, vt, nt, kn, vn, t_new, dm, store_new, lane, Q.qh, Q.cq, L.sw, m_u,
                                                m_lane, l_lane, tacc, alpha, prep);
    };
    if constexpr (C::VM) {
      // the tail's sums stay in acct, beside the MFMA layout, which the
      // tiles' rescales do not reach: the running max here is kept, and the
      // merge scales acct by exp2(max here - final max)
      run(acct);
      rescale_mfma<GS>(acc.m, alpha, lane);
      if (lane == 0) {
#pragma unroll
        for (int g = 0; g < GS; ++g) tail_m[g] = m_u[g];
      }
    } else {
      run(acc.v);
    }
  };
  // Eight-head groups, head_dim 256 and 32 kept rows hold more registers
  // than the tail pass can find beside a requested tile (it would spill, and
  // each reload is a round trip while the other waves stream): there the
  // tail runs after the wave's tiles (the tail wave has the fewest),
  // elsewhere before them.
  constexpr bool kTailAfter = GS >= 8 || D >= 256 || SP >= 32;
  if constexpr (!kTailAfter) {
    if (tail_wave) run_tail();
    stamp(2);
  }
  for (int t0 = wave; t0 < ntiles; t0 += C::NBUF * W) {
#pragma unroll
    for (int i = 0; i < C::NBUF; ++i) {
      // the buffer's next tile: K rows requested once the K phase is done,
      // V rows once the V phase is done
      const int t = t0 + i * W;
      const int tn = t + C::NBUF * W;
      const int n0 = tile_ref(t).nrows;
      if (n0 > 0) process_k<D, GS, SP, KF, VF>(bufs[i], n0, lane, Q, L);
      issue_k(bufs[i], tile_ref(tn), lane);
      __builtin_amdgcn_sched_barrier(0);
      if (n0 > 0) process_lv<D, GS, SP, KF, VF>(bufs[i], n0, S, R, lane, bas, L, m_u, m_lane, l_lane, acc);
      issue_v(bufs[i], tile_ref(tn), lane);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  stamp(3);
  if constexpr (kTailAfter) {
    if (tail_wave) run_tail();
    stamp(2);
  }
  // ---- wave totals: l over the lanes of a head, acc over the rows of a step
  float l_u[GS];
  {
    const float lt = strided<GS, false>(l_lane);
#pragma unroll
    for (int g = 0; g < GS; ++g) l_u[g] = readlane(lt, g);
  }
  if constexpr (!C::VM) {
#pragma unroll
    for (int g = 0; g < GS; ++g)
#pragma unroll
      for (int e = 0; e < EV; ++e) acc.v[g][e] = strided<C::LV, false>(acc.v[g][e]);
  } else if (tail_wave) {
#pragma unroll
    for (int g = 0; g < GS; ++g)
#pragma unroll
      for (int e = 0; e < ET; ++e) acct[g][e] = strided<LT, false>(acct[g][e]);
  }

  // ---- merge the waves in LDS, in a fixed order (the result does not
  // depend on timing): each wave's raw accumulator and (max, sum) per head.
  __syncthreads();   // all waves done with their scratch
  float *macc = lds;                    // [W][GS][D]
  float *mml = lds + W * GS * D;        // [W][GS][2]
  if constexpr (C::VM) {
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
      const int g = 4 * mb + lane / 16;
      if (g < GS) {
#pragma unroll
        for (int nb = 0; nb < C::NBV; ++nb) macc[(wave * GS + g) * D + 16 * nb + lane % 16] = acc.m[mb][nb];
      }
    }
    if (tail_wave) {
      wave_lds_sync();
      if (lane < LT) {
#pragma unroll
        for (int g = 0; g < GS; ++g) {
          const float f = __builtin_amdgcn_exp2f(tail_m[g] - m_u[g]);   // the tiles' rescales since the tail
#pragma unroll
          for (int e = 0; e < ET; ++e) macc[(wave * GS + g) * D + lane * ET + e] += acct[g][e] * f;
        }
      }
    }
  } else {
    if (lane < C::LV) {
#pragma unroll
      for (int g = 0; g < GS; ++g)
#pragma unroll
        for (int e = 0; e < EV; ++e) macc[(wave * GS + g) * D + lane * EV + e] = acc.v[g][e];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < GS; ++g) {
      mml[(wave * GS + g) * 2] = m_u[g];
      mml[(wave * GS + g) * 2 + 1] = l_u[g];
    }
  }
  __syncthreads();
  stamp(4);
  // workgroup (max, sum, acc) of head g at column d
  auto wg_partial = [&](int g, int d, float &m, float &l, float &sacc) {
    m = -INFINITY;
    for (int w = 0; w < W; ++w) m = fmaxf(m, mml[(w * GS + g) * 2]);
    l = 0.0f;
    sacc = 0.0f;
    for (int w = 0; w < W; ++w) {
      const float lw = mml[(w * GS + g) * 2 + 1];
      if (lw > 0.0f) {
        const float f = __builtin_amdgcn_exp2f(mml[(w * GS + g) * 2] - m);
        l += lw * f;
        sacc += macc[(w * GS + g) * D + d] * f;
      }
    }
  };

  // columns at or past dm and heads at or past gv are padding: never stored
  auto store_out = [&](int g, int d, float o) {
    if (d >= dm || g >= gv) return;
    const int64_t off = b * a.o_sb + (int64_t)(hq0 + g) * a.o_sh + d;
    if (a.out_f32) {
      static_cast<float *>(a.out)[off] = o;
    } else {
      uint32_t u = __float_as_uint(o);
      u += 0x7FFFu + ((u >> 16) & 1u);
      static_cast<uint16_t *>(a.out)[off] = (uint16_t)(u >> 16);
    }
  };

  if (a.ns == 1) {
    // the only split of its (b, h, group): normalise and write directly
    for (int idx = tid; idx < GS * D; idx += NT) {
      float m, l, sacc;
      wg_partial(idx / D, idx % D, m, l, sacc);
      store_out(idx / D, idx % D, sacc / l);
    }
    stamp(7);
    tl_store();
    return;
  }

  // ---- the workgroup's partial, published with device-scope stores
  float *pacc = a.part_acc + (pairq * a.ns + split) * GS * D;
  float *pml = a.part_ml + (pairq * a.ns + split) * GS * 2;
  for (int idx = tid; idx < GS * D; idx += NT) {
    const int g = idx / D, d = idx % D;
    float m, l, sacc;
    wg_partial(g, d, m, l, sacc);
    __hip_atomic_store(pacc + idx, sacc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (d == 0) {
      __hip_atomic_store(pml + 2 * g, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(pml + 2 * g + 1, l, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // Device-scope stores are complete once this thread's memory counter
  // drains; only after every thread's have drained is the arrival counted.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  stamp(5);
  if (tid == 0) {
    const uint32_t old =
        __hip_atomic_fetch_add(a.counters + pairq * kCounterStride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_flag = (old == (uint32_t)(a.ns - 1)) ? 1 : 0;
  }
  __syncthreads();
  stamp(6);
  if (!last_flag) {
    tl_store();
    return;
  }

  // ---- last arrival: fold the ns partials of every (head, column).  Wave
  // g < GS turns head g's (max, sum) pairs into split weights exp2(m - M)
  // (zero for empty splits) and the total sum; every thread sums the weighted
  // partials of one float4 column over every NG-th split (its loads issued
  // before the weights are known), and the NG shares are added in a fixed
  // order.  Partials and pairs are read with system-scope (sc0 sc1) buffer
  // loads, coherent across the XCDs; out-of-range splits read zeros.
  constexpr int kSysScope = 1 | 16;
  constexpr int NC = GS * D / 4, NG = NT / NC, CP = 8, KS = kMaxSplits / 64;
  static_assert(NG >= 1 && NG * NC == NT, "float4 columns tile the workgroup");
  const int ns = a.ns;
  const rsrc_t racc = make_rsrc(a.part_acc + pairq * ns * GS * D, (uint32_t)ns * GS * D * 4);
  const rsrc_t rml = make_rsrc(a.part_ml + pairq * ns * GS * 2, (uint32_t)ns * GS * 2 * 4);
  float4 *red = reinterpret_cast<float4 *>(lds);   // [NG][NC] shares
  float *fw = lds + 4 * NT;                        // [kMaxSplits][GS] split weights
  float *ltot = fw + kMaxSplits * GS;              // [GS] total sums
  const int c = tid % NC, gi = tid / NC, g = c / (D / 4);
  const int gw = wave % GS;
  float2 ml[KS];
#pragma unroll
  for (int k = 0; k < KS; ++k)
    ml[k] = __builtin_bit_cast(
        float2, __builtin_amdgcn_raw_buffer_load_b64(rml, 8 * ((lane + 64 * k) * GS + gw), 0, kSysScope));
  auto load_round = [&](int s0, float4 (&p)[CP]) {
#pragma unroll
    for (int u = 0; u < CP; ++u)
      p[u] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                            racc, 4 * ((s0 + u * NG) * GS * D + 4 * c), 0, kSysScope));
  };
  float4 p[CP];
  load_round(gi, p);
  __builtin_amdgcn_sched_barrier(0);
  {
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < KS; ++k)
      if (ml[k].y > 0.0f) M = fmaxf(M, ml[k].x);
    M = group_red<64, true>(M);
    float Ls = 0.0f;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const float f = ml[k].y > 0.0f ? __builtin_amdgcn_exp2f(ml[k].x - M) : 0.0f;
      Ls = fmaf(ml[k].y, f, Ls);
      if (wave < GS && lane + 64 * k < ns) fw[(lane + 64 * k) * GS + gw] = f;
    }
    Ls = group_red<64, false>(Ls);
    if (wave < GS && lane == 0) ltot[gw] = Ls;
  }
  __syncthreads();
  float4 s4 = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s0 = gi;;) {
#pragma unroll
    for (int u = 0; u < CP; ++u) {
      const int sp = s0 + u * NG;
      const float f = sp < ns ? fw[sp * GS + g] : 0.0f;
      if (f != 0.0f) {
        s4.x = fmaf(f, p[u].x, s4.x);
        s4.y = fmaf(f, p[u].y, s4.y);
        s4.z = fmaf(f, p[u].z, s4.z);
        s4.w = fmaf(f, p[u].w, s4.w);
      }
    }
    s0 += CP * NG;
    if (s0 >= ns) break;
    load_round(s0, p);
  }
  red[gi * NC + c] = s4;
  __syncthreads();
  if (gi == 0) {
    float4 t = red[c];
    for (int j = 1; j < NG; ++j) {
      const float4 r = red[j * NC + c];
      t.x += r.x;
      t.y += r.y;
      t.z += r.z;
      t.w += r.w;
    }
    const float Lg = ltot[g];
    const int d0 = 4 * (c % (D / 4));
    store_out(g, d0, t.x / Lg);
    store_out(g, d0 + 1, t.y / Lg);
    store_out(g, d0 + 2, t.z / Lg);
    store_out(g, d0 + 3, t.w / Lg);
  }
  stamp(7);
  tl_store();
  if (tid == 0) __hip_atomic_store(a.counters + pairq * kCounterStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, int GS, int SP, int KF, int VF, bool FULL>
int launch_one(const DecodeArgs &a, int64_t n_wg, hipStream_t stream) {
  using C = Cfg<D, GS, KF, VF>;
  const unsigned gy = (unsigned)a.NQG;
  const int64_t gz = n_wg / ((int64_t)a.ns * gy);   // batch rows x kv heads
  const int64_t tile_rows = (int64_t)(C::TR / a.S) * a.S;
  const int64_t chunk_rows = a.chunk * a.S, n_rows = a.n_blocks * a.S;
  if (gz > 65535 || a.k_bh_rows > INT32_MAX || a.v_bh_rows > INT32_MAX || chunk_rows > INT32_MAX ||
      n_rows > INT32_MAX)
    return -1;
  hipLaunchKernelGGL((decode_kernel<D, GS, SP, KF, VF, FULL>), dim3((unsigned)a.ns, gy, (unsigned)gz),
                     dim3(64 * kDecodeWaves), 0, stream, static_cast<const char *>(a.krows),
                     static_cast<const char *>(a.vrows), a.kscales, a.vscales, (int32_t)a.k_bh_rows,
                     (int32_t)a.v_bh_rows, (int32_t)chunk_rows, (int32_t)n_rows, (int32_t)tile_rows, a);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// One kernel instance, picked at run time from (D, GS, SP): launched, or
// asked how many of its workgroups one CU holds at a time.
template <bool FULL>
struct LaunchOp {
  const DecodeArgs &a;
  int64_t n_wg;
  hipStream_t stream;
  template <int D, int GS, int SP, int KF, int VF>
  int run() const { return launch_one<D, GS, SP, KF, VF, FULL>(a, n_wg, stream); }
};

template <bool FULL>
struct ResidentOp {
  // workgroups of the instance resident on one CU of the current device
  // (its registers and LDS decide; -1 if the runtime cannot say)
  template <int D, int GS, int SP, int KF, int VF>
  int run() const {
    int n = 0;
    const hipError_t e =
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel<D, GS, SP, KF, VF, FULL>, 64 * kDecodeWaves, 0);
    return e == hipSuccess ? n : -1;
  }
};

template <int D, int GS, int KF, int VF, class Op>
int by_sp(int SP, const Op &op) {
  switch (SP) {
    case 2: return op.template run<D, GS, 2, KF, VF>();
    case 4: return op.template run<D, GS, 4, KF, VF>();
    case 8: return op.template run<D, GS, 8, KF, VF>();
    case 16: return op.template run<D, GS, 16, KF, VF>();
    case 32: return op.template run<D, GS, 32, KF, VF>();
    default: return -1;
  }
}

template <int D, int KF, int VF, class Op>
int by_gs(int GS, int SP, const Op &op) {
  switch (GS) {
    case 1: return by_sp<D, 1, KF, VF>(SP, op);
    case 2: return by_sp<D, 2, KF, VF>(SP, op);
    case 4: return by_sp<D, 4, KF, VF>(SP, op);
    case 8: return by_sp<D, 8, KF, VF>(SP, op);
    default: return -1;
  }
}

template <int KF, int VF, class Op>
int by_dim(int D, int GS, int SP, const Op &op) {
  switch (D) {
    case 64: return by_gs<64, KF, VF>(GS, SP, op);
    case 128: return by_gs<128, KF, VF>(GS, SP, op);
    case 256: return by_gs<256, KF, VF>(GS, SP, op);
    default: return -1;
  }
}

}  // namespace dec
}  // namespace cdattn
