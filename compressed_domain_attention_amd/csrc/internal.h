// Internal declarations shared by the host API and the kernel translation
// units of libcdattn.so.  Not part of the public ABI (include/cdattn.h).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

struct codec_stream;   // include/cdattn.h

namespace cdattn {

constexpr int kMaxR = 32;      // tokens per block
constexpr int kMaxS = 32;      // kept frequencies
constexpr int kMaxD = 256;     // head_dim (a multiple of 8)

// Compute width of the kernels for head_dim D: the next of 64, 128 and 256.
// Rows in memory keep their own pitch D; columns past D are read as zeros
// (or multiply zero query digits) and never written.
constexpr int pad_dim(int D) { return D <= 64 ? 64 : (D <= 128 ? 128 : 256); }
constexpr int kDecodeWaves = 8;   // waves per decode workgroup
constexpr int kEncodeWaves = 4;   // waves (one block each) per encode workgroup

enum Fmt : int32_t { F32 = 0, BF16 = 1, I8 = 2 };

// ---------------------------------------------------------------- encode --
// Where the R tokens of a block come from.  Token i of block n of (b, h):
//   i <  split_i : src0 + b*s0_b + h*s0_h + (n*R + i)*s0_t      (x or tail)
//   i >= split_i : src1 + b*s1_b + h*s1_h                        (new token)
struct EncodeArgs {
  const void *src0;
  int64_t s0_b, s0_h, s0_t;
  const void *src1;
  int64_t s1_b, s1_h;
  int32_t split_i;        // R for a plain run of tokens, R-1 for an append
  int32_t raw;            // Fmt of the source tokens (BF16 or F32)
  int32_t fmt;            // Fmt of the coefficient rows
  int32_t png;            // 1: PNG mode analysis (anchor and differences), else the DCT-II table
  int32_t R, S;
  int32_t D;              // head_dim: row pitch of tokens, rows and tail
  int64_t H;              // heads (b = bh / H)
  int64_t n_new;          // blocks to encode per (b, h)
  int64_t n0;             // first destination slot
  int64_t cap;            // archive capacity (blocks)
  void *rows;             // [B][H][cap][S][D]
  float *scales;          // [B][H][cap][S] (I8)
  // tail copy (encode_blocks only): tokens n_new*R .. n_new*R + n_copy - 1
  int32_t n_copy;
  void *tail;             // [B][H][R][D], raw dtype
};

// Append one token: tail slot t <- new token; if t + 1 == R the same launch
// encodes the block (tail slots 0..R-2 and the new token) into slot n.
struct AppendArgs {
  EncodeArgs e[2];        // [0] = keys, [1] = values; src0 = tail, src1 = new
  int32_t t;              // tail slot the new token goes to
  int32_t complete;       // 1 if this token completes a block
};

int launch_encode(const EncodeArgs &a, int64_t BH, hipStream_t stream);
int launch_append(const AppendArgs &a, int64_t BH, hipStream_t stream);

// ------------------------------------------------------ view, crop, gather --
// Decoded view: blocks blk0 .. blk0+nblk-1 of every (b, h); token i of block
// n goes to dst token (n - blk0)*R + i + o_t0 (i < tok_limit); then, if
// n_copy > 0, tail slots 0..n_copy-1 go to dst tokens nblk*R + o_t0 + i.
struct ViewArgs {
  const void *rows;       // [BH][cap][S][D] of rf
  const float *scales;    // [BH][cap][S] (I8)
  const void *tail;       // [BH][R][D] of raw
  int32_t rf, raw, out;   // row, tail and view formats
  int32_t png;            // 1: PNG mode synthesis (cumulative sum)
  int32_t R, S, D;
  int64_t H, BH, cap;
  int64_t blk0, nblk;
  int32_t tok_limit;
  int32_t n_copy;
  void *dst;
  int64_t o_sb, o_sh, o_st, o_t0;
};

constexpr int kGatherChunk = 256;   // destination batch rows per gather launch

// Batch gather of up to kGatherChunk destination rows i0 .. i0+n-1.
struct GatherArgs {
  const void *src_rows;
  void *dst_rows;
  int64_t slab_bytes, dst_slab_bytes, row_bytes;   // per (b, h): allocated, allocated, used
  const float *src_scales;                         // NULL unless I8
  float *dst_scales;
  int64_t scale_slab, dst_scale_slab, n_scales;    // floats
  const void *src_tail;
  void *dst_tail;
  int64_t tail_bytes;                              // all R slots
  int64_t H, i0;
  int32_t idx[kGatherChunk];                       // source batch row of destination row i0 + k
};

int launch_view(const ViewArgs &a, hipStream_t stream);
int launch_gather(const GatherArgs &g, int64_t n_units, hipStream_t stream);

// ---------------------------------------------------------------- decode --
struct DecodeArgs {
  // The first 64 bytes hold what the first tile requests need, the next 64
  // the shape and the query, so a workgroup starts on two scalar loads.
  const void *krows;
  const void *vrows;
  const float *kscales;
  const float *vscales;
  int64_t k_bh_rows;      // coefficient rows per (b, h) in the key archive
  int64_t v_bh_rows;
  int64_t n_blocks;
  int64_t chunk;          // blocks per split
  int32_t H, G, NQG;      // kv heads, group size, query groups per kv head
  int32_t R, S;
  int32_t n_tail;
  int32_t ns;             // splits per (b, h, query group)
  float qk_scale;         // softmax scale * log2(e)
  const uint16_t *q;      // bf16 (B, Hq, 1, D)
  int64_t q_sb, q_sh;
  int32_t kf, vf;         // row formats
  int32_t kraw, vraw;     // tail formats
  int32_t png;            // 1: PNG mode synthesis (cumulative sum), else the DCT-II basis
  int32_t Dm;             // head_dim: row pitch in memory (<= the kernel's compute width)
  // Fused append (fuse_new = 1): one new key / value token per (b, h) joins
  // the raw tail as slot n_tail (it does not complete a block); the tail
  // pass reads it from knew / vnew and query group 0 stores it to the slot.
  int32_t fuse_new;
  const void *ktail;
  const void *vtail;
  const void *knew;
  const void *vnew;
  int64_t kn_sb, kn_sh, vn_sb, vn_sh;
  void *out;
  int64_t o_sb, o_sh;
  int32_t out_f32;        // 1: fp32 out, 0: bf16 out
  uint32_t *counters;     // one per (b, h, query group), kCounterStride apart
  float *part_ml;         // [pairs][ns][GS][2]
  float *part_acc;        // [pairs][ns][GS][D]
#ifdef CDATTN_TIMELINE
  // Measurement builds only: per-wave phase stamps of each decode launch
  // (s_memrealtime) at word ((workgroup * waves + wave) * 8 + phase).
  unsigned long long *timeline;
  int64_t timeline_words;
#endif
};
static_assert(offsetof(DecodeArgs, H) == 64 && offsetof(DecodeArgs, q_sh) == 112, "kernel argument lines");

// Heads of one query group handled per workgroup, and padded kept rows.
int decode_group_size(int G);
int decode_pad_keep(int S);

constexpr int kMaxSplits = 256;   // splits per (b, kv head, query group)
constexpr int kCounterStride = 64; // uint32 slots between arrival counters (256 bytes)
// Decode workgroups that fill a device once, at most (the arrival-counter
// region of every workspace holds this many counters: 256 KiB).
constexpr int kMaxTargetWorkgroups = 1024;

// Coefficient rows per decode tile: about 8 KB of key plus value rows.  The
// MFMA value paths (int8 / bf16 rows) work in 32-row chunks, so a tile below
// 32 rows is raised to 32 when that stays within 12 KB (int8 keys with bf16
// values at head_dim 128: 21 -> 32 rows, measured 10 % faster).  Int8 keys
// with int8 or bf16 values at head_dim 64 take one 32-row chunk per tile
// instead of 64 or 42 rows: a larger tile holds up to 256 (block, head)
// logits at once and spilled registers inside the tile loop, and 42 rows left
// a second value chunk with 10 live rows (B 8, GQA 4, 4K context: int8 values
// 14.3 -> 11.5 us per decode, bf16 values 13.8 -> 12.2 us).
constexpr int decode_elem_bytes(int f) { return f == I8 ? 1 : (f == BF16 ? 2 : 4); }
constexpr int decode_tile_rows(int D, int kf, int vf) {
  const int rb = D * (decode_elem_bytes(kf) + decode_elem_bytes(vf));
  const int rows = D == 64 && kf == I8 && (vf == I8 || vf == BF16) ? 32 : 8192 / rb;
  return (vf == I8 || vf == BF16) && rows < 32 && 32 * rb <= 12288 ? 32 : rows;
}

// Decode kernel instances: compute width D (64, 128, 256), group size GS,
// padded kept rows SP, row formats kf / vf; `full` selects the instance for
// rows whose head_dim is D (else a.Dm < D).
int launch_decode(int D, int GS, int SP, int kf, int vf, bool full, const DecodeArgs &a, int64_t n_wg,
                  hipStream_t stream);
// Workgroups of a decode kernel instance that one CU of the current device
// holds at a time (-1 if unknown).
int resident_decode(int D, int GS, int SP, int kf, int vf, bool full);
// The device `stream` belongs to (the current device for the null stream).
int stream_device(hipStream_t stream, int *dev);

// Split plan of a decode: group size, query groups per kv head, padded kept
// rows, the workgroups that fill the device once, splits per (b, kv head,
// query group), blocks per split, workgroups, and the workspace layout
// (counters, then (max, sum) pairs, then partial accumulators).  A function
// of the shapes and of the device's CU count and the kernel's occupancy.
struct DecodePlan {
  bool ok;
  int GS, NQG, SP, ns;
  int64_t target, pairs, chunk, n_wg;
  size_t off_ml, off_acc, bytes;
};

// Validation of a decode call apart from its workspace; fills the plan for
// the device of `stream` (no launch; the first call per device and kernel
// instance asks the runtime for its CU count and the kernel's occupancy).
int decode_check_args(const void *q, const int64_t q_stride[2], int64_t Hq, const codec_stream *k,
                      const codec_stream *v, float scale, const void *out, const int64_t out_stride[2],
                      int32_t out_dtype, hipStream_t stream, DecodePlan *p);
// The decode launch for validated arguments and a workspace of p.bytes
// (fuse_k / fuse_v non-null: one new token joins the tail as slot n_tail).
int launch_decode_call(const void *q, const int64_t q_stride[2], int64_t Hq, const codec_stream *k,
                       const codec_stream *v, float scale, void *out, const int64_t out_stride[2],
                       int32_t out_dtype, void *workspace, const DecodePlan &p, const void *fuse_k,
                       const int64_t kn_stride[2], const void *fuse_v, const int64_t vn_stride[2],
                       hipStream_t stream);
#define CDATTN_DECL_DECODE(K, V)                                                                             \
  int launch_decode_##K##_##V(int D, int GS, int SP, const DecodeArgs &a, int64_t n_wg, hipStream_t stream); \
  int resident_decode_##K##_##V(int D, int GS, int SP);                                                      \
  int launch_decode_##K##_##V##_pad(int D, int GS, int SP, const DecodeArgs &a, int64_t n_wg,                \
                                    hipStream_t stream);                                                     \
  int resident_decode_##K##_##V##_pad(int D, int GS, int SP);
CDATTN_DECL_DECODE(i8, i8)
CDATTN_DECL_DECODE(i8, bf16)
CDATTN_DECL_DECODE(i8, f32)
CDATTN_DECL_DECODE(bf16, i8)
CDATTN_DECL_DECODE(bf16, bf16)
CDATTN_DECL_DECODE(bf16, f32)
CDATTN_DECL_DECODE(f32, i8)
CDATTN_DECL_DECODE(f32, bf16)
CDATTN_DECL_DECODE(f32, f32)
#undef CDATTN_DECL_DECODE

}  // namespace cdattn
