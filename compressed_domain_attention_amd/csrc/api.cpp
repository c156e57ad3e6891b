// Host side of the C ABI declared in include/cdattn.h: argument validation
// (always before any launch), the DCT basis, the split plan of the decode,
// and kernel launches.  No allocation and no synchronisation; the only state
// is the per-device, per-kernel split target the plan asks the runtime for
// once.

#include <math.h>
#include <string.h>

#include <array>
#include <map>
#include <mutex>

#include "basis.h"
#include "cdattn.h"
#include "internal.h"

using namespace cdattn;

namespace {

#ifdef CDATTN_TIMELINE
// Measurement builds only: where decode launches write their phase stamps.
unsigned long long *g_timeline = nullptr;
int64_t g_timeline_words = 0;
#endif

// The codec's basis table (see basis.h), host copy.
const float kBasisHost[kBasisEntries] = {
#include "cdattn_basis_table.inc"
};

bool fmt_ok(int f) { return f == CODEC_F32 || f == CODEC_BF16 || f == CODEC_I8 || f == CODEC_PNG; }
bool raw_ok(int f) { return f == CODEC_F32 || f == CODEC_BF16; }
int elem_bytes(int f) { return (f == CODEC_F32 || f == CODEC_PNG) ? 4 : (f == CODEC_BF16 ? 2 : 1); }
// Storage format of the rows as the kernels see it (PNG rows are fp32).
int row_fmt(int f) { return f == CODEC_PNG ? CODEC_F32 : f; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_stream(const codec_stream *s) {
  if (!s) return CODEC_ERR_NULL;
  if (s->block < 1 || s->block > CODEC_MAX_BLOCK) return CODEC_ERR_SHAPE;
  if (s->keep < 1 || s->keep > s->block || s->keep > CODEC_MAX_KEEP) return CODEC_ERR_SHAPE;
  if (s->head_dim < 1) return CODEC_ERR_SHAPE;
  if (s->head_dim > kMaxD || s->head_dim % 8 != 0) return CODEC_ERR_UNSUPPORTED;
  if (s->batch < 1 || s->heads < 1) return CODEC_ERR_SHAPE;
  if (s->batch * s->heads > (int64_t)1 << 31) return CODEC_ERR_SHAPE;
  if (!fmt_ok(s->fmt) || !raw_ok(s->raw_dtype)) return CODEC_ERR_FORMAT;
  if (s->fmt == CODEC_PNG && s->keep != s->block) return CODEC_ERR_SHAPE;   // anchor + R-1 deltas
  if (s->n_tail < 0 || s->n_tail >= s->block) return CODEC_ERR_STATE;
  if (s->n_blocks < 0) return CODEC_ERR_STATE;
  if (s->capacity < s->n_blocks) return CODEC_ERR_CAPACITY;
  if (!s->tail) return CODEC_ERR_NULL;
  if (s->capacity > 0 && !s->rows) return CODEC_ERR_NULL;
  if (s->capacity > 0 && s->fmt == CODEC_I8 && !s->scales) return CODEC_ERR_NULL;
  if (!aligned16(s->tail) || (s->rows && !aligned16(s->rows)) ||
      (s->fmt == CODEC_I8 && s->scales && !aligned16(s->scales)))
    return CODEC_ERR_SHAPE;
  return CODEC_OK;
}

bool same_geometry(const codec_stream *a, const codec_stream *b) {
  return a->block == b->block && a->keep == b->keep && a->head_dim == b->head_dim && a->batch == b->batch &&
         a->heads == b->heads && a->n_blocks == b->n_blocks && a->n_tail == b->n_tail;
}

EncodeArgs stream_encode_args(const codec_stream *s) {
  EncodeArgs e;
  memset(&e, 0, sizeof(e));
  e.raw = s->raw_dtype;
  e.fmt = row_fmt(s->fmt);
  e.png = s->fmt == CODEC_PNG ? 1 : 0;
  e.R = s->block;
  e.S = s->keep;
  e.D = s->head_dim;
  e.H = s->heads;
  e.n0 = s->n_blocks;
  e.cap = s->capacity;
  e.rows = s->rows;
  e.scales = s->scales;
  e.tail = s->tail;
  return e;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workgroups that fill a device once when the runtime cannot be asked (a
// host without a GPU): MI355X's 256 CUs with one 8-wave decode workgroup each.
constexpr int64_t kDefaultTargetWorkgroups = 256;

// Workgroups that fill device `dev` once with decode kernel instance (D, GS,
// SP, kf, vf): its CU count times the instance's workgroups resident per CU
// (the kernel's registers and LDS decide), at most kMaxTargetWorkgroups.
// Asked once per device and instance, then kept.
int64_t target_workgroups(int dev, int D, int GS, int SP, int kf, int vf, bool full) {
  static std::mutex mu;
  static std::map<std::array<int, 7>, int64_t> known;
  if (dev < 0) return kDefaultTargetWorkgroups;
  const std::array<int, 7> key{dev, D, GS, SP, kf, vf, full ? 1 : 0};
  std::lock_guard<std::mutex> lock(mu);
  const auto it = known.find(key);
  if (it != known.end()) return it->second;
  int64_t t = kDefaultTargetWorkgroups;
  int cus = 0, cur = -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0 &&
      hipGetDevice(&cur) == hipSuccess && (cur == dev || hipSetDevice(dev) == hipSuccess)) {
    const int per_cu = resident_decode(D, GS, SP, kf, vf, full);   // asks the current device
    if (cur != dev) (void)hipSetDevice(cur);
    if (per_cu > 0) t = (int64_t)cus * per_cu;
  }
  if (t > kMaxTargetWorkgroups) t = kMaxTargetWorkgroups;
  known[key] = t;
  return t;
}

DecodePlan make_plan(const codec_stream *k, const codec_stream *v, int64_t Hq, int dev) {
  DecodePlan p;
  const int64_t G = Hq / k->heads;
  p.GS = decode_group_size((int)G);
  p.NQG = (int)((G + p.GS - 1) / p.GS);
  p.SP = decode_pad_keep(k->keep);
  p.pairs = k->batch * k->heads * p.NQG;
  const int64_t n = k->n_blocks;
  const int DP = pad_dim(k->head_dim);   // compute width of the kernels
  const int64_t NB = decode_tile_rows(DP, row_fmt(k->fmt), row_fmt(v->fmt)) / k->keep;   // blocks per tile
  p.ok = NB >= 1;
  p.target = p.ok ? target_workgroups(dev, DP, p.GS, p.SP, row_fmt(k->fmt), row_fmt(v->fmt), DP == k->head_dim)
                  : kDefaultTargetWorkgroups;
  if (n == 0 || !p.ok) {
    p.ns = 1;
    p.chunk = 0;
  } else {
    // enough splits to fill the device once; every wave of a split gets a
    // tile or more.  A split only pays when one split would leave some wave
    // more than two tiles: the combine costs about what a wave spends on a
    // tile or two (a C1-sized decode: 10.8 us with one split, 11.7 with two).
    const int64_t tiles = (n + NB - 1) / NB;
    int64_t ns = (p.target + p.pairs - 1) / p.pairs;
    int64_t ns_max = (tiles + kDecodeWaves - 1) / kDecodeWaves;
    if (tiles <= 2 * kDecodeWaves) ns_max = 1;
    if (ns > ns_max) ns = ns_max;
    if (ns < 1) ns = 1;
    if (ns > kMaxSplits) ns = kMaxSplits;
    const int64_t chunk_tiles = (tiles + ns - 1) / ns;
    p.chunk = chunk_tiles * NB;
    p.ns = (int)((n + p.chunk - 1) / p.chunk);
  }
  p.n_wg = p.pairs * p.ns;
  // Arrival counters live in a fixed region at the start of every workspace,
  // so calls of different shapes that share one workspace never see another
  // call's partials where they expect a zero counter.  More than one split
  // only happens below p.target <= kMaxTargetWorkgroups pairs, which bounds
  // the region.
  if (p.ns > 1 && p.pairs > kMaxTargetWorkgroups) p.ok = false;
  // the launch: grid z = batch rows x kv heads, row counts per (b, h) in 32 bits
  if (k->batch * k->heads > 65535 || k->capacity * k->keep > INT32_MAX || v->capacity * v->keep > INT32_MAX)
    p.ok = false;
  const size_t counters = (size_t)kMaxTargetWorkgroups * kCounterStride * 4;
  const size_t ml = align256((size_t)p.pairs * p.ns * p.GS * 2 * 4);
  const size_t acc = (size_t)p.pairs * p.ns * p.GS * DP * 4;
  p.off_ml = counters;
  p.off_acc = counters + ml;
  p.bytes = counters + ml + acc;
  return p;
}

int check_decode(const codec_stream *k, const codec_stream *v, int64_t Hq) {
  int rc = check_stream(k);
  if (rc) return rc;
  rc = check_stream(v);
  if (rc) return rc;
  if (!same_geometry(k, v)) return CODEC_ERR_SHAPE;
  if ((k->fmt == CODEC_PNG) != (v->fmt == CODEC_PNG)) return CODEC_ERR_FORMAT;   // one synthesis for both
  if (Hq < 1 || Hq % k->heads != 0) return CODEC_ERR_SHAPE;
  if (k->n_blocks * k->block + k->n_tail == 0) return CODEC_ERR_SHAPE;
  return CODEC_OK;
}

}  // namespace

namespace cdattn {
// Query heads per workgroup: G rounded up to 1, 2, 4 or 8 (at most 8), so
// every coefficient row is read once per group of up to 8 query heads; a
// group past the kv head's G heads computes its absent heads on a live
// head's query and stores nothing for them.
int decode_group_size(int G) {
  if (G >= 8) return 8;
  int gs = 1;
  while (gs < G) gs *= 2;
  return gs;
}
int decode_pad_keep(int S) {
  int sp = 2;
  while (sp < S) sp *= 2;
  return sp;
}
int launch_decode(int D, int GS, int SP, int kf, int vf, bool full, const DecodeArgs &a, int64_t n_wg,
                  hipStream_t stream) {
  switch (kf * 3 + vf) {
    case I8 * 3 + I8:
      return full ? launch_decode_i8_i8(D, GS, SP, a, n_wg, stream) : launch_decode_i8_i8_pad(D, GS, SP, a, n_wg, stream);
    case I8 * 3 + BF16:
      return full ? launch_decode_i8_bf16(D, GS, SP, a, n_wg, stream) : launch_decode_i8_bf16_pad(D, GS, SP, a, n_wg, stream);
    case I8 * 3 + F32:
      return full ? launch_decode_i8_f32(D, GS, SP, a, n_wg, stream) : launch_decode_i8_f32_pad(D, GS, SP, a, n_wg, stream);
    case BF16 * 3 + I8:
      return full ? launch_decode_bf16_i8(D, GS, SP, a, n_wg, stream) : launch_decode_bf16_i8_pad(D, GS, SP, a, n_wg, stream);
    case BF16 * 3 + BF16:
      return full ? launch_decode_bf16_bf16(D, GS, SP, a, n_wg, stream) : launch_decode_bf16_bf16_pad(D, GS, SP, a, n_wg, stream);
    case BF16 * 3 + F32:
      return full ? launch_decode_bf16_f32(D, GS, SP, a, n_wg, stream) : launch_decode_bf16_f32_pad(D, GS, SP, a, n_wg, stream);
    case F32 * 3 + I8:
      return full ? launch_decode_f32_i8(D, GS, SP, a, n_wg, stream) : launch_decode_f32_i8_pad(D, GS, SP, a, n_wg, stream);
    case F32 * 3 + BF16:
      return full ? launch_decode_f32_bf16(D, GS, SP, a, n_wg, stream) : launch_decode_f32_bf16_pad(D, GS, SP, a, n_wg, stream);
    case F32 * 3 + F32:
      return full ? launch_decode_f32_f32(D, GS, SP, a, n_wg, stream) : launch_decode_f32_f32_pad(D, GS, SP, a, n_wg, stream);
    default: return -1;
  }
}
int resident_decode(int D, int GS, int SP, int kf, int vf, bool full) {
  switch (kf * 3 + vf) {
    case I8 * 3 + I8: return full ? resident_decode_i8_i8(D, GS, SP) : resident_decode_i8_i8_pad(D, GS, SP);
    case I8 * 3 + BF16: return full ? resident_decode_i8_bf16(D, GS, SP) : resident_decode_i8_bf16_pad(D, GS, SP);
    case I8 * 3 + F32: return full ? resident_decode_i8_f32(D, GS, SP) : resident_decode_i8_f32_pad(D, GS, SP);
    case BF16 * 3 + I8: return full ? resident_decode_bf16_i8(D, GS, SP) : resident_decode_bf16_i8_pad(D, GS, SP);
    case BF16 * 3 + BF16: return full ? resident_decode_bf16_bf16(D, GS, SP) : resident_decode_bf16_bf16_pad(D, GS, SP);
    case BF16 * 3 + F32: return full ? resident_decode_bf16_f32(D, GS, SP) : resident_decode_bf16_f32_pad(D, GS, SP);
    case F32 * 3 + I8: return full ? resident_decode_f32_i8(D, GS, SP) : resident_decode_f32_i8_pad(D, GS, SP);
    case F32 * 3 + BF16: return full ? resident_decode_f32_bf16(D, GS, SP) : resident_decode_f32_bf16_pad(D, GS, SP);
    case F32 * 3 + F32: return full ? resident_decode_f32_f32(D, GS, SP) : resident_decode_f32_f32_pad(D, GS, SP);
    default: return -1;
  }
}
int stream_device(hipStream_t stream, int *dev) {
  if (stream == nullptr) return hipGetDevice(dev) == hipSuccess ? CODEC_OK : CODEC_ERR_HIP;
  hipDevice_t d = 0;
  if (hipStreamGetDevice(stream, &d) != hipSuccess) return CODEC_ERR_HIP;
  *dev = (int)d;
  return CODEC_OK;
}
}  // namespace cdattn

namespace {

// Validation of codec_append_step (no HIP call).
int check_append(const codec_stream *k, const codec_stream *v, const void *k_new, const int64_t kn_stride[2],
                 const void *v_new, const int64_t vn_stride[2]) {
  int rc = check_stream(k);
  if (rc) return rc;
  rc = check_stream(v);
  if (rc) return rc;
  if (!same_geometry(k, v)) return CODEC_ERR_SHAPE;
  if ((k->fmt == CODEC_PNG) != (v->fmt == CODEC_PNG)) return CODEC_ERR_FORMAT;   // one analysis for both
  if (!k_new || !v_new || !kn_stride || !vn_stride) return CODEC_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new)) return CODEC_ERR_SHAPE;
  for (int i = 0; i < 2; ++i)
    if (kn_stride[i] < 0 || kn_stride[i] % 8 != 0 || vn_stride[i] < 0 || vn_stride[i] % 8 != 0)
      return CODEC_ERR_SHAPE;
  const int complete = (k->n_tail + 1 == k->block) ? 1 : 0;
  if (complete && (k->n_blocks + 1 > k->capacity || v->n_blocks + 1 > v->capacity)) return CODEC_ERR_CAPACITY;
  return CODEC_OK;
}

// The append launch for validated arguments; advances both streams' counters.
int launch_append_step(codec_stream *k, codec_stream *v, const void *k_new, const int64_t kn_stride[2],
                       const void *v_new, const int64_t vn_stride[2], hipStream_t stream) {
  const int complete = (k->n_tail + 1 == k->block) ? 1 : 0;
  AppendArgs A;
  memset(&A, 0, sizeof(A));
  const codec_stream *ss[2] = {k, v};
  const void *nw[2] = {k_new, v_new};
  const int64_t *ns[2] = {kn_stride, vn_stride};
  for (int i = 0; i < 2; ++i) {
    EncodeArgs &e = A.e[i];
    e = stream_encode_args(ss[i]);
    const int64_t R = ss[i]->block, D = ss[i]->head_dim;
    e.src0 = ss[i]->tail;
    e.s0_b = ss[i]->heads * R * D;
    e.s0_h = R * D;
    e.s0_t = D;
    e.src1 = nw[i];
    e.s1_b = ns[i][0];
    e.s1_h = ns[i][1];
    e.split_i = (int32_t)(R - 1);
    e.n_new = 1;
  }
  A.t = k->n_tail;
  A.complete = complete;
  (void)hipGetLastError();
  if (launch_append(A, k->batch * k->heads, stream) != 0) return CODEC_ERR_HIP;
  for (codec_stream *s : {k, v}) {
    if (complete) {
      s->n_blocks += 1;
      s->n_tail = 0;
    } else {
      s->n_tail += 1;
    }
  }
  return CODEC_OK;
}

}  // namespace

namespace cdattn {
// Validation of a decode call apart from its workspace; fills the plan for
// the device of `stream` (no launch).
int decode_check_args(const void *q, const int64_t q_stride[2], int64_t Hq, const codec_stream *k,
                      const codec_stream *v, float scale, const void *out, const int64_t out_stride[2],
                      int32_t out_dtype, hipStream_t stream, DecodePlan *p) {
  if (!q || !q_stride || !out || !out_stride) return CODEC_ERR_NULL;
  int rc = check_decode(k, v, Hq);
  if (rc) return rc;
  if (out_dtype != CODEC_F32 && out_dtype != CODEC_BF16) return CODEC_ERR_FORMAT;
  if (!(scale > 0.0f) || !isfinite(scale)) return CODEC_ERR_SCALE;
  if (!aligned16(q) || q_stride[0] < 0 || q_stride[1] < 0 || q_stride[0] % 8 || q_stride[1] % 8)
    return CODEC_ERR_SHAPE;
  if (out_stride[0] < 0 || out_stride[1] < 0) return CODEC_ERR_SHAPE;
  int dev = -1;
  if (stream_device(stream, &dev) != CODEC_OK) dev = -1;
  *p = make_plan(k, v, Hq, dev);
  if (!p->ok) return CODEC_ERR_UNSUPPORTED;
  return CODEC_OK;
}
}  // namespace cdattn

namespace {
// Validation of codec_decode_attention (no launch); fills the plan.
int check_decode_call(const void *q, const int64_t q_stride[2], int64_t Hq, const codec_stream *k,
                      const codec_stream *v, float scale, const void *out, const int64_t out_stride[2],
                      int32_t out_dtype, const void *workspace, size_t workspace_bytes, hipStream_t stream,
                      DecodePlan *p) {
  const int rc = decode_check_args(q, q_stride, Hq, k, v, scale, out, out_stride, out_dtype, stream, p);
  if (rc) return rc;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) || workspace_bytes < p->bytes)
    return CODEC_ERR_WORKSPACE;
  return CODEC_OK;
}
}  // namespace

namespace cdattn {
// The decode launch for validated arguments.  fuse_k / fuse_v (non-null)
// bring one new token that joins the tail as slot k->n_tail.
int launch_decode_call(const void *q, const int64_t q_stride[2], int64_t Hq, const codec_stream *k,
                       const codec_stream *v, float scale, void *out, const int64_t out_stride[2],
                       int32_t out_dtype, void *workspace, const DecodePlan &p, const void *fuse_k,
                       const int64_t kn_stride[2], const void *fuse_v, const int64_t vn_stride[2],
                       hipStream_t stream) {
  DecodeArgs a;
  memset(&a, 0, sizeof(a));
  a.q = static_cast<const uint16_t *>(q);
  a.q_sb = q_stride[0];
  a.q_sh = q_stride[1];
  a.krows = k->rows;
  a.kscales = k->scales;
  a.ktail = k->tail;
  a.vrows = v->rows;
  a.vscales = v->scales;
  a.vtail = v->tail;
  a.k_bh_rows = k->capacity * k->keep;
  a.v_bh_rows = v->capacity * v->keep;
  a.kf = row_fmt(k->fmt);
  a.vf = row_fmt(v->fmt);
  a.png = k->fmt == CODEC_PNG ? 1 : 0;
  a.Dm = k->head_dim;
  a.kraw = k->raw_dtype;
  a.vraw = v->raw_dtype;
  a.H = (int32_t)k->heads;
  a.G = (int32_t)(Hq / k->heads);
  a.NQG = p.NQG;
  a.R = k->block;
  a.S = k->keep;
  a.n_blocks = k->n_blocks;
  a.n_tail = k->n_tail;
  a.ns = p.ns;
  a.chunk = p.chunk;
  a.qk_scale = (float)((double)scale * 1.4426950408889634);   // log2(e)
  if (fuse_k) {
    a.fuse_new = 1;
    a.knew = fuse_k;
    a.vnew = fuse_v;
    a.kn_sb = kn_stride[0];
    a.kn_sh = kn_stride[1];
    a.vn_sb = vn_stride[0];
    a.vn_sh = vn_stride[1];
  }
  a.out = out;
  a.o_sb = out_stride[0];
  a.o_sh = out_stride[1];
  a.out_f32 = out_dtype == CODEC_F32 ? 1 : 0;
  char *ws = static_cast<char *>(workspace);
  a.counters = reinterpret_cast<uint32_t *>(ws);
  a.part_ml = reinterpret_cast<float *>(ws + p.off_ml);
  a.part_acc = reinterpret_cast<float *>(ws + p.off_acc);
#ifdef CDATTN_TIMELINE
  a.timeline = g_timeline;
  a.timeline_words = g_timeline_words;
#endif
  (void)hipGetLastError();
  const int DP = pad_dim(k->head_dim);
  const int lr = launch_decode(DP, p.GS, p.SP, row_fmt(k->fmt), row_fmt(v->fmt), DP == k->head_dim, a, p.n_wg, stream);
  if (lr < 0) return CODEC_ERR_UNSUPPORTED;
  if (lr > 0) return CODEC_ERR_HIP;
  return CODEC_OK;
}
}  // namespace cdattn

extern "C" {

const char *codec_status_string(int status) {
  switch (status) {
    case CODEC_OK: return "ok";
    case CODEC_ERR_NULL: return "a required pointer is NULL";
    case CODEC_ERR_SHAPE: return "size out of range, shapes disagree, or misaligned buffer";
    case CODEC_ERR_FORMAT: return "unknown or unsupported format";
    case CODEC_ERR_CAPACITY: return "archive capacity too small";
    case CODEC_ERR_STATE: return "stream counters forbid this call";
    case CODEC_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case CODEC_ERR_UNSUPPORTED: return "no kernel for this configuration";
    case CODEC_ERR_HIP: return "HIP runtime or kernel launch error";
    case CODEC_ERR_SCALE: return "scale must be finite and positive";
    default: return "unknown status";
  }
}

int codec_basis(int32_t R, int32_t S, float *A_host) {
  if (!A_host) return CODEC_ERR_NULL;
  if (R < 1 || R > CODEC_MAX_BLOCK || S < 1 || S > R || S > CODEC_MAX_KEEP) return CODEC_ERR_SHAPE;
  for (int i = 0; i < R; ++i)
    for (int j = 0; j < S; ++j) A_host[i * S + j] = kBasisHost[basis_index(R, j, i)];
  return CODEC_OK;
}

int codec_encode_blocks(codec_stream *s, const void *x, const int64_t x_stride[3], int64_t T,
                        hipStream_t stream) {
  int rc = check_stream(s);
  if (rc) return rc;
  if (!x_stride) return CODEC_ERR_NULL;
  if (T < 0) return CODEC_ERR_SHAPE;
  if (T > 0 && !x) return CODEC_ERR_NULL;
  if (s->n_tail != 0) return CODEC_ERR_STATE;
  const int64_t R = s->block;
  const int64_t n_new = T / R;
  const int32_t t = (int32_t)(T % R);
  if (n_new > 0 && s->n_blocks + n_new > s->capacity) return CODEC_ERR_CAPACITY;
  if (T > 0) {
    if (!aligned16(x)) return CODEC_ERR_SHAPE;
    for (int i = 0; i < 3; ++i)
      if (x_stride[i] < 0 || x_stride[i] % 8 != 0) return CODEC_ERR_SHAPE;
  }
  if (T == 0) return CODEC_OK;
  EncodeArgs e = stream_encode_args(s);
  e.src0 = x;
  e.s0_b = x_stride[0];
  e.s0_h = x_stride[1];
  e.s0_t = x_stride[2];
  e.src1 = x;
  e.split_i = (int32_t)R;
  e.n_new = n_new;
  e.n_copy = t;
  (void)hipGetLastError();
  rc = launch_encode(e, s->batch * s->heads, stream);
  if (rc < 0) return CODEC_ERR_UNSUPPORTED;   // grid beyond 2^31 - 1 workgroups
  if (rc > 0) return CODEC_ERR_HIP;
  s->n_blocks += n_new;
  s->n_tail = t;
  return CODEC_OK;
}

int codec_append_step(codec_stream *k, codec_stream *v, const void *k_new, const int64_t kn_stride[2],
                      const void *v_new, const int64_t vn_stride[2], hipStream_t stream) {
  const int rc = check_append(k, v, k_new, kn_stride, v_new, vn_stride);
  if (rc) return rc;
  return launch_append_step(k, v, k_new, kn_stride, v_new, vn_stride, stream);
}

int codec_decode_workspace_bytes(const codec_stream *k, const codec_stream *v, int64_t Hq, size_t *bytes) {
  if (!bytes) return CODEC_ERR_NULL;
  const int rc = check_decode(k, v, Hq);
  if (rc) return rc;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  const DecodePlan p = make_plan(k, v, Hq, dev);
  if (!p.ok) return CODEC_ERR_UNSUPPORTED;
  *bytes = p.bytes;
  return CODEC_OK;
}

int codec_decode_attention(const void *q, const int64_t q_stride[2], int64_t Hq, const codec_stream *k,
                           const codec_stream *v, float scale, void *out, const int64_t out_stride[2],
                           int32_t out_dtype, void *workspace, size_t workspace_bytes, hipStream_t stream) {
  DecodePlan p;
  const int rc = check_decode_call(q, q_stride, Hq, k, v, scale, out, out_stride, out_dtype, workspace,
                                   workspace_bytes, stream, &p);
  if (rc) return rc;
  return launch_decode_call(q, q_stride, Hq, k, v, scale, out, out_stride, out_dtype, workspace, p, nullptr,
                            nullptr, nullptr, nullptr, stream);
}

int codec_decode_attention_append(const void *q, const int64_t q_stride[2], int64_t Hq, codec_stream *k,
                                  codec_stream *v, const void *k_new, const int64_t kn_stride[2],
                                  const void *v_new, const int64_t vn_stride[2], float scale, void *out,
                                  const int64_t out_stride[2], int32_t out_dtype, void *workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  int rc = check_append(k, v, k_new, kn_stride, v_new, vn_stride);
  if (rc) return rc;
  // the decode is validated on the streams as the append leaves them
  const bool complete = k->n_tail + 1 == k->block;
  codec_stream k2 = *k, v2 = *v;
  for (codec_stream *s : {&k2, &v2}) {
    if (complete) {
      s->n_blocks += 1;
      s->n_tail = 0;
    } else {
      s->n_tail += 1;
    }
  }
  DecodePlan p;
  rc = check_decode_call(q, q_stride, Hq, &k2, &v2, scale, out, out_stride, out_dtype, workspace,
                         workspace_bytes, stream, &p);
  if (rc) return rc;
  if (complete) {
    // the token completes a block: archive it, then attend.  If the decode
    // launch fails, the counters go back to their values before the call:
    // the archive launch wrote only slot n_blocks (spare capacity under the
    // restored counters) and left tail slots 0..R-2 as they were, so the
    // restored stream is the one the caller passed in.
    const codec_stream k0 = *k, v0 = *v;
    rc = launch_append_step(k, v, k_new, kn_stride, v_new, vn_stride, stream);
    if (rc) return rc;
    rc = launch_decode_call(q, q_stride, Hq, k, v, scale, out, out_stride, out_dtype, workspace, p, nullptr,
                            nullptr, nullptr, nullptr, stream);
    if (rc) {
      *k = k0;
      *v = v0;
    }
    return rc;
  }
  rc = launch_decode_call(q, q_stride, Hq, k, v, scale, out, out_stride, out_dtype, workspace, p, k_new,
                          kn_stride, v_new, vn_stride, stream);
  if (rc) return rc;
  k->n_tail += 1;
  v->n_tail += 1;
  return CODEC_OK;
}

namespace {

// Arguments of the view kernel for one stream (rows, scales, tail, basis).
ViewArgs stream_view_args(const codec_stream *s) {
  ViewArgs a;
  memset(&a, 0, sizeof(a));
  a.rows = s->rows;
  a.scales = s->scales;
  a.tail = s->tail;
  a.rf = row_fmt(s->fmt);
  a.raw = s->raw_dtype;
  a.png = s->fmt == CODEC_PNG ? 1 : 0;
  a.R = s->block;
  a.S = s->keep;
  a.D = s->head_dim;
  a.H = s->heads;
  a.BH = s->batch * s->heads;
  a.cap = s->capacity;
  return a;
}

}  // namespace

int codec_materialise(const codec_stream *s, int64_t block_begin, void *dst, const int64_t dst_stride[3],
                      int32_t dst_dtype, hipStream_t stream) {
  int rc = check_stream(s);
  if (rc) return rc;
  if (!dst || !dst_stride) return CODEC_ERR_NULL;
  if (!raw_ok(dst_dtype)) return CODEC_ERR_FORMAT;
  if (block_begin < 0 || block_begin > s->n_blocks) return CODEC_ERR_STATE;
  if (!aligned16(dst)) return CODEC_ERR_SHAPE;
  for (int i = 0; i < 3; ++i)
    if (dst_stride[i] < 0 || dst_stride[i] % 8 != 0) return CODEC_ERR_SHAPE;
  ViewArgs a = stream_view_args(s);
  a.out = dst_dtype;
  a.blk0 = block_begin;
  a.nblk = s->n_blocks - block_begin;
  a.tok_limit = s->block;
  a.n_copy = s->n_tail;
  a.dst = dst;
  a.o_sb = dst_stride[0];
  a.o_sh = dst_stride[1];
  a.o_st = dst_stride[2];
  a.o_t0 = block_begin * s->block;
  (void)hipGetLastError();
  const int lr = launch_view(a, stream);
  if (lr < 0) return CODEC_ERR_UNSUPPORTED;
  if (lr > 0) return CODEC_ERR_HIP;
  return CODEC_OK;
}

int codec_crop(codec_stream *s, int64_t new_len, hipStream_t stream) {
  int rc = check_stream(s);
  if (rc) return rc;
  const int64_t R = s->block;
  if (new_len < 0 || new_len > s->n_blocks * R + s->n_tail) return CODEC_ERR_STATE;
  const int64_t kb = new_len / R;
  const int32_t t = (int32_t)(new_len % R);
  if (kb < s->n_blocks && t > 0) {
    // the boundary block's first t tokens, decoded into tail slots 0..t-1
    ViewArgs a = stream_view_args(s);
    a.out = s->raw_dtype;
    a.blk0 = kb;
    a.nblk = 1;
    a.tok_limit = t;
    a.n_copy = 0;
    a.dst = s->tail;
    a.o_sb = s->heads * R * s->head_dim;
    a.o_sh = R * s->head_dim;
    a.o_st = s->head_dim;
    a.o_t0 = 0;
    (void)hipGetLastError();
    const int lr = launch_view(a, stream);
    if (lr < 0) return CODEC_ERR_UNSUPPORTED;
    if (lr > 0) return CODEC_ERR_HIP;
  }
  if (kb < s->n_blocks) s->n_blocks = kb;
  s->n_tail = t;
  return CODEC_OK;
}

int codec_select_batch(const codec_stream *src, codec_stream *dst, const int64_t *idx, int64_t n,
                       hipStream_t stream) {
  int rc = check_stream(src);
  if (rc) return rc;
  if (!dst || !idx) return CODEC_ERR_NULL;
  if (n < 1 || dst->batch != n) return CODEC_ERR_SHAPE;
  if (dst->heads != src->heads || dst->block != src->block || dst->keep != src->keep ||
      dst->head_dim != src->head_dim)
    return CODEC_ERR_SHAPE;
  if (dst->fmt != src->fmt || dst->raw_dtype != src->raw_dtype) return CODEC_ERR_FORMAT;
  if (!dst->tail || (src->n_blocks > 0 && !dst->rows) ||
      (src->n_blocks > 0 && src->fmt == CODEC_I8 && !dst->scales))
    return CODEC_ERR_NULL;
  if (dst->capacity < src->n_blocks) return CODEC_ERR_CAPACITY;
  if (!aligned16(dst->tail) || (dst->rows && !aligned16(dst->rows)) ||
      (dst->fmt == CODEC_I8 && dst->scales && !aligned16(dst->scales)))
    return CODEC_ERR_SHAPE;
  for (int64_t i = 0; i < n; ++i)
    if (idx[i] < 0 || idx[i] >= src->batch) return CODEC_ERR_SHAPE;
  const int64_t H = src->heads, S = src->keep, D = src->head_dim;
  const int64_t eb = elem_bytes(src->fmt);
  GatherArgs g;
  memset(&g, 0, sizeof(g));
  g.src_rows = src->rows;
  g.dst_rows = dst->rows;
  g.slab_bytes = src->capacity * S * D * eb;
  g.dst_slab_bytes = dst->capacity * S * D * eb;
  g.row_bytes = src->n_blocks * S * D * eb;
  if (src->fmt == CODEC_I8 && src->n_blocks > 0) {
    g.src_scales = src->scales;
    g.dst_scales = dst->scales;
    g.scale_slab = src->capacity * S;
    g.dst_scale_slab = dst->capacity * S;
    g.n_scales = src->n_blocks * S;
  }
  g.src_tail = src->tail;
  g.dst_tail = dst->tail;
  g.tail_bytes = (int64_t)src->block * D * elem_bytes(src->raw_dtype);
  g.H = H;
  // destination rows in chunks: at most kGatherChunk indices and 65535 (row, head) units per launch
  int64_t chunk = kGatherChunk;
  if (chunk * H > 65535) chunk = 65535 / H;
  if (chunk < 1) return CODEC_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  for (int64_t i0 = 0; i0 < n; i0 += chunk) {
    const int64_t m = n - i0 < chunk ? n - i0 : chunk;
    g.i0 = i0;
    for (int64_t k = 0; k < m; ++k) g.idx[k] = (int32_t)idx[i0 + k];
    if (launch_gather(g, m * H, stream) != 0) return CODEC_ERR_HIP;
  }
  dst->n_blocks = src->n_blocks;
  dst->n_tail = src->n_tail;
  return CODEC_OK;
}

}  // extern "C"

#ifdef CDATTN_TIMELINE
extern "C" int codec_timeline_set(void *buf, size_t bytes) {
  g_timeline = static_cast<unsigned long long *>(buf);
  g_timeline_words = buf ? (int64_t)(bytes / 8) : 0;
  return CODEC_OK;
}
#endif
