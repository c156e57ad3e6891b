/*
 * cdattn.h -- C ABI of the compressed-domain decode attention library
 * (libcdattn.so, HIP kernels for AMD Instinct MI355X / gfx950).
 *
 * The method (flashcodec-kv 1.0.0; README sections "Math", "Causal-safety
 * design" and "Materialization-free decode attention"; cache.py
 * ``_CodecStream``; triton_attention.py):
 *   - the sequence axis of a (batch, heads, seq, head_dim) key or value
 *     tensor is cut into blocks of R tokens;
 *   - every complete block X (R x D) is stored as the S lowest-frequency
 *     rows of its orthonormal DCT-II, C = M X (S x D), either as floats or as
 *     int8 codes with one fp32 scale per (block, frequency) row;
 *   - the incomplete last block stays raw (the "tail");
 *   - one decode query attends to the archive without reconstructing it:
 *     s = rows . q, logits = A s (A = M^T, R x S), online softmax,
 *     w = p A, acc += w . rows, split over block chunks and merged with a
 *     (max, sum, acc) combine.
 *
 * Conventions for every call
 *   - Tensor pointers are DEVICE pointers unless stated otherwise.
 *   - Strides are in elements.  The head_dim axis is always contiguous.
 *   - Every call validates all arguments synchronously BEFORE it enqueues
 *     anything; on error it returns a non-zero status, enqueues nothing and
 *     changes nothing (stream counters included).  The decode calls' split
 *     plan asks the runtime, once per device and kernel, for the stream's
 *     device, its CU count and the kernel's occupancy; every other check
 *     makes no HIP call.
 *   - Work is enqueued on the caller's `stream` and the call returns without
 *     waiting.  The library allocates no memory and keeps no pointer past
 *     the call.  The caller owns every buffer.
 *   - Calls that share a stream descriptor or a workspace must not run
 *     concurrently on different HIP streams.
 */
#ifndef CDATTN_H
#define CDATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status */
enum {
  CODEC_OK = 0,
  CODEC_ERR_NULL = 1,        /* a required pointer is NULL                            */
  CODEC_ERR_SHAPE = 2,       /* a size is out of range or two shapes disagree         */
  CODEC_ERR_FORMAT = 3,      /* unknown or unsupported row / raw / query / out format */
  CODEC_ERR_CAPACITY = 4,    /* archive capacity too small for the blocks to write    */
  CODEC_ERR_STATE = 5,       /* stream counters forbid the call (e.g. tail not empty) */
  CODEC_ERR_WORKSPACE = 6,   /* decode workspace missing, too small or misaligned     */
  CODEC_ERR_UNSUPPORTED = 7, /* valid arguments but no kernel compiled for them       */
  CODEC_ERR_HIP = 8,         /* a HIP runtime call or kernel launch failed            */
  CODEC_ERR_SCALE = 9        /* softmax scale not finite or not positive              */
};

/* ------------------------------------------------------------- formats  */
enum {
  CODEC_F32 = 0,   /* IEEE binary32                                            */
  CODEC_BF16 = 1,  /* bfloat16 (upper half of binary32), round-to-nearest-even */
  CODEC_I8 = 2,    /* int8 codes in [-127, 127] + fp32 scale per (block, row)  */
  CODEC_PNG = 3    /* rows only: PNG mode (README "Math", PNG item), S == R    */
                   /* fp32 rows per block: the anchor x_0, then the deltas     */
                   /* x_i - x_{i-1}; decoded by the cumulative sum.  Both      */
                   /* streams of a decode or append use it, or neither.        */
};

/* Limits of this build. */
#define CODEC_MAX_BLOCK 32   /* R: tokens per block                            */
#define CODEC_MAX_KEEP 32    /* S: kept frequencies (S <= R)                   */
#define CODEC_MAX_HEAD_DIM 256
/* head_dim D: 8 .. 256, a multiple of 8 (other values: UNSUPPORTED; the
 * pages' kernel declines only D > 256).  The kernels compute at D rounded up
 * to 64, 128 or 256; rows in memory keep the pitch D.  GQA group G = Hq / H
 * must be >= 1; the decode reads every coefficient row once per group of up
 * to 8 query heads (any G: 3 runs as a group of four, 12 as eight plus four).
 *                                                                            */

/*
 * One compressed key or value stream: the archive of complete blocks and the
 * raw tail of one (B, H, seq, D) tensor (cache.py ``_CodecStream``: raw tail
 * plus capacity-grown archive of coefficient rows; README "Causal-safety
 * design": only complete blocks are archived and never rewritten).
 *
 * Memory layouts (dense, row-major, owned by the caller):
 *   rows   [B][H][capacity][S][D]  elements of `fmt`
 *          block n of (b, h) holds the S coefficient rows of tokens
 *          n*R .. n*R+R-1 (frequency j = 0 .. S-1, lowest first)
 *   scales [B][H][capacity][S]     fp32, only when fmt == CODEC_I8
 *          (stored value = code * scale)
 *   tail   [B][H][R][D]            elements of `raw_dtype`; slots
 *          0 .. n_tail-1 hold the newest tokens, in order
 * The sequence length is n_blocks * R + n_tail.  The library advances
 * n_blocks / n_tail itself on success of encode and append calls; the caller
 * grows `capacity` (and re-points `rows` / `scales`) when a call returns
 * CODEC_ERR_CAPACITY.
 *
 * Layer stacks: the batch axis may hold (layer, batch row) pairs, layer-major
 * (batch = L * B, row l * B + b is batch row b of layer l), when the L layers
 * share R, S, D, formats, capacity and length.  Every call then does one
 * step for all L layers in one launch (the decode with its combine, the
 * fused append, the prefill, crop and gather); queries, tokens and outputs
 * use the same folded batch axis.  A stream whose `rows`, `scales` and `tail`
 * point at layer l's B rows of such a stack (batch = B) is that layer alone,
 * with its own counters.  flashcodec-kv README, end-to-end decode paragraph:
 * the remaining gap there is the per-layer launch pair; one launch per step
 * across layers needs every layer's query at once.
 */
typedef struct codec_stream {
  int32_t block;      /* R, 1 .. CODEC_MAX_BLOCK                          */
  int32_t keep;       /* S, 1 .. min(R, CODEC_MAX_KEEP)                    */
  int32_t head_dim;   /* D, 8 .. 256, a multiple of 8                      */
  int32_t fmt;        /* CODEC_F32 | CODEC_BF16 | CODEC_I8 (rows)          */
  int32_t raw_dtype;  /* CODEC_BF16 | CODEC_F32 (raw tokens and tail)      */
  int32_t n_tail;     /* raw tokens in the tail, 0 .. R-1                  */
  int64_t batch;      /* B >= 1                                            */
  int64_t heads;      /* H >= 1 (kv heads)                                 */
  int64_t capacity;   /* blocks allocated per (b, h), >= n_blocks          */
  int64_t n_blocks;   /* archived blocks per (b, h)                        */
  void *rows;         /* device, see layout above                          */
  float *scales;      /* device, fmt == CODEC_I8 only (else ignored)       */
  void *tail;         /* device, see layout above                          */
} codec_stream;

/*
 * Rows in PNG mode (fmt == CODEC_PNG) are produced by the arithmetic of the
 * fp32 rows with the difference matrix in place of M: row 0 = fp32(x_0), row
 * i = fp32(x_i - x_{i-1}) (exact fp64 difference, one rounding).  The
 * Top-M pruning of the pages is not applied (keep ratio 1: the lossless tier).
 *
 * codec_basis -- synthesis matrix A = M^T of the kept DCT-II rows, on the host.
 * README "Math", JPEG item: M[j, i] = c_j cos(pi (2i + 1) j / (2R)),
 * c_0 = sqrt(1/R), c_j = sqrt(2/R) (the normalisation that makes the rows
 * orthonormal).  Evaluated in double precision and rounded to fp32; this is
 * exactly the basis the kernels encode and decode with.
 *   A_host: caller-owned host array of R*S floats, A[i*S + j] = fp32(M[j][i]).
 * Errors: CODEC_ERR_NULL, CODEC_ERR_SHAPE (R or S out of range).
 */
int codec_basis(int32_t R, int32_t S, float *A_host);

/*
 * codec_encode_blocks -- archive a run of raw tokens (prefill).
 * cache.py ``_CodecStream.append`` / ``_archive``: the floor(T/R) complete
 * blocks are projected onto the kept DCT-II rows and written at archive
 * slots n_blocks .. n_blocks + floor(T/R) - 1 in one launch; the last T mod R
 * tokens are copied verbatim into tail slots 0 .. T mod R - 1.
 * Arithmetic (bit-exact contract): c = sum_{i<R} fp64(A[i][j]) * fp64(x_i)
 * accumulated left to right from +0.0 in fp64; fp32 rows = fp32(c); bf16
 * rows = bf16(fp32(c)) (both round-to-nearest-even); int8 rows:
 * a = max_d |c|, scale = fp32(a / 127), code = clamp(rint(c / scale), +-127)
 * with ties to even, scale 0 -> codes 0.
 *   s        stream; requires s->n_tail == 0; on success n_blocks grows by
 *            floor(T/R) and n_tail = T mod R.
 *   x        device, (B, H, T, D) elements of s->raw_dtype.
 *   x_stride element strides of the b, h and t axes (d stride is 1).
 *   T        tokens, >= 0 (T == 0 is a no-op).
 * Errors: NULL, SHAPE, FORMAT, STATE (tail not empty), CAPACITY,
 * UNSUPPORTED (a launch of more than 2^31 - 1 workgroups: about 2^33 blocks
 * over all (b, h)), HIP.
 */
int codec_encode_blocks(codec_stream *s, const void *x, const int64_t x_stride[3],
                        int64_t T, hipStream_t stream);

/*
 * codec_append_step -- append one decode token to a key and a value stream.
 * cache.py ``_CodecStream.append`` with one token: the token goes into tail
 * slot n_tail; when that completes a block (n_tail + 1 == R) the same launch
 * encodes the R tail tokens into archive slot n_blocks with the arithmetic of
 * codec_encode_blocks (bit-identical), and the tail becomes empty.  Archived
 * blocks are never touched (README "Causal-safety design").
 *   k, v          the two streams (same B, H, R, D; formats may differ).
 *   k_new, v_new  device, (B, H, 1, D) of the stream's raw_dtype.
 *   kn_stride, vn_stride  element strides of the b and h axes.
 * Errors: NULL, SHAPE, FORMAT, CAPACITY (a block completes and capacity ==
 * n_blocks), HIP.  Counters of both streams change only on success.
 */
int codec_append_step(codec_stream *k, codec_stream *v,
                      const void *k_new, const int64_t kn_stride[2],
                      const void *v_new, const int64_t vn_stride[2],
                      hipStream_t stream);

/*
 * codec_decode_workspace_bytes -- workspace needed by codec_decode_attention
 * for these streams and Hq query heads on the current device.  The split
 * count, and so the size, follows from the shapes and from the number of
 * decode workgroups that fill the device once (its CU count times the
 * kernel's workgroups resident per CU, asked of the runtime once per device
 * and kernel; 256 on a host without a GPU, at most 1024): a decode on a
 * stream of another device of the same kind plans the same.
 * The workspace holds a fixed 256 KiB region of arrival counters (one per
 * (b, kv head, query group), 256 bytes apart) followed by the per-split
 * (max, sum, acc) partials.  It must be zero-filled once before its first
 * use; every completed decode call leaves the counters at zero again, so
 * one workspace (of the largest size needed) can be reused without clearing
 * by calls of any shape, one call at a time.
 * Errors: NULL, SHAPE, FORMAT, UNSUPPORTED.
 */
int codec_decode_workspace_bytes(const codec_stream *k, const codec_stream *v,
                                 int64_t Hq, size_t *bytes);

/*
 * codec_decode_attention -- one decode query per head against the
 * compressed archive and the raw tail, without reconstructing K or V.
 * README "Materialization-free decode attention" (q . K[p] = (q . S^T) A[p],
 * out = (p A) S) and triton_attention.py (split over block chunks, partial
 * (max, sum, acc) per split, flash-decoding combine).  Query head hq uses kv
 * head hq / (Hq / H).  Result = softmax(scale * q . K_t) weighted sum of V_t
 * over all n_blocks * R + n_tail tokens, K_t / V_t being the decoded rows.
 *   q            device, (B, Hq, 1, D) bf16; q_stride = strides of b and h.
 *   Hq           query heads, a multiple of k->heads.
 *   k, v         streams with equal B, H, R, S, D, n_blocks, n_tail.
 *   scale        softmax scale (> 0, finite); the usual choice is D^-1/2.
 *   out          device, (B, Hq, 1, D) of out_dtype (CODEC_F32 | CODEC_BF16);
 *                out_stride = strides of b and h.
 *   workspace    device, >= codec_decode_workspace_bytes, 256-byte aligned,
 *                zero-filled before its first use (see above).
 * Errors: NULL, SHAPE (includes an empty sequence), FORMAT, SCALE,
 * WORKSPACE, UNSUPPORTED (no kernel for the shape, B * H above 65535, or
 * 2^31 or more coefficient rows per (b, h) in a stream's capacity), HIP.
 * Shapes with a kernel: a decode tile must hold whole blocks, so S may not
 * exceed the tile's rows, 8192 / (D' (bytes per key element + bytes per
 * value element)) with D' = D rounded up to 64, 128 or 256, raised to 32
 * when the values are int8 or bf16 and 32 such rows take at most 12 KB.
 * That is S <= 32 for int8 keys and values up to D = 128 and S <= 16 at
 * D <= 256; bf16 keys and values: 32 / 16 / 8 at D' = 64 / 128 / 256; fp32
 * (and PNG) keys and values: 16 / 8 / 4.  Other S give UNSUPPORTED (from
 * codec_decode_workspace_bytes as well).
 */
int codec_decode_attention(const void *q, const int64_t q_stride[2], int64_t Hq,
                           const codec_stream *k, const codec_stream *v, float scale,
                           void *out, const int64_t out_stride[2], int32_t out_dtype,
                           void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * codec_decode_attention_append -- one decode step of a layer in one call:
 * codec_append_step(k, v, k_new, .., v_new, ..) followed by
 * codec_decode_attention(q, .., k, v, ..), with identical results, stream
 * state and output.  The pages attend to the new token as part of the
 * cache (cache.py ``append`` then triton_attention.py); when the token does
 * not complete a block, the decode launch itself reads it as tail row
 * n_tail and stores it to that tail slot (one launch instead of two); a
 * token that completes a block is archived by the append launch first.
 * Arguments as in the two calls; the workspace must satisfy
 * codec_decode_workspace_bytes for the streams as the append leaves them.
 * Errors: those of both calls, all checked before any launch; counters
 * change only on success.  One exception to "an error enqueues nothing":
 * when the token completes a block and the decode launch itself fails
 * (CODEC_ERR_HIP) after the archive launch was enqueued, that launch has
 * written archive slot n_blocks; the counters are restored, so the slot is
 * spare capacity again and the stream holds what it held before the call.
 */
int codec_decode_attention_append(const void *q, const int64_t q_stride[2], int64_t Hq, codec_stream *k,
                                  codec_stream *v, const void *k_new, const int64_t kn_stride[2],
                                  const void *v_new, const int64_t vn_stride[2], float scale, void *out,
                                  const int64_t out_stride[2], int32_t out_dtype, void *workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/*
 * codec_decode_attention_noalloc -- codec_decode_attention without a caller
 * workspace, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments (minus the workspace), kernels, split plan and results as
 * codec_decode_attention, bit for bit.  The split partials and arrival
 * counters live in a library-owned device array of CODEC_SCRATCH_BYTES per
 * GPU (zero when the library is loaded, held until the process ends; every
 * completed call leaves its counters at zero again).  The call allocates
 * nothing; its first call on a device looks up that device's copy of the
 * array (hipGetSymbolAddress, which may load the library's code onto the
 * device) and keeps the address, so make that first call outside graph
 * capture; later calls may be captured.
 * Limit: a decode whose split plan has more than one split per (b, kv head,
 * query group) needs codec_decode_workspace_bytes(k, v, Hq) of scratch and
 * is rejected with CODEC_ERR_WORKSPACE when that exceeds CODEC_SCRATCH_BYTES
 * (only the largest head_dim / group-size shapes with about 255 (b, kv head)
 * pairs reach it); a single-split plan uses none.
 * Concurrency: all calls on one GPU share the array, so calls that overlap
 * on that GPU (different HIP streams, or one graph replayed on two streams)
 * race and must be serialised by the caller.
 * Errors: those of codec_decode_attention (WORKSPACE as above), UNSUPPORTED
 * (device index of 64 or more), HIP (including a failed address lookup).
 */
#define CODEC_SCRATCH_BYTES (4u << 20)
int codec_decode_attention_noalloc(const void *q, const int64_t q_stride[2], int64_t Hq,
                                   const codec_stream *k, const codec_stream *v, float scale, void *out,
                                   const int64_t out_stride[2], int32_t out_dtype, hipStream_t stream);

/*
 * codec_materialise -- the decoded (materialised) view of a stream, e.g. for
 * prefill attention.  cache.py ``_CodecStream.read`` / ``_decode_pending``:
 * the view is the archived blocks decoded, X_hat = M^T C block by block
 * (README "Math"), followed by the raw tail, in the stream's dtype; it is
 * memoised and append-only (README "Causal-safety design": archived blocks
 * never change), so a read only decodes the blocks archived since the last.
 * This call decodes blocks block_begin .. n_blocks-1 into dst tokens
 * block_begin*R .. n_blocks*R-1 and copies the n_tail raw tokens to dst
 * tokens n_blocks*R .. n_blocks*R+n_tail-1; dst tokens below block_begin*R
 * are not touched.
 * Arithmetic (bit-exact contract): x_hat = sum over j = 0..S-1, in order,
 * from +0.0, of fp64(A[i][j]) * c_hat[j] with separately rounded fp64
 * products and sums (no fused multiply-add); c_hat = fp64(code) *
 * fp64(scale) for int8 rows (exact), the stored value for float rows.
 * Output fp32(x_hat), or bf16(fp32(x_hat)) (RNE); tail tokens converted
 * (bf16 -> fp32 exact, fp32 -> bf16 RNE).
 *   s            the stream (not modified).
 *   block_begin  0 .. n_blocks (n_blocks: only the tail is written).
 *   dst          device, (B, H, >= n_blocks*R + n_tail, D) of dst_dtype,
 *                16-byte aligned; dst_stride = element strides of the b, h
 *                and t axes, each a multiple of 8 (d is contiguous).
 *   dst_dtype    CODEC_F32 | CODEC_BF16.
 * Errors: NULL, SHAPE, FORMAT, STATE (block_begin out of range),
 * UNSUPPORTED (B or H above 65535), HIP.
 */
int codec_materialise(const codec_stream *s, int64_t block_begin, void *dst, const int64_t dst_stride[3],
                      int32_t dst_dtype, hipStream_t stream);

/*
 * codec_crop -- remove trailing tokens exactly (cache.py
 * ``_CodecStream.crop``).  With kb = new_len / R and t = new_len mod R:
 *   kb <  n_blocks: blocks kb .. leave the archive (their rows are left as
 *                   they are); when t > 0 the first t tokens of block kb,
 *                   decoded as in codec_materialise into the raw dtype,
 *                   become tail slots 0..t-1; n_blocks = kb, n_tail = t.
 *   kb == n_blocks: the cut is inside the raw tail: n_tail = t (no launch).
 * Archived blocks below kb are never re-encoded, so repeated crops are
 * idempotent and crops compose (crop to L1, then to L2 <= L1, equals crop
 * to L2).
 *   s        the stream; counters change only on success.
 *   new_len  tokens to keep, 0 .. n_blocks*R + n_tail.
 * Errors: NULL, SHAPE, FORMAT, STATE (new_len out of range), UNSUPPORTED
 * (B or H above 65535), HIP.
 */
int codec_crop(codec_stream *s, int64_t new_len, hipStream_t stream);

/*
 * codec_select_batch -- gather rows of the batch axis (beam reorder; cache.py
 * ``_CodecStream.select_batch``).  Batch row i of dst becomes batch row
 * idx[i] of src: archived rows 0..n_blocks-1, their scales and all R tail
 * slots; dst's n_blocks and n_tail are set to src's.
 *   src   stream, not modified.
 *   dst   stream with batch == n and the same heads, R, S, D, fmt and
 *         raw_dtype, capacity >= src->n_blocks; its buffers must not
 *         overlap src's (gathering in place needs new buffers).
 *   idx   HOST array of n source batch rows, each in [0, src->batch).
 * Errors: NULL, SHAPE (geometry or an index out of range), FORMAT,
 * CAPACITY, UNSUPPORTED (more than 65535 heads), HIP.
 */
int codec_select_batch(const codec_stream *src, codec_stream *dst, const int64_t *idx, int64_t n,
                       hipStream_t stream);

/* codec_status_string -- static text for a status code (never NULL). */
const char *codec_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* CDATTN_H */
