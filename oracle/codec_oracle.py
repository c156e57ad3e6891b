"""fp64 CPU oracle for compressed-domain decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code, tables or constants
with the HIP library; the two meet only through the seeded synthetic inputs.

What it computes, and where the pages fix it
--------------------------------------------
Citations name the page and the section on it.  "README" is the project
description shipped in the flashcodec-kv 1.0.0 wheel (page "flashcodec-kv
1.0.0 .whl, page 4"); "cache.py" is the stream manager source on page
"flashcodec-kv 1.0.0 .whl, page 2"; "triton_attention.py" is the kernel
source on page 4.

* Block DCT-II basis, lowest S of R frequencies kept, orthonormal rows
  (README, section "Math", JPEG item).
* Encode: every complete block of R tokens along the sequence axis becomes
  S coefficient rows C = M X (README "Math"; cache.py ``_CodecStream._archive``).
* int8 variant: codes plus one fp32 scale per (block, frequency)
  (README, paragraph on ``quant_bits=8``; cache.py ``_archive_spec``).
* Only complete blocks are archived; the rest stays raw at full fidelity
  (README "Causal-safety design"; cache.py ``append``).
* Decode attention is, up to rounding, ordinary softmax attention over the
  reconstructed keys/values X_hat = M^T C followed by the raw tail
  (README "Materialization-free decode attention": the coefficient-domain
  form equals the materialised one).  The oracle therefore materialises.
* GQA: query head hq reads kv head hq // G (triton_attention.py, program
  id decomposition in the split kernel).

Readings where the pages are silent (each also listed in the design notes)
---------------------------------------------------------------------------
1. c_0 = sqrt(1/R), c_j = sqrt(2/R) for j >= 1: the only constants that make
   the rows orthonormal.
2. The basis used by the codec is M32 = fp32(M64) (round to nearest even).
3. Projection: fp64, products M32[j,i]*x exact, summed left to right over
   i = 0..R-1 starting from +0.0.
4. Float rows are fp32(C); bf16 rows are bf16(fp32(C)), both RNE.
5. int8: a = max_d |C|, scale = fp32(a / 127) (fp64 division, then RNE),
   code = clamp(rint_half_even(C / fp64(scale)), -127, 127); a zero scale
   gives zero codes.
6. Dequantised row = code * scale (exact in fp64).
7. Softmax uses the natural exponential, max-subtracted; default
   scale = D ** -0.5 (triton_attention.py host wrapper).
8. n = 0 complete blocks is allowed (tail-only attention); T = 0 is an error.
9. The materialised view is the fp64 reconstruction rounded to the view's
   format like a float row (reading 4); a crop that cuts into the archive
   re-exposes the boundary block's first tokens from that view, in the
   stream's raw format.
10. PNG mode (README "Math", PNG item; cache.py ``_archive_spec``): S = R
    fp32 rows per block, the anchor x_0 and the deltas x_i - x_{i-1}, formed
    by the same fixed-order fp64 projection with the difference matrix and
    rounded to fp32 (the README keeps PNG deltas in fp32); the anchor is
    stored in fp32 too (it holds a bf16 or fp32 token exactly).  Decoding is
    the cumulative sum.  The Top-M pruning rule is not on the pages: only
    keep_ratio = 1.0 (no pruning, the lossless tier) is implemented.
"""

import math

import numpy as np

F32 = "f32"
BF16 = "bf16"
I8 = "i8"
PNG = "png"     # PNG mode: S = R fp32 rows, anchor + first-order deltas
FORMATS = (F32, BF16, I8, PNG)


# ---------------------------------------------------------------------------
# basis
# ---------------------------------------------------------------------------
def dct_basis_f64(R, S):
    """Analysis matrix M64 (S x R): M[j, i] = c_j cos(pi (2i + 1) j / (2R)).

    README "Math", JPEG item: M[j, n] = c_j cos(pi/r (n + 1/2) j) with
    orthonormal rows; the lowest S frequencies are kept.  Reading 1 fixes
    c_j.  Evaluated element by element with the C library's cos.
    """
    if not (1 <= S <= R):
        raise ValueError("need 1 <= S <= R")
    M = np.empty((S, R), dtype=np.float64)
    for j in range(S):
        cj = math.sqrt(1.0 / R) if j == 0 else math.sqrt(2.0 / R)
        for i in range(R):
            M[j, i] = cj * math.cos(math.pi * (2 * i + 1) * j / (2 * R))
    return M


def dct_basis_f32(R, S):
    """The codec's basis: M64 rounded to fp32 (reading 2)."""
    return dct_basis_f64(R, S).astype(np.float32)


def png_analysis(R):
    """PNG mode's analysis matrix (R x R): row 0 keeps the anchor x_0, row
    i >= 1 the first-order delta x_i - x_{i-1} (README "Math", PNG item)."""
    M = np.zeros((R, R), dtype=np.float64)
    M[0, 0] = 1.0
    for i in range(1, R):
        M[i, i], M[i, i - 1] = 1.0, -1.0
    return M


def png_synthesis(R):
    """PNG mode's synthesis (R x R): x_hat_i = x_0 + sum_{j=1..i} delta_j,
    the cumulative sum of the README's rebuild (A[i, j] = 1 for j <= i)."""
    return np.tril(np.ones((R, R), dtype=np.float64))


def analysis(R, S, fmt):
    """Rows x tokens matrix that encodes a block in format `fmt`."""
    if fmt == PNG:
        if S != R:
            raise ValueError("PNG mode keeps S = R rows")
        return png_analysis(R)
    return dct_basis_f32(R, S).astype(np.float64)


def synthesis(R, S, fmt):
    """Tokens x rows matrix that decodes a block (A, with X_hat = A C)."""
    if fmt == PNG:
        return png_synthesis(R)
    return dct_basis_f32(R, S).astype(np.float64).T


# ---------------------------------------------------------------------------
# rounding helpers (bit-level, so results can be compared byte for byte)
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(v):
    """Round fp32 values to bf16, nearest-even; returns the uint16 patterns."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f64(bits):
    """Exact value of bf16 bit patterns as fp64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# encode
# ---------------------------------------------------------------------------
def project_blocks(x, R, S, fmt=F32):
    """fp64 coefficients of every complete block.

    x: (..., T, D) real values (bf16 or fp32 values held in any float dtype).
    Returns C: (..., n, S, D) with n = T // R and
        C[..., n, j, :] = sum_{i<R} M32[j, i] * x[..., n*R + i, :]
    summed left to right from +0.0 (reading 3).  README "Math": C = M X
    block by block along the sequence axis.  PNG mode uses the difference
    matrix instead of M32 (reading 10).
    """
    x = np.asarray(x, dtype=np.float64)
    T, D = x.shape[-2], x.shape[-1]
    lead = x.shape[:-2]
    n = T // R
    xb = x[..., : n * R, :].reshape(*lead, n, R, D)
    M = analysis(R, S, fmt)
    C = np.empty((*lead, n, S, D), dtype=np.float64)
    for j in range(S):
        acc = np.zeros((*lead, n, D), dtype=np.float64)
        for i in range(R):
            acc = acc + M[j, i] * xb[..., i, :]
        C[..., j, :] = acc
    return C


def quantize_rows(C):
    """int8 codes and fp32 scales, one scale per (block, frequency) row.

    README paragraph on ``quant_bits=8`` (int8 coefficients with a
    per-(block, frequency) scale); the scale rule and rounding are
    reading 5.  Returns (codes int8 (..., S, D), scales float32 (..., S)).
    """
    C = np.asarray(C, dtype=np.float64)
    a = np.max(np.abs(C), axis=-1)
    s32 = (a / 127.0).astype(np.float32)
    s64 = s32.astype(np.float64)[..., None]
    codes = np.zeros(C.shape, dtype=np.int8)
    nz = np.broadcast_to(s64 != 0.0, C.shape)
    y = np.divide(C, s64, out=np.zeros_like(C), where=nz)
    codes[nz] = np.clip(np.rint(y[nz]), -127, 127).astype(np.int8)
    return codes, s32


def encode_rows(C, fmt):
    """Store fp64 coefficients in format `fmt` (reading 4 / 5).

    Returns (rows, scales): rows float32 for F32, uint16 bf16 patterns for
    BF16, int8 codes for I8; scales float32 for I8 else None.
    """
    if fmt in (F32, PNG):
        return np.asarray(C, dtype=np.float64).astype(np.float32), None
    if fmt == BF16:
        return f32_to_bf16_bits(np.asarray(C, dtype=np.float64).astype(np.float32)), None
    if fmt == I8:
        return quantize_rows(C)
    raise ValueError(f"unknown format {fmt!r}")


def encode(x, R, S, fmt):
    """Archive a (…, T, D) sequence: complete blocks encoded, tail kept raw.

    cache.py ``append``/``_archive``: the first (T // R) * R tokens are
    compressed block by block; the last T mod R tokens stay verbatim.
    Returns dict(rows, scales, tail, n_blocks) with tail the raw values as
    fp64 (..., T mod R, D).
    """
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[-2]
    n = T // R
    rows, scales = encode_rows(project_blocks(x, R, S, fmt), fmt)
    return dict(fmt=fmt, R=R, S=S, rows=rows, scales=scales,
                tail=x[..., n * R:, :].copy(), n_blocks=n)


# ---------------------------------------------------------------------------
# decode (materialise) and attention
# ---------------------------------------------------------------------------
def dequantize(rows, scales, fmt):
    """fp64 coefficient rows from their stored form (reading 6)."""
    if fmt in (F32, PNG):
        return np.asarray(rows, dtype=np.float32).astype(np.float64)
    if fmt == BF16:
        return bf16_bits_to_f64(rows)
    if fmt == I8:
        return np.asarray(rows, dtype=np.int8).astype(np.float64) * \
            np.asarray(scales, dtype=np.float32).astype(np.float64)[..., None]
    raise ValueError(f"unknown format {fmt!r}")


def reconstruct(C, R, fmt=F32):
    """Synthesis X_hat = A C per block: A = M32^T for the DCT formats
    (README "Math": X_hat = M^T C), the cumulative sum for PNG mode.

    C: (..., n, S, D) fp64 -> (..., n * R, D) fp64, with
    X_hat[..., n*R + i, :] = sum_j A[i, j] * C[..., n, j, :].
    """
    C = np.asarray(C, dtype=np.float64)
    *lead, n, S, D = C.shape
    A = synthesis(R, S, fmt)
    X = np.zeros((*lead, n, R, D), dtype=np.float64)
    for i in range(R):
        for j in range(S):
            X[..., i, :] += A[i, j] * C[..., j, :]
    return X.reshape(*lead, n * R, D)


def materialise(archive):
    """Full (..., n*R + t, D) fp64 view: reconstructed blocks then raw tail."""
    C = dequantize(archive["rows"], archive["scales"], archive["fmt"])
    X = reconstruct(C, archive["R"], archive["fmt"])
    return np.concatenate([X, np.asarray(archive["tail"], dtype=np.float64)], axis=-2)


def round_to(x, fmt):
    """fp64 values rounded to a stored float format: float32 array for F32,
    uint16 bf16 patterns (of the fp32 rounding) for BF16 (reading 4)."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if fmt == F32:
        return x32
    if fmt == BF16:
        return f32_to_bf16_bits(x32)
    raise ValueError(f"view format must be f32 or bf16, not {fmt!r}")


def view(archive, out_fmt, block_begin=0):
    """The reconstructed (materialised) view in a float format.

    cache.py ``_CodecStream.read``: the archived blocks decoded (X_hat =
    M^T C, ``reconstruct`` above: products of the fp32 basis and the
    dequantised rows in fp64, summed over j = 0..S-1 from +0.0), restored to
    the stream's dtype, then the raw tail.  ``_decode_pending`` decodes only
    blocks archived since the last read; ``block_begin`` selects that range:
    the result covers tokens block_begin*R .. n*R + t - 1.  Rounding fp64 ->
    out_fmt follows reading 4 (bf16 through fp32).
    """
    R = archive["R"]
    n = archive["n_blocks"]
    rows = archive["rows"][..., block_begin:n, :, :]
    scales = None if archive["scales"] is None else archive["scales"][..., block_begin:n, :]
    X = reconstruct(dequantize(rows, scales, archive["fmt"]), R, archive["fmt"])
    X = np.concatenate([X, np.asarray(archive["tail"], dtype=np.float64)], axis=-2)
    return round_to(X, out_fmt)


def crop(archive, new_len, raw_fmt):
    """Remove trailing tokens exactly (cache.py ``_CodecStream.crop``).

    With keep = new_len, keep_blocks = keep // R and t = keep mod R:
    archived blocks below keep_blocks stay verbatim (never re-compressed);
    when the cut falls inside the archive, the block at the boundary leaves
    it and its first t tokens become the raw tail, taken from the decoded
    view in the stream's dtype (raw_fmt); when it falls inside the raw tail,
    the tail is truncated.  Returns a new archive dict (tail as fp64 values).
    """
    R = archive["R"]
    n = archive["n_blocks"]
    t_old = archive["tail"].shape[-2]
    if not (0 <= new_len <= n * R + t_old):
        raise ValueError("crop keeps between 0 and all tokens")
    kb, t = divmod(new_len, R)
    out = dict(archive)
    if kb < n:
        blk = dict(archive)
        blk["rows"] = archive["rows"][..., kb:kb + 1, :, :]
        blk["scales"] = None if archive["scales"] is None else archive["scales"][..., kb:kb + 1, :]
        blk["n_blocks"] = 1
        blk["tail"] = archive["tail"][..., :0, :]
        v = view(blk, raw_fmt)[..., :t, :]
        tail = v.astype(np.float64) if raw_fmt == F32 else bf16_bits_to_f64(v)
        out["rows"] = archive["rows"][..., :kb, :, :].copy()
        out["scales"] = None if archive["scales"] is None else archive["scales"][..., :kb, :].copy()
        out["n_blocks"] = kb
        out["tail"] = tail
    else:
        out["tail"] = np.asarray(archive["tail"], dtype=np.float64)[..., :t, :].copy()
    return out


def select_batch(archive, idx):
    """Gather batch rows (cache.py ``_CodecStream.select_batch``, beam
    reorder): row i of the result is row idx[i] of the archive, for the
    archived rows, their scales and the raw tail alike."""
    idx = np.asarray(idx, dtype=np.int64)
    out = dict(archive)
    out["rows"] = archive["rows"][idx].copy()
    out["scales"] = None if archive["scales"] is None else archive["scales"][idx].copy()
    out["tail"] = np.asarray(archive["tail"])[idx].copy()
    return out


def attention(q, K, V, scale):
    """Single-query softmax attention, fp64, GQA by hq // G.

    q: (B, Hq, D); K, V: (B, Hkv, T, D).  Returns (B, Hq, D).
    z_t = scale * q . K_t ;  p = exp(z - max z) / sum ;  out = sum_t p_t V_t.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv, T = K.shape[1], K.shape[2]
    if T == 0:
        raise ValueError("nothing to attend: T = 0")
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    out = np.empty((B, Hq, D), dtype=np.float64)
    for b in range(B):
        for hq in range(Hq):
            h = hq // G
            z = scale * (K[b, h] @ q[b, hq])
            p = np.exp(z - z.max())
            out[b, hq] = (p @ V[b, h]) / p.sum()
    return out


def decode_attention(q, k_archive, v_archive, scale=None):
    """Decode attention over a compressed K/V archive (materialised).

    q: (B, Hq, D) (a (B, Hq, 1, D) query is accepted too).  Default scale is
    D ** -0.5, as in the Triton host wrapper.
    """
    q = np.asarray(q, dtype=np.float64)
    if q.ndim == 4:
        q = q[:, :, 0, :]
    if scale is None:
        scale = q.shape[-1] ** -0.5
    return attention(q, materialise(k_archive), materialise(v_archive), scale)


def decode_attention_heads(q, k_archive, v_archive, scale, pairs):
    """Same as ``decode_attention`` but only for the listed (b, hq) pairs.

    Materialises one kv head at a time so full-size archives can be sampled
    without building every head.  Returns {(b, hq): out (D,)}.
    """
    q = np.asarray(q, dtype=np.float64)
    if q.ndim == 4:
        q = q[:, :, 0, :]
    Hq = q.shape[1]
    Hkv = k_archive["rows"].shape[1]
    G = Hq // Hkv
    res = {}
    cache = {}
    for (b, hq) in pairs:
        h = hq // G
        if (b, h) not in cache:
            cache.clear()
            cache[(b, h)] = tuple(materialise(_head(a, b, h)) for a in (k_archive, v_archive))
        K, V = cache[(b, h)]
        res[(b, hq)] = attention(q[b:b + 1, hq:hq + 1], K[None, None], V[None, None], scale)[0, 0]
    return res


def _head(archive, b, h):
    out = dict(archive)
    out["rows"] = archive["rows"][b, h]
    out["scales"] = None if archive["scales"] is None else archive["scales"][b, h]
    out["tail"] = archive["tail"][b, h]
    return out


# ---------------------------------------------------------------------------
# the pages' coefficient-domain algorithm, split over block ranges
# ---------------------------------------------------------------------------
def decode_attention_split(q, k_archive, v_archive, scale=None, ns=1):
    """Decode attention computed the way the pages compute it, in fp64.

    README "Materialization-free decode attention" and triton_attention.py:
    the blocks of each (b, kv head) are cut into ns consecutive ranges of
    chunk = ceil(n / ns) blocks (the split kernel's grid); within a range,
    block by block, s = rows . q (rows dequantised, reading 6), the R
    logits z = scale * A s (A = the synthesis matrix), an online-softmax
    update of the running (max m, sum l, accumulator acc) with
    alpha = exp(m_old - m_new), the weights w = p A and acc += w . rows;
    the last range also takes the raw tail tokens one by one.  A combine then
    merges the ranges (the combine kernel): M = max m_i over ranges with
    l_i > 0, L = sum l_i exp(m_i - M), out = sum acc_i exp(m_i - M) / L.
    Ranges left empty (ns > n) contribute nothing.  Nothing is ever
    reconstructed, so agreement with ``decode_attention`` (which
    materialises) is the identity the README states.
    q: (B, Hq, D) or (B, Hq, 1, D).  Returns (B, Hq, D).
    """
    q = np.asarray(q, dtype=np.float64)
    if q.ndim == 4:
        q = q[:, :, 0, :]
    B, Hq, D = q.shape
    if scale is None:
        scale = D ** -0.5
    R, fmt = k_archive["R"], k_archive["fmt"]
    S = k_archive["S"]
    A = synthesis(R, S, fmt)                                   # R x S
    Kc = dequantize(k_archive["rows"], k_archive["scales"], k_archive["fmt"])
    Vc = dequantize(v_archive["rows"], v_archive["scales"], v_archive["fmt"])
    Kt = np.asarray(k_archive["tail"], dtype=np.float64)
    Vt = np.asarray(v_archive["tail"], dtype=np.float64)
    Hkv = Kc.shape[1]
    G = Hq // Hkv
    n = k_archive["n_blocks"]
    if n + Kt.shape[-2] == 0:
        raise ValueError("nothing to attend: T = 0")
    chunk = -(-n // ns) if n else 0
    out = np.empty((B, Hq, D), dtype=np.float64)
    for b in range(B):
        for hq in range(Hq):
            h = hq // G
            qv = q[b, hq]
            parts = []
            for sid in range(ns):
                m, l, acc = -np.inf, 0.0, np.zeros(D)

                def update(z, w_of_p, rows):
                    nonlocal m, l, acc
                    m_new = max(m, float(z.max()))
                    alpha = math.exp(m - m_new) if m > -np.inf else 0.0
                    p = np.exp(z - m_new)
                    l = l * alpha + p.sum()
                    acc = acc * alpha + w_of_p(p) @ rows
                    m = m_new

                lo, hi = sid * chunk, min((sid + 1) * chunk, n)
                for blk in range(lo, hi):
                    sj = Kc[b, h, blk] @ qv                      # (S,)
                    z = scale * (A @ sj)                         # (R,)
                    update(z, lambda p: p @ A, Vc[b, h, blk])    # w = p A (S,)
                if sid == ns - 1:
                    for t in range(Kt.shape[-2]):
                        z = np.array([scale * (Kt[b, h, t] @ qv)])
                        update(z, lambda p: p, Vt[b, h, t:t + 1])
                parts.append((m, l, acc))
            live = [(m, l, a) for (m, l, a) in parts if l > 0.0]
            M = max(m for (m, _, _) in live)
            L = sum(l * math.exp(m - M) for (m, l, _) in live)
            out[b, hq] = sum(a * math.exp(m - M) for (m, _, a) in live) / L
    return out


# ---------------------------------------------------------------------------
# streaming (append with automatic archiving at block boundaries)
# ---------------------------------------------------------------------------
class Stream:
    """One K or V stream: a growing archive of complete blocks + a raw tail.

    cache.py ``_CodecStream.append``: new tokens are concatenated onto the
    raw tail, every complete block is archived, the remainder stays raw.
    Archived entries are never rewritten (README "Causal-safety design").
    """

    def __init__(self, R, S, fmt):
        self.R, self.S, self.fmt = R, S, fmt
        self.rows = []      # list of (..., S, D) per archived block
        self.scales = []
        self.tail = None    # (..., t, D) fp64

    def append(self, tokens):
        tokens = np.asarray(tokens, dtype=np.float64)
        buf = tokens if self.tail is None else np.concatenate([self.tail, tokens], axis=-2)
        n_full = buf.shape[-2] // self.R
        if n_full:
            rows, scales = encode_rows(project_blocks(buf[..., : n_full * self.R, :], self.R, self.S, self.fmt),
                                       self.fmt)
            for k in range(n_full):
                self.rows.append(rows[..., k, :, :])
                self.scales.append(None if scales is None else scales[..., k, :])
        self.tail = buf[..., n_full * self.R:, :]

    @property
    def n_blocks(self):
        return len(self.rows)

    def archive(self):
        """Snapshot in the same dict form as ``encode``."""
        lead = self.tail.shape[:-2]
        D = self.tail.shape[-1]
        if self.rows:
            rows = np.stack(self.rows, axis=-3)
            scales = np.stack(self.scales, axis=-2) if self.fmt == I8 else None
        else:
            dt = {F32: np.float32, BF16: np.uint16, I8: np.int8, PNG: np.float32}[self.fmt]
            rows = np.zeros((*lead, 0, self.S, D), dtype=dt)
            scales = np.zeros((*lead, 0, self.S), dtype=np.float32) if self.fmt == I8 else None
        return dict(fmt=self.fmt, R=self.R, S=self.S, rows=rows, scales=scales,
                    tail=self.tail.copy(), n_blocks=len(self.rows))


def storage_bytes(n_blocks, S, D, fmt, tail_tokens, tail_elem_bytes):
    """Logical bytes of one (b, h) stream: archived rows (+ scales) + tail.

    cache.py ``storage_bytes``: valid archive region plus the raw tail.
    """
    row_b = {F32: 4, BF16: 2, I8: 1, PNG: 4}[fmt]
    return n_blocks * S * (D * row_b + (4 if fmt == I8 else 0)) + tail_tokens * D * tail_elem_bytes
