"""ctypes binding of libcdattn.so (argument marshalling only).

Every step of the path runs in the library's HIP kernels; this module turns
torch tensors into pointers and strides, keeps the two host-side counters of
each stream, and grows archives by capacity doubling (start at 16 blocks,
double when full), the policy of cache.py ``_CodecStream._grow``.  PyTorch
is used only to allocate device memory and to name the current HIP stream.
"""

import ctypes
import math
import os

import torch

FMT_F32, FMT_BF16, FMT_I8, FMT_PNG = 0, 1, 2, 3
_FMT_NAMES = {"f32": FMT_F32, "bf16": FMT_BF16, "i8": FMT_I8, "png": FMT_PNG}
_TORCH_DTYPE = {FMT_F32: torch.float32, FMT_BF16: torch.bfloat16, FMT_I8: torch.int8, FMT_PNG: torch.float32}
_ELEM_BYTES = {FMT_F32: 4, FMT_BF16: 2, FMT_I8: 1, FMT_PNG: 4}
INITIAL_BLOCKS = 16

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def library_path():
    """libcdattn.so beside this file, or the library CDATTN_LIBRARY names
    (the measurement build, compressed_domain_attention_amd/timeline/)."""
    return os.environ.get("CDATTN_LIBRARY") or os.path.join(_HERE, "libcdattn.so")


class CodecError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        msg = _lib().codec_status_string(status).decode() if _LIB is not None else str(status)
        super().__init__(f"{what}: {msg} (status {status})")


class _Stream(ctypes.Structure):
    _fields_ = [
        ("block", ctypes.c_int32), ("keep", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("fmt", ctypes.c_int32), ("raw_dtype", ctypes.c_int32), ("n_tail", ctypes.c_int32),
        ("batch", ctypes.c_int64), ("heads", ctypes.c_int64), ("capacity", ctypes.c_int64),
        ("n_blocks", ctypes.c_int64),
        ("rows", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("tail", ctypes.c_void_p),
    ]


_I64_2 = ctypes.c_int64 * 2
_I64_3 = ctypes.c_int64 * 3


def _lib():
    """Load libcdattn.so once; raise if it has not been built."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build the HIP library first "
                               "(python -m compressed_domain_attention_amd.build)")
        lib = ctypes.CDLL(path)
        P = ctypes.POINTER(_Stream)
        vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        lib.codec_basis.argtypes = [i32, i32, ctypes.POINTER(ctypes.c_float)]
        LP = ctypes.POINTER(ctypes.c_int64)
        lib.codec_encode_blocks.argtypes = [P, vp, LP, i64, vp]
        lib.codec_append_step.argtypes = [P, P, vp, LP, vp, LP, vp]
        lib.codec_decode_workspace_bytes.argtypes = [P, P, i64, ctypes.POINTER(ctypes.c_size_t)]
        lib.codec_decode_attention.argtypes = [vp, LP, i64, P, P, f32, vp, LP, i32,
                                               vp, ctypes.c_size_t, vp]
        lib.codec_decode_attention_append.argtypes = [vp, LP, i64, P, P, vp, LP, vp, LP, f32, vp, LP, i32,
                                                      vp, ctypes.c_size_t, vp]
        lib.codec_decode_attention_noalloc.argtypes = [vp, LP, i64, P, P, f32, vp, LP, i32, vp]
        lib.codec_materialise.argtypes = [P, i64, vp, LP, i32, vp]
        lib.codec_crop.argtypes = [P, i64, vp]
        lib.codec_select_batch.argtypes = [P, P, LP, i64, vp]
        lib.codec_measure_read.argtypes = [vp, ctypes.c_size_t, vp, i32, vp]
        lib.codec_measure_read.restype = ctypes.c_int
        lib.codec_status_string.argtypes = [ctypes.c_int]
        lib.codec_status_string.restype = ctypes.c_char_p
        for name in ("codec_basis", "codec_encode_blocks", "codec_append_step",
                     "codec_decode_workspace_bytes", "codec_decode_attention",
                     "codec_materialise", "codec_crop", "codec_select_batch", "codec_decode_attention_append",
                     "codec_decode_attention_noalloc"):
            getattr(lib, name).restype = ctypes.c_int
        _LIB = lib
    return _LIB


def library():
    """The loaded ctypes library (loads it on first use)."""
    return _lib()


def timeline_set(buf):
    """Measurement builds only: decode launches write per-wave phase stamps
    (uint64, 100 MHz clock) into `buf`, a device tensor; None stops them."""
    lib = _lib()
    if not hasattr(lib, "codec_timeline_set"):
        raise RuntimeError(f"{library_path()} is not a timeline build (python -m "
                           "compressed_domain_attention_amd.build --timeline)")
    lib.codec_timeline_set.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    lib.codec_timeline_set.restype = ctypes.c_int
    if buf is None:
        return lib.codec_timeline_set(None, 0)
    return lib.codec_timeline_set(buf.data_ptr(), buf.numel() * buf.element_size())


def _check(status, what):
    if status != 0:
        raise CodecError(status, what)


def _fmt(f):
    if isinstance(f, str):
        return _FMT_NAMES[f]
    return int(f)


def _hip_stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def basis(R, S):
    """A (R x S) fp32 synthesis matrix as a CPU tensor (A[i, j] = M[j, i])."""
    A = (ctypes.c_float * (R * S))()
    _check(_lib().codec_basis(R, S, A), "codec_basis")
    return torch.tensor(list(A), dtype=torch.float32).reshape(R, S)


class CodecStream:
    """A compressed key or value stream in device memory.

    Holds rows (B, H, capacity, S, D), scales (B, H, capacity, S) for int8,
    and the raw tail (B, H, R, D).  ``n_blocks`` / ``n_tail`` mirror the
    library's counters.
    """

    def __init__(self, B, H, D, R, S, fmt="i8", raw_dtype="bf16", device="cuda", capacity=0):
        self.B, self.H, self.D, self.R, self.S = int(B), int(H), int(D), int(R), int(S)
        self.fmt, self.raw_dtype = _fmt(fmt), _fmt(raw_dtype)
        self.device = torch.device(device)
        self.n_blocks, self.n_tail = 0, 0
        self.capacity = 0
        self.rows = self.scales = None
        self.tail = torch.zeros((self.B, self.H, self.R, self.D), dtype=_TORCH_DTYPE[self.raw_dtype],
                                device=self.device)
        self._grow(max(int(capacity), INITIAL_BLOCKS))
        self.discard_view()

    # cache.py ``_CodecStream._grow``: start at 16 blocks and double until the
    # request fits; archived blocks are copied over verbatim.
    def _grow(self, need):
        if need <= self.capacity:
            return
        cap = max(INITIAL_BLOCKS, self.capacity)
        while cap < need:
            cap *= 2
        rows = torch.empty((self.B, self.H, cap, self.S, self.D), dtype=_TORCH_DTYPE[self.fmt],
                           device=self.device)
        scales = (torch.empty((self.B, self.H, cap, self.S), dtype=torch.float32, device=self.device)
                  if self.fmt == FMT_I8 else None)
        if self.n_blocks:
            rows[:, :, :self.n_blocks].copy_(self.rows[:, :, :self.n_blocks])
            if scales is not None:
                scales[:, :, :self.n_blocks].copy_(self.scales[:, :, :self.n_blocks])
        self.rows, self.scales, self.capacity = rows, scales, cap

    def _desc(self):
        d = _Stream()
        d.block, d.keep, d.head_dim = self.R, self.S, self.D
        d.fmt, d.raw_dtype, d.n_tail = self.fmt, self.raw_dtype, self.n_tail
        d.batch, d.heads, d.capacity, d.n_blocks = self.B, self.H, self.capacity, self.n_blocks
        d.rows = self.rows.data_ptr()
        d.scales = self.scales.data_ptr() if self.scales is not None else None
        d.tail = self.tail.data_ptr()
        return d

    def _sync(self, d):
        self.n_blocks, self.n_tail = int(d.n_blocks), int(d.n_tail)

    @property
    def seq_len(self):
        return self.n_blocks * self.R + self.n_tail

    def storage_bytes(self):
        """Logical bytes: valid archive region (+ scales) and the raw tail
        (cache.py ``storage_bytes``; spare capacity is not counted)."""
        per_block = self.S * self.D * _ELEM_BYTES[self.fmt] + (4 * self.S if self.fmt == FMT_I8 else 0)
        return self.B * self.H * (self.n_blocks * per_block + self.n_tail * self.D * _ELEM_BYTES[self.raw_dtype])

    def encode(self, x, stream=None):
        """Archive a (B, H, T, D) run of raw tokens; the tail must be empty."""
        return encode_blocks(self, x, stream)

    # ---- the materialised view (cache.py ``read`` / ``_decode_pending``)
    def discard_view(self):
        """Drop the memoised view (rebuilt on the next ``read``)."""
        self._rec, self._rec_blocks, self._rec_cap = None, 0, 0

    def read(self, dtype=None, stream=None):
        """The decoded (B, H, seq_len, D) view in the raw dtype (or `dtype`).

        Memoised and append-only: only blocks archived since the last read
        are decoded (codec_materialise from the memo's block count), then the
        raw tail is written after them.  The archived prefix of a returned
        tensor never changes; its last n_tail tokens are rewritten by later
        reads once more tokens arrive.
        """
        fmt = self.raw_dtype if dtype is None else _fmt(dtype)
        tdt = _TORCH_DTYPE[fmt]
        if self._rec is not None and self._rec.dtype != tdt:
            self.discard_view()
        need = self.seq_len
        if self._rec is None or self._rec_cap < need:
            cap = max(need, 2 * self._rec_cap, INITIAL_BLOCKS * self.R)
            new = torch.empty((self.B, self.H, cap, self.D), dtype=tdt, device=self.device)
            done = self._rec_blocks * self.R
            if self._rec is not None and done:
                new[:, :, :done].copy_(self._rec[:, :, :done])
            self._rec, self._rec_cap = new, cap
        materialise(self, self._rec, block_begin=self._rec_blocks, stream=stream)
        self._rec_blocks = self.n_blocks
        return self._rec[:, :, :need]

    def crop(self, new_len, stream=None):
        """Keep the first new_len tokens exactly (codec_crop)."""
        crop(self, new_len, stream)

    def select_batch(self, idx, stream=None):
        """Gather batch rows idx (beam reorder) into new buffers (codec_select_batch)."""
        select_batch(self, idx, stream)



class _LayerView(CodecStream):
    """Layer l of a CodecLayerStack's key or value archive: batch rows
    [l B, (l + 1) B) of the stack's stream, with this layer's own counters.
    Rows, scales and tail are slices of the stack's tensors, looked up at each
    use (the stack reallocates them when it grows), so every per-stream call
    (encode, append, decode, view, crop) works on one layer alone."""

    def __init__(self, parent, stack, layer):
        self._parent, self._stack, self._layer = parent, stack, layer
        self.H, self.D, self.R, self.S = parent.H, parent.D, parent.R, parent.S
        self.fmt, self.raw_dtype, self.device = parent.fmt, parent.raw_dtype, parent.device
        self.n_blocks, self.n_tail = 0, 0
        self.discard_view()

    @property
    def B(self):
        return self._stack.B

    def _slice(self, t):
        return None if t is None else t[self._layer * self.B:(self._layer + 1) * self.B]

    @property
    def rows(self):
        return self._slice(self._parent.rows)

    @property
    def scales(self):
        return self._slice(self._parent.scales)

    @property
    def tail(self):
        return self._slice(self._parent.tail)

    @property
    def capacity(self):
        return self._parent.capacity

    def _grow(self, need):
        self._stack._grow(need)

    def select_batch(self, idx, stream=None):
        raise ValueError("a layer's batch rows are reordered for every layer at once (CodecLayerStack.select_batch)")


class CodecLayerStack:
    """The key and value archives of L layers in one allocation: one stream
    per side whose batch axis is (layer, batch row), i.e. rows
    (L * B, H, capacity, S, D), scales (L * B, H, capacity, S) and tails
    (L * B, H, R, D), all layers at one capacity.

    ``layer(l)`` gives layer l's key and value streams (slices with their own
    counters) for models that run layer by layer.  When every layer is at the
    same length, the stack-wide calls do one step for all layers in one
    launch: ``decode`` (split-K decode with the combine in the same launch,
    for all L x B x Hkv pairs), ``decode_append`` (the step's tokens of all
    layers appended, then the decode, in one launch unless the token completes
    a block), ``append``, ``encode`` (prefill), ``crop`` and
    ``select_batch`` (the same beam reorder in every layer).  Queries, tokens
    and outputs of the stack-wide calls are (L, B, heads, 1 or T, D).
    flashcodec-kv README, end-to-end decode paragraph: the remaining gap is
    the per-layer launch pair, which one launch per step across layers
    removes.
    """

    def __init__(self, L, B, H, D, R, S, k_fmt="i8", v_fmt=None, raw_dtype="bf16", device="cuda", capacity=0):
        if int(L) < 1 or int(B) < 1:
            raise ValueError("a layer stack needs L >= 1 layers of B >= 1 batch rows")
        self.L, self.B = int(L), int(B)
        self.k = CodecStream(self.L * self.B, H, D, R, S, fmt=k_fmt, raw_dtype=raw_dtype, device=device,
                             capacity=capacity)
        self.v = CodecStream(self.L * self.B, H, D, R, S, fmt=v_fmt if v_fmt is not None else k_fmt,
                             raw_dtype=raw_dtype, device=device, capacity=capacity)
        self._layers = [(_LayerView(self.k, self, l), _LayerView(self.v, self, l)) for l in range(self.L)]

    def layer(self, l):
        """Layer l's (key stream, value stream)."""
        return self._layers[l]

    @property
    def capacity(self):
        return self.k.capacity

    @property
    def seq_len(self):
        return self._common()[0] * self.k.R + self._common()[1]

    def _grow(self, need):
        # capacity doubling for all layers at once; every layer's archived
        # blocks are copied over (the stack copies the longest layer's count)
        for p, side in ((self.k, 0), (self.v, 1)):
            p.n_blocks = max(lay[side].n_blocks for lay in self._layers)
            p._grow(need)

    def _common(self):
        counts = {(s.n_blocks, s.n_tail) for lay in self._layers for s in lay}
        if len(counts) != 1:
            raise ValueError(f"stack-wide calls need every layer at the same length; layers hold {sorted(counts)}")
        return counts.pop()

    def _enter(self):
        nb, nt = self._common()
        for p in (self.k, self.v):
            p.n_blocks, p.n_tail = nb, nt

    def _leave(self):
        for lay in self._layers:
            for s, p in zip(lay, (self.k, self.v)):
                s.n_blocks, s.n_tail = p.n_blocks, p.n_tail
                s._rec_blocks = min(s._rec_blocks, s.n_blocks)

    def _flat(self, t, what):
        if t.dim() != 5 or t.shape[0] != self.L or t.shape[1] != self.B:
            raise ValueError(f"{what} must be (L, B, heads, tokens, D) = ({self.L}, {self.B}, ...)")
        try:
            return t.view(self.L * self.B, *t.shape[2:])
        except RuntimeError:
            raise ValueError(f"{what}: the (layer, batch) axes must fold into one (a view, no copy)") from None

    def encode(self, k, v, stream=None):
        """Prefill every layer: k, v (L, B, H, T, D); every tail must be empty."""
        kf, vf = self._flat(k, "k"), self._flat(v, "v")
        self._enter()
        try:
            encode_blocks(self.k, kf, stream)
            encode_blocks(self.v, vf, stream)
        finally:
            self._leave()   # a failed value encode leaves K ahead of V: stack-wide calls then refuse

    def append(self, k_new, v_new, stream=None):
        """One token per layer: k_new, v_new (L, B, H, 1, D)."""
        kf, vf = self._flat(k_new, "k_new"), self._flat(v_new, "v_new")
        self._enter()
        try:
            append_step(self.k, self.v, kf, vf, stream)
        finally:
            self._leave()

    def decode(self, q, scale=None, out=None, out_dtype=torch.float32, workspace=None, stream=None):
        """Decode attention of every layer in one launch: q (L, B, Hq, 1, D)
        bf16; returns out (L, B, Hq, 1, D)."""
        self._enter()
        qf = self._flat(q, "q")
        of = None if out is None else self._flat(out, "out")
        of = decode_attention(qf, self.k, self.v, scale, of, out_dtype, workspace, stream)
        return of.view(self.L, self.B, *of.shape[1:])

    def decode_append(self, q, k_new, v_new, scale=None, out=None, out_dtype=torch.float32, workspace=None,
                      stream=None):
        """``append`` then ``decode`` for all layers (codec_decode_attention_append
        on the stack: one launch unless the token completes a block)."""
        self._enter()
        qf = self._flat(q, "q")
        of = None if out is None else self._flat(out, "out")
        try:
            of = decode_attention_append(qf, self.k, self.v, self._flat(k_new, "k_new"),
                                         self._flat(v_new, "v_new"), scale, of, out_dtype, workspace, stream)
        finally:
            self._leave()
        return of.view(self.L, self.B, *of.shape[1:])

    def crop(self, new_len, stream=None):
        """Keep the first new_len tokens of every layer (codec_crop on the stack)."""
        self._enter()
        try:
            crop(self.k, new_len, stream)
            crop(self.v, new_len, stream)
        finally:
            self._leave()

    def select_batch(self, idx, stream=None):
        """Batch row i of every layer becomes its old row idx[i] (beam
        reorder; new buffers, one gather launch per side for all layers)."""
        idx = [int(i) for i in (idx.tolist() if hasattr(idx, "tolist") else idx)]
        if not idx:
            raise ValueError("a beam reorder keeps at least one batch row")
        if any(i < 0 or i >= self.B for i in idx):
            raise ValueError(f"batch index out of range [0, {self.B})")
        self._enter()
        flat = [l * self.B + i for l in range(self.L) for i in idx]
        select_batch(self.k, flat, stream)
        select_batch(self.v, flat, stream)
        self.B = len(idx)
        self._leave()
        for lay in self._layers:
            for s in lay:
                s.discard_view()


def encode_blocks(s, x, stream=None):
    if x.dtype != _TORCH_DTYPE[s.raw_dtype] or x.dim() != 4 or x.stride(3) != 1:
        raise ValueError("x must be (B, H, T, D) of the stream's raw dtype with unit d stride")
    T = x.shape[2]
    s._grow(s.n_blocks + T // s.R)
    d = s._desc()
    st = _hip_stream(s.device) if stream is None else ctypes.c_void_p(stream)
    _check(_lib().codec_encode_blocks(ctypes.byref(d), ctypes.c_void_p(x.data_ptr()),
                                      _I64_3(x.stride(0), x.stride(1), x.stride(2)), T, st),
           "codec_encode_blocks")
    s._sync(d)


def append_step(k, v, k_new, v_new, stream=None):
    """Append one token (B, H, 1, D) to both streams (archives at block ends)."""
    for s, t in ((k, k_new), (v, v_new)):
        if t.dtype != _TORCH_DTYPE[s.raw_dtype] or t.dim() != 4 or t.stride(3) != 1:
            raise ValueError("new token must be (B, H, 1, D) of the raw dtype with unit d stride")
    if k.n_tail + 1 == k.R:
        k._grow(k.n_blocks + 1)
        v._grow(v.n_blocks + 1)
    dk, dv = k._desc(), v._desc()
    st = _hip_stream(k.device) if stream is None else ctypes.c_void_p(stream)
    _check(_lib().codec_append_step(ctypes.byref(dk), ctypes.byref(dv),
                                    ctypes.c_void_p(k_new.data_ptr()), _I64_2(k_new.stride(0), k_new.stride(1)),
                                    ctypes.c_void_p(v_new.data_ptr()), _I64_2(v_new.stride(0), v_new.stride(1)),
                                    st), "codec_append_step")
    k._sync(dk)
    v._sync(dv)


def materialise(s, dst, block_begin=0, stream=None):
    """Decode blocks block_begin.. of s into dst (B, H, >= seq_len, D) and
    write the raw tail after them (codec_materialise)."""
    if dst.dim() != 4 or dst.stride(3) != 1 or dst.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("dst must be (B, H, T, D) float32 / bfloat16 with unit d stride")
    fmt = FMT_F32 if dst.dtype == torch.float32 else FMT_BF16
    d = s._desc()
    st = _hip_stream(s.device) if stream is None else ctypes.c_void_p(stream)
    _check(_lib().codec_materialise(ctypes.byref(d), int(block_begin), ctypes.c_void_p(dst.data_ptr()),
                                    _I64_3(dst.stride(0), dst.stride(1), dst.stride(2)), fmt, st),
           "codec_materialise")
    return dst


def crop(s, new_len, stream=None):
    d = s._desc()
    st = _hip_stream(s.device) if stream is None else ctypes.c_void_p(stream)
    _check(_lib().codec_crop(ctypes.byref(d), int(new_len), st), "codec_crop")
    s._sync(d)
    s._rec_blocks = min(s._rec_blocks, s.n_blocks)


def select_batch(s, idx, stream=None):
    """Batch row i of s becomes its old row idx[i]; new buffers are allocated
    (rows keep their capacity), the memoised view is dropped."""
    if isinstance(s, _LayerView):
        raise ValueError("a layer's batch rows are reordered for every layer at once (CodecLayerStack.select_batch)")
    idx = [int(i) for i in (idx.tolist() if hasattr(idx, "tolist") else idx)]
    n = len(idx)
    rows = torch.empty((n, s.H, s.capacity, s.S, s.D), dtype=_TORCH_DTYPE[s.fmt], device=s.device)
    scales = (torch.empty((n, s.H, s.capacity, s.S), dtype=torch.float32, device=s.device)
              if s.fmt == FMT_I8 else None)
    tail = torch.empty((n, s.H, s.R, s.D), dtype=_TORCH_DTYPE[s.raw_dtype], device=s.device)
    src = s._desc()
    dst = s._desc()
    dst.batch = n
    dst.rows = rows.data_ptr()
    dst.scales = scales.data_ptr() if scales is not None else None
    dst.tail = tail.data_ptr()
    ia = (ctypes.c_int64 * max(n, 1))(*idx)
    st = _hip_stream(s.device) if stream is None else ctypes.c_void_p(stream)
    _check(_lib().codec_select_batch(ctypes.byref(src), ctypes.byref(dst), ia, n, st), "codec_select_batch")
    s.B, s.rows, s.scales, s.tail = n, rows, scales, tail
    s._sync(dst)
    s.discard_view()


def decode_workspace_bytes(k, v, Hq):
    n = ctypes.c_size_t(0)
    _check(_lib().codec_decode_workspace_bytes(ctypes.byref(k._desc()), ctypes.byref(v._desc()),
                                               int(Hq), ctypes.byref(n)), "codec_decode_workspace_bytes")
    return int(n.value)


_WS_CACHE = {}


def _torch_stream(device, stream):
    """The torch stream object for a raw HIP stream handle (None: the
    current stream of `device`)."""
    if stream is None:
        return torch.cuda.current_stream(device)
    return torch.cuda.ExternalStream(int(stream), device=device)


def _workspace(nbytes, device, ts):
    """A zero-filled decode workspace for one (device, HIP stream), grown on
    demand and then reused: the kernels leave its arrival counters at zero
    after every call, so calls in order on one stream can share it.  The
    zero fill is enqueued on that stream, ahead of the kernel that first
    uses it, and the buffer belongs to that stream in torch's allocator, so a
    replaced buffer is not handed out again before the stream has passed
    the work already enqueued on it.  Calls on different streams get
    different workspaces (overlapping calls must not share arrival
    counters)."""
    key = (device.type, device.index, ts.cuda_stream)
    ws = _WS_CACHE.get(key)
    if ws is None or ws.numel() < nbytes:
        with torch.cuda.stream(ts):
            ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _WS_CACHE[key] = ws
    return ws


def decode_attention(q, k, v, scale=None, out=None, out_dtype=torch.float32, workspace=None, stream=None):
    """Decode attention of q (B, Hq, 1, D) bf16 over streams k, v.

    Default scale D ** -0.5 (the Triton wrapper's default).  Returns out
    (B, Hq, 1, D) in out_dtype (float32 or bfloat16).
    """
    if q.dtype != torch.bfloat16 or q.dim() != 4 or q.shape[2] != 1 or q.stride(3) != 1:
        raise ValueError("q must be (B, Hq, 1, D) bf16 with unit d stride")
    B, Hq, _, D = q.shape
    if scale is None:
        scale = D ** -0.5
    if out is None:
        out = torch.empty((B, Hq, 1, D), dtype=out_dtype, device=q.device)
    odt = {torch.float32: FMT_F32, torch.bfloat16: FMT_BF16}[out.dtype]
    dk, dv = k._desc(), v._desc()
    need = decode_workspace_bytes(k, v, Hq)
    ts = _torch_stream(q.device, stream)
    if workspace is None:
        workspace = _workspace(need, q.device, ts)
    st = ctypes.c_void_p(ts.cuda_stream)
    _check(_lib().codec_decode_attention(
        ctypes.c_void_p(q.data_ptr()), _I64_2(q.stride(0), q.stride(1)), Hq,
        ctypes.byref(dk), ctypes.byref(dv), ctypes.c_float(float(scale)),
        ctypes.c_void_p(out.data_ptr()), _I64_2(out.stride(0), out.stride(1)), odt,
        ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(), st),
        "codec_decode_attention")
    return out


def decode_attention_noalloc(q, k, v, scale=None, out=None, out_dtype=torch.float32, stream=None):
    """decode_attention without a workspace (codec_decode_attention_noalloc):
    the split partials live in the library's own per-GPU scratch array, so
    the call allocates nothing when `out` is given.  Calls that overlap on one
    GPU race on that array."""
    if q.dtype != torch.bfloat16 or q.dim() != 4 or q.shape[2] != 1 or q.stride(3) != 1:
        raise ValueError("q must be (B, Hq, 1, D) bf16 with unit d stride")
    B, Hq, _, D = q.shape
    if scale is None:
        scale = D ** -0.5
    if out is None:
        out = torch.empty((B, Hq, 1, D), dtype=out_dtype, device=q.device)
    odt = {torch.float32: FMT_F32, torch.bfloat16: FMT_BF16}[out.dtype]
    dk, dv = k._desc(), v._desc()
    st = ctypes.c_void_p(_torch_stream(q.device, stream).cuda_stream)
    _check(_lib().codec_decode_attention_noalloc(
        ctypes.c_void_p(q.data_ptr()), _I64_2(q.stride(0), q.stride(1)), Hq,
        ctypes.byref(dk), ctypes.byref(dv), ctypes.c_float(float(scale)),
        ctypes.c_void_p(out.data_ptr()), _I64_2(out.stride(0), out.stride(1)), odt, st),
        "codec_decode_attention_noalloc")
    return out


def decode_attention_append(q, k, v, k_new, v_new, scale=None, out=None, out_dtype=torch.float32, workspace=None,
                            stream=None):
    """append_step(k, v, k_new, v_new) then decode_attention(q, k, v) in one
    call (codec_decode_attention_append: one launch unless the token
    completes a block)."""
    if q.dtype != torch.bfloat16 or q.dim() != 4 or q.shape[2] != 1 or q.stride(3) != 1:
        raise ValueError("q must be (B, Hq, 1, D) bf16 with unit d stride")
    for s, t in ((k, k_new), (v, v_new)):
        if t.dtype != _TORCH_DTYPE[s.raw_dtype] or t.dim() != 4 or t.stride(3) != 1:
            raise ValueError("new token must be (B, H, 1, D) of the raw dtype with unit d stride")
    B, Hq, _, D = q.shape
    if scale is None:
        scale = D ** -0.5
    if out is None:
        out = torch.empty((B, Hq, 1, D), dtype=out_dtype, device=q.device)
    odt = {torch.float32: FMT_F32, torch.bfloat16: FMT_BF16}[out.dtype]
    if k.n_tail + 1 == k.R:
        k._grow(k.n_blocks + 1)
        v._grow(v.n_blocks + 1)
    dk, dv = k._desc(), v._desc()
    ts = _torch_stream(q.device, stream)
    if workspace is None:
        # sized for the streams as the append leaves them (the split plan
        # depends on the block count only)
        nb = k.n_blocks + (1 if k.n_tail + 1 == k.R else 0)
        dk2, dv2 = k._desc(), v._desc()
        dk2.n_blocks = dv2.n_blocks = nb
        dk2.n_tail = dv2.n_tail = (k.n_tail + 1) % k.R
        n = ctypes.c_size_t(0)
        _check(_lib().codec_decode_workspace_bytes(ctypes.byref(dk2), ctypes.byref(dv2), int(Hq), ctypes.byref(n)),
               "codec_decode_workspace_bytes")
        workspace = _workspace(int(n.value), q.device, ts)
    st = ctypes.c_void_p(ts.cuda_stream)
    _check(_lib().codec_decode_attention_append(
        ctypes.c_void_p(q.data_ptr()), _I64_2(q.stride(0), q.stride(1)), Hq,
        ctypes.byref(dk), ctypes.byref(dv),
        ctypes.c_void_p(k_new.data_ptr()), _I64_2(k_new.stride(0), k_new.stride(1)),
        ctypes.c_void_p(v_new.data_ptr()), _I64_2(v_new.stride(0), v_new.stride(1)),
        ctypes.c_float(float(scale)),
        ctypes.c_void_p(out.data_ptr()), _I64_2(out.stride(0), out.stride(1)), odt,
        ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(), st),
        "codec_decode_attention_append")
    k._sync(dk)
    v._sync(dv)
    return out


def measure_read(src, sink, workgroups, stream=None):
    """One streaming read of the whole of `src` (a device tensor, 16-byte
    aligned, size a multiple of 16 bytes) by `workgroups` workgroups
    (codec_measure_read; a measurement helper, not part of the method)."""
    st = ctypes.c_void_p(_torch_stream(src.device, stream).cuda_stream)
    _check(_lib().codec_measure_read(ctypes.c_void_p(src.data_ptr()), src.numel() * src.element_size(),
                                     ctypes.c_void_p(sink.data_ptr()), int(workgroups), st), "codec_measure_read")


def default_scale(D):
    return 1.0 / math.sqrt(D)
