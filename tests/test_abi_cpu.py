"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, the host-computed basis equals the oracle's bit for bit, and
every validation error is reported before any HIP call, leaving the stream
counters untouched.  Only calls that fail validation (or are pure host
functions) are made here.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
from compressed_domain_attention_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cdattn.h")

OK, NULL, SHAPE, FORMAT, CAPACITY, STATE, WORKSPACE, UNSUPPORTED, HIP, SCALE = range(10)

pytestmark = pytest.mark.skipif(not os.path.exists(bd.library_path()), reason="libcdattn.so not built")


@pytest.fixture(scope="module")
def lib():
    return bd.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^(?:int|size_t|const char \*)\s*\*?\s*(codec_\w+)\s*\(", text, flags=re.M)


def test_header_symbols_exported(lib):
    names = declared_functions()
    assert set(names) == {"codec_basis", "codec_encode_blocks", "codec_append_step",
                          "codec_decode_workspace_bytes", "codec_decode_attention", "codec_status_string",
                          "codec_materialise", "codec_crop", "codec_select_batch", "codec_decode_attention_append",
                          "codec_decode_attention_noalloc"}
    for n in names:
        assert hasattr(lib, n), n


def test_measure_header_symbols_and_checks(lib):
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "cdattn_measure.h")).read(), flags=re.S)
    names = re.findall(r"^int\s+(codec_\w+)\s*\(", text, flags=re.M)
    assert names == ["codec_measure_read", "codec_timeline_set"]
    assert hasattr(lib, "codec_measure_read")
    # the phase-stamp hook exists only in the measurement build
    assert not hasattr(lib, "codec_timeline_set")
    assert lib.codec_measure_read(None, 16, FAKE, 4, None) == NULL
    assert lib.codec_measure_read(FAKE, 16, None, 4, None) == NULL
    assert lib.codec_measure_read(FAKE + 8, 16, FAKE, 4, None) == SHAPE
    assert lib.codec_measure_read(FAKE, 24, FAKE, 4, None) == SHAPE
    assert lib.codec_measure_read(FAKE, 0, FAKE, 4, None) == SHAPE
    assert lib.codec_measure_read(FAKE, 16, FAKE, 0, None) == SHAPE


def test_status_strings(lib):
    seen = set()
    for s in range(10):
        t = lib.codec_status_string(s).decode()
        assert t and t not in seen
        seen.add(t)
    assert lib.codec_status_string(1234).decode() == "unknown status"


@pytest.mark.parametrize("R", [1, 2, 3, 5, 8, 12, 16, 31, 32])
def test_basis_bitwise_equals_oracle(lib, R):
    for S in range(1, R + 1):
        A = (ctypes.c_float * (R * S))()
        assert lib.codec_basis(R, S, A) == OK
        got = np.frombuffer(A, dtype=np.float32).reshape(R, S)
        want = O.dct_basis_f32(R, S).T
        assert got.tobytes() == np.ascontiguousarray(want).tobytes(), (R, S)


def test_basis_errors(lib):
    A = (ctypes.c_float * 1024)()
    assert lib.codec_basis(8, 2, None) == NULL
    assert lib.codec_basis(0, 1, A) == SHAPE
    assert lib.codec_basis(8, 9, A) == SHAPE
    assert lib.codec_basis(33, 2, A) == SHAPE
    assert lib.codec_basis(32, 33, A) == SHAPE


FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation


def stream(**kw):
    d = bd._Stream()
    d.block, d.keep, d.head_dim, d.fmt, d.raw_dtype, d.n_tail = 8, 2, 128, bd.FMT_I8, bd.FMT_BF16, 0
    d.batch, d.heads, d.capacity, d.n_blocks = 2, 4, 16, 0
    d.rows, d.scales, d.tail = FAKE, FAKE, FAKE
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def encode(lib, s, x=FAKE, strides=(4096, 1024, 128), T=40):
    return lib.codec_encode_blocks(ctypes.byref(s) if s is not None else None, x, bd._I64_3(*strides), T, None)


def test_encode_validation(lib):
    assert encode(lib, None) == NULL
    for kw, want in [({"block": 0}, SHAPE), ({"block": 33}, SHAPE), ({"keep": 9}, SHAPE), ({"keep": 33, "block": 32}, SHAPE),
                     ({"fmt": 7}, FORMAT), ({"raw_dtype": bd.FMT_I8}, FORMAT), ({"n_tail": 3}, STATE),
                     ({"n_tail": 8}, STATE), ({"capacity": 4}, CAPACITY), ({"head_dim": 100}, UNSUPPORTED),
                     ({"head_dim": 264}, UNSUPPORTED), ({"head_dim": 4}, UNSUPPORTED),
                     ({"head_dim": 0}, SHAPE), ({"batch": 0}, SHAPE), ({"tail": None}, NULL),
                     ({"rows": None}, NULL), ({"scales": None}, NULL), ({"tail": FAKE + 4}, SHAPE),
                     ({"n_blocks": 10, "capacity": 8}, CAPACITY)]:
        s = stream(**kw)
        before = (s.n_blocks, s.n_tail)
        assert encode(lib, s, T=200) == want, kw
        assert (s.n_blocks, s.n_tail) == before
    s = stream()
    assert encode(lib, s, x=None) == NULL
    assert encode(lib, s, T=-1) == SHAPE
    assert encode(lib, s, x=FAKE + 8) == SHAPE
    assert encode(lib, s, strides=(4096, 1024, 3)) == SHAPE
    assert lib.codec_encode_blocks(ctypes.byref(s), FAKE, None, 8, None) == NULL
    # 16 blocks fit, 17 do not
    assert encode(lib, stream(capacity=16), T=17 * 8) == CAPACITY
    # T == 0 is a no-op that succeeds without touching the GPU
    s = stream()
    assert encode(lib, s, T=0) == OK and (s.n_blocks, s.n_tail) == (0, 0)


def test_append_validation(lib):
    two = bd._I64_2(1024, 128)

    def app(k, v, kn=FAKE, vn=FAKE, ks=two, vs=two):
        return lib.codec_append_step(ctypes.byref(k), ctypes.byref(v), kn, ks, vn, vs, None)

    assert app(stream(), stream(head_dim=64)) == SHAPE
    assert app(stream(), stream(n_tail=1)) == SHAPE
    assert app(stream(), stream(n_blocks=1)) == SHAPE
    assert app(stream(), stream(), kn=None) == NULL
    assert app(stream(), stream(), vs=None) == NULL
    assert app(stream(), stream(), kn=FAKE + 2) == SHAPE
    assert app(stream(), stream(), ks=bd._I64_2(1024, 130)) == SHAPE
    # completing a block with a full archive
    k, v = stream(n_tail=7, n_blocks=16), stream(n_tail=7, n_blocks=16)
    assert app(k, v) == CAPACITY
    assert (k.n_blocks, k.n_tail, v.n_blocks, v.n_tail) == (16, 7, 16, 7)
    k, v = stream(n_tail=7, n_blocks=3), stream(n_tail=7, n_blocks=3, capacity=3)
    assert app(k, v) == CAPACITY


def ws_bytes(lib, k, v, Hq):
    n = ctypes.c_size_t(0)
    rc = lib.codec_decode_workspace_bytes(ctypes.byref(k), ctypes.byref(v), Hq, ctypes.byref(n))
    return rc, n.value


def test_query_groups_round_up(lib):
    # query heads per workgroup: G rounded up to 1, 2, 4 or 8, then groups of
    # eight (the last one partial), so each coefficient row is read once per
    # group; the plan, and so the workspace, is the one of the rounded group
    big = dict(n_blocks=4096, capacity=4096, heads=1)
    k, v = stream(**big), stream(**big)
    same = [(3, 4), (5, 8), (6, 8), (7, 8), (9, 16), (12, 16), (20, 24)]
    for g, like in same:
        assert ws_bytes(lib, k, v, g) == ws_bytes(lib, k, v, like), (g, like)
    # and the rounded groups differ from each other
    assert len({ws_bytes(lib, k, v, g)[1] for g in (1, 2, 4, 8, 16, 24)}) == 6


def test_workspace_plan(lib):
    k = stream(n_blocks=16, capacity=16)
    v = stream(n_blocks=16, capacity=16, fmt=bd.FMT_BF16)
    rc, n = ws_bytes(lib, k, v, 16)
    assert rc == OK and n > 0
    assert ws_bytes(lib, k, v, 6)[0] == SHAPE          # 6 % 4 kv heads
    assert ws_bytes(lib, k, stream(n_blocks=15), 16)[0] == SHAPE
    assert ws_bytes(lib, stream(), stream(), 16)[0] == SHAPE     # empty sequence
    assert ws_bytes(lib, stream(n_tail=1), stream(n_tail=1), 16)[0] == OK
    assert lib.codec_decode_workspace_bytes(ctypes.byref(k), ctypes.byref(v), 16, None) == NULL
    # the plan grows with the problem and is deterministic
    big = stream(n_blocks=8192, capacity=8192)
    assert ws_bytes(lib, big, big, 16) == ws_bytes(lib, big, big, 16)
    assert ws_bytes(lib, big, big, 16)[1] >= n
    # launch limits: batch rows x kv heads on one grid axis, rows per (b, h) in 32 bits
    wide = stream(n_blocks=16, capacity=16, batch=16383, heads=4)
    assert ws_bytes(lib, wide, wide, 16)[0] == OK
    wide = stream(n_blocks=16, capacity=16, batch=16384, heads=4)
    assert ws_bytes(lib, wide, wide, 16)[0] == UNSUPPORTED
    deep = stream(n_blocks=16, capacity=(1 << 30), keep=2)
    assert ws_bytes(lib, deep, deep, 16)[0] == UNSUPPORTED


def test_decode_validation(lib):
    k = stream(n_blocks=16, capacity=16)
    v = stream(n_blocks=16, capacity=16)
    two = bd._I64_2(2048, 128)
    _, need = ws_bytes(lib, k, v, 16)

    def dec(q=FAKE, Hq=16, scale=0.1, out=FAKE, odt=bd.FMT_F32, ws=FAKE, wsb=need, qs=two, kk=k, vv=v):
        return lib.codec_decode_attention(q, qs, Hq, ctypes.byref(kk), ctypes.byref(vv), ctypes.c_float(scale),
                                          out, two, odt, ws, wsb, None)

    assert dec(q=None) == NULL
    assert dec(out=None) == NULL
    assert dec(Hq=6) == SHAPE
    assert dec(Hq=0) == SHAPE
    assert dec(scale=0.0) == SCALE
    assert dec(scale=-1.0) == SCALE
    assert dec(scale=float("nan")) == SCALE
    assert dec(scale=float("inf")) == SCALE
    assert dec(odt=bd.FMT_I8) == FORMAT
    assert dec(ws=None) == WORKSPACE
    assert dec(ws=FAKE + 16) == WORKSPACE
    assert dec(wsb=need - 1) == WORKSPACE
    assert dec(q=FAKE + 2) == SHAPE
    assert dec(qs=bd._I64_2(2048, 100)) == SHAPE
    assert dec(vv=stream(n_blocks=16, capacity=16, keep=3)) == SHAPE
    assert dec(kk=stream(), vv=stream()) == SHAPE


def test_materialise_validation(lib):
    three = bd._I64_3(8192, 2048, 128)

    def mat(s, b0=0, dst=FAKE, st=three, odt=bd.FMT_BF16):
        return lib.codec_materialise(ctypes.byref(s) if s is not None else None, b0, dst, st, odt, None)

    s = stream(n_blocks=4, capacity=16)
    assert mat(None) == NULL
    assert mat(s, dst=None) == NULL
    assert lib.codec_materialise(ctypes.byref(s), 0, FAKE, None, bd.FMT_BF16, None) == NULL
    assert mat(s, odt=bd.FMT_I8) == FORMAT
    assert mat(s, b0=-1) == STATE
    assert mat(s, b0=5) == STATE
    assert mat(s, dst=FAKE + 8) == SHAPE
    assert mat(s, st=bd._I64_3(8192, 2048, 130)) == SHAPE
    assert mat(stream(fmt=9)) == FORMAT
    assert (s.n_blocks, s.n_tail) == (4, 0)
    # nothing to write (no new blocks, empty tail): succeeds without a launch
    assert mat(s, b0=4) == OK


def test_crop_validation_and_host_only_cases(lib):
    s = stream(n_blocks=4, capacity=16, n_tail=3)       # 35 tokens
    assert lib.codec_crop(None, 3, None) == NULL
    assert lib.codec_crop(ctypes.byref(s), -1, None) == STATE
    assert lib.codec_crop(ctypes.byref(s), 36, None) == STATE
    assert (s.n_blocks, s.n_tail) == (4, 3)
    # inside the raw tail: counters only
    assert lib.codec_crop(ctypes.byref(s), 34, None) == OK
    assert (s.n_blocks, s.n_tail) == (4, 2)
    # on a block boundary: counters only (archived rows are left as they are)
    assert lib.codec_crop(ctypes.byref(s), 16, None) == OK
    assert (s.n_blocks, s.n_tail) == (2, 0)
    assert lib.codec_crop(ctypes.byref(s), 16, None) == OK
    assert (s.n_blocks, s.n_tail) == (2, 0)
    assert lib.codec_crop(ctypes.byref(s), 0, None) == OK
    assert (s.n_blocks, s.n_tail) == (0, 0)


def test_select_batch_validation(lib):
    src = stream(n_blocks=4, capacity=16)
    idx = (ctypes.c_int64 * 3)(1, 0, 1)

    def sel(dst, ix=idx, n=3, s=src):
        return lib.codec_select_batch(ctypes.byref(s), ctypes.byref(dst) if dst is not None else None, ix, n, None)

    assert sel(None) == NULL
    assert sel(stream(batch=3), ix=None) == NULL
    assert sel(stream(batch=2)) == SHAPE                      # dst batch != n
    assert sel(stream(batch=3), n=0) == SHAPE
    assert sel(stream(batch=3, heads=2)) == SHAPE
    assert sel(stream(batch=3, keep=3)) == SHAPE
    assert sel(stream(batch=3, fmt=bd.FMT_BF16)) == FORMAT
    assert sel(stream(batch=3, raw_dtype=bd.FMT_F32)) == FORMAT
    assert sel(stream(batch=3, capacity=3)) == CAPACITY
    assert sel(stream(batch=3, rows=None)) == NULL
    assert sel(stream(batch=3, tail=FAKE + 4)) == SHAPE
    assert sel(stream(batch=3), ix=(ctypes.c_int64 * 3)(0, 2, 1)) == SHAPE   # index out of range
    assert sel(stream(batch=3), ix=(ctypes.c_int64 * 3)(0, -1, 1)) == SHAPE
    d = stream(batch=3)
    before = (d.n_blocks, d.n_tail)
    assert sel(d, ix=(ctypes.c_int64 * 3)(0, 5, 1)) == SHAPE
    assert (d.n_blocks, d.n_tail) == before


def test_png_mode_validation(lib):
    # PNG mode keeps S = R rows; keys and values share the synthesis
    assert encode(lib, stream(fmt=bd.FMT_PNG, keep=2, block=8)) == SHAPE
    assert encode(lib, stream(fmt=bd.FMT_PNG, keep=16, block=16), T=0) == OK
    assert encode(lib, stream(fmt=bd.FMT_PNG, keep=31, block=32)) == SHAPE    # PNG keeps all R rows
    two = bd._I64_2(1024, 128)
    k = stream(fmt=bd.FMT_PNG, keep=8, block=8)
    v = stream(fmt=bd.FMT_F32, keep=8, block=8)
    assert lib.codec_append_step(ctypes.byref(k), ctypes.byref(v), FAKE, two, FAKE, two, None) == FORMAT
    n = ctypes.c_size_t(0)
    k.n_blocks = v.n_blocks = 2
    assert lib.codec_decode_workspace_bytes(ctypes.byref(k), ctypes.byref(v), 8, ctypes.byref(n)) == FORMAT
    v.fmt = bd.FMT_PNG
    assert lib.codec_decode_workspace_bytes(ctypes.byref(k), ctypes.byref(v), 8, ctypes.byref(n)) == OK


def test_decode_append_validation(lib):
    k = stream(n_blocks=16, capacity=16, n_tail=3)
    v = stream(n_blocks=16, capacity=16, n_tail=3)
    two, qs = bd._I64_2(1024, 128), bd._I64_2(2048, 128)
    n = ctypes.c_size_t(0)
    k2, v2 = stream(n_blocks=16, capacity=16, n_tail=4), stream(n_blocks=16, capacity=16, n_tail=4)
    assert lib.codec_decode_workspace_bytes(ctypes.byref(k2), ctypes.byref(v2), 16, ctypes.byref(n)) == OK

    def call(kk=k, vv=v, kn=FAKE, ks=two, scale=0.1, ws=FAKE, wsb=n.value, Hq=16):
        return lib.codec_decode_attention_append(FAKE, qs, Hq, ctypes.byref(kk), ctypes.byref(vv), kn, ks, FAKE, two,
                                                 ctypes.c_float(scale), FAKE, qs, bd.FMT_F32, ws, wsb, None)

    assert call(kn=None) == NULL
    assert call(ks=bd._I64_2(1024, 130)) == SHAPE
    assert call(vv=stream(n_blocks=16, capacity=16, n_tail=2)) == SHAPE
    assert call(scale=-1.0) == SCALE
    assert call(Hq=6) == SHAPE
    assert call(ws=None) == WORKSPACE
    assert call(wsb=n.value - 1) == WORKSPACE
    # a token that completes a block needs archive capacity
    kf, vf = stream(n_blocks=16, capacity=16, n_tail=7), stream(n_blocks=16, capacity=16, n_tail=7)
    assert call(kk=kf, vv=vf) == CAPACITY
    for s in (k, v, kf, vf):
        assert s.n_blocks == 16 and s.n_tail in (3, 7)


SCRATCH_BYTES = 4 << 20      # CODEC_SCRATCH_BYTES


def test_decode_noalloc_validation(lib):
    # the same argument checks as codec_decode_attention (no workspace), all
    # before any HIP call
    k = stream(n_blocks=16, capacity=16)
    v = stream(n_blocks=16, capacity=16)
    two = bd._I64_2(2048, 128)

    def dec(q=FAKE, Hq=16, scale=0.1, out=FAKE, odt=bd.FMT_F32, qs=two, kk=k, vv=v):
        return lib.codec_decode_attention_noalloc(q, qs, Hq, ctypes.byref(kk), ctypes.byref(vv), ctypes.c_float(scale),
                                                  out, two, odt, None)

    assert dec(q=None) == NULL
    assert dec(out=None) == NULL
    assert dec(Hq=6) == SHAPE
    assert dec(scale=0.0) == SCALE
    assert dec(odt=bd.FMT_I8) == FORMAT
    assert dec(q=FAKE + 2) == SHAPE
    assert dec(vv=stream(n_blocks=16, capacity=16, keep=3)) == SHAPE
    assert dec(kk=stream(), vv=stream()) == SHAPE
    assert dec(kk=stream(head_dim=100), vv=stream(head_dim=100)) == UNSUPPORTED
    assert lib.codec_decode_attention_noalloc(FAKE, None, 16, ctypes.byref(k), ctypes.byref(v), ctypes.c_float(0.1),
                                              FAKE, two, bd.FMT_F32, None) == NULL


def test_decode_noalloc_rejects_plans_beyond_the_scratch(lib):
    # 255 (b, kv head) pairs, eight-head groups, head_dim 256: two splits per
    # pair and more partials than the scratch array holds -> WORKSPACE,
    # before any HIP call; the plan's workspace size says the same
    kw = dict(batch=255, heads=1, head_dim=256, n_blocks=4096, capacity=4096)
    k, v = stream(**kw), stream(**kw)
    rc, need = ws_bytes(lib, k, v, 8)
    assert rc == OK and need > SCRATCH_BYTES
    two = bd._I64_2(2048, 256)
    assert lib.codec_decode_attention_noalloc(FAKE, two, 8, ctypes.byref(k), ctypes.byref(v), ctypes.c_float(0.1),
                                              FAKE, two, bd.FMT_F32, None) == WORKSPACE
