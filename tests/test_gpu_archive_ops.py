"""GPU parity of the structural archive operations through the C ABI:
the materialised view (codec_materialise, CodecStream.read), the exact crop
(codec_crop) and the batch gather (codec_select_batch), against the fp64
oracle.  All three are bit-exact: the view follows a fixed-order fp64
contract, crop and gather move bytes.  Cases span several blocks with ragged
tails, every row format, both raw and view formats, a memoised partial
decode, crops inside the tail, on a block boundary and inside the archive,
and gathers with repeated and reordered rows.
"""

import numpy as np
import pytest
import torch

import oracle as O
from compressed_domain_attention_amd import binding as bd
from compressed_domain_attention_amd import synthetic as syn
from parity_util import FMT_NAME, TOL, assert_archive_equal, gpu_archive, gpu_head_archive, make_streams, note, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda"


def view_bits(t):
    """A bf16 / fp32 device view as the oracle's representation (uint16 patterns / float32)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def oracle_stream(arch):
    """An oracle Stream holding exactly the given archive (for appends after a crop)."""
    st = O.Stream(arch["R"], arch["S"], arch["fmt"])
    for n in range(arch["n_blocks"]):
        st.rows.append(arch["rows"][..., n, :, :])
        st.scales.append(None if arch["scales"] is None else arch["scales"][..., n, :])
    st.tail = np.asarray(arch["tail"], dtype=np.float64)
    return st


VIEW_CASES = [
    # D, R, S, fmt, raw, out, B, H, T, block_begin
    (128, 8, 2, "i8", "bf16", "bf16", 2, 3, 8 * 37 + 5, 0),
    (128, 16, 4, "i8", "bf16", "bf16", 1, 2, 16 * 21 + 15, 7),
    (128, 16, 4, "i8", "bf16", "f32", 1, 2, 16 * 21 + 15, 0),
    (64, 8, 3, "bf16", "bf16", "bf16", 2, 2, 8 * 40, 40),
    (256, 8, 3, "i8", "bf16", "bf16", 1, 2, 8 * 9 + 1, 3),
    (64, 2, 2, "f32", "f32", "f32", 2, 1, 65, 0),
    (128, 32, 16, "i8", "f32", "bf16", 1, 2, 32 * 3 + 31, 1),
    (64, 1, 1, "f32", "bf16", "f32", 1, 2, 33, 0),
    (128, 5, 3, "i8", "bf16", "bf16", 1, 1, 5 * 11 + 2, 0),
    (128, 8, 2, "i8", "bf16", "bf16", 1, 1, 5, 0),            # tail only
]


@pytest.mark.parametrize("D,R,S,fmt,raw,out,B,H,T,b0", VIEW_CASES)
def test_materialise_bitexact(D, R, S, fmt, raw, out, B, H, T, b0):
    note("materialise", D, R, S, fmt, raw, out, B, H, T, b0)
    dt = torch.bfloat16 if raw == "bf16" else torch.float32
    k, _, _ = syn.small_case(B, H, H, D, T, seed=3 * R + S, dtype=dt, offset_var=2.0)
    st = bd.CodecStream(B, H, D, R, S, fmt=fmt, raw_dtype=raw, device=DEV)
    st.encode(k.to(DEV))
    odt = torch.bfloat16 if out == "bf16" else torch.float32
    # a padded destination pre-filled with a sentinel: rows before the
    # memoised block and past the sequence must stay untouched
    dst = torch.full((B, H, T + 7, D), float("nan"), dtype=odt, device=DEV)
    sentinel = view_bits(dst[:, :, :1])
    bd.materialise(st, dst, block_begin=b0)
    torch.cuda.synchronize()
    got = view_bits(dst)
    want = O.view(gpu_archive(st), FMT_NAME[bd._fmt(out)], block_begin=b0)
    assert got[:, :, b0 * R:T].tobytes() == np.ascontiguousarray(want).tobytes(), \
        np.argwhere(got[:, :, b0 * R:T] != want)[:5].tolist()
    for part in (got[:, :, :b0 * R], got[:, :, T:]):
        assert part.tobytes() == np.broadcast_to(sentinel, part.shape).tobytes()


def test_read_is_memoised_across_appends():
    # cache.py ``read``: every read equals the full view of the current
    # archive; only new blocks are decoded in between (the memo advances).
    note("read memo")
    B, H, D, R, S = 2, 2, 128, 8, 2
    T0, steps = 8 * 5 + 3, 21
    k, v, _ = syn.small_case(B, H, H, D, T0 + steps, seed=41)
    ks, vs = make_streams(k[:, :, :T0], v[:, :, :T0], R, S, "i8", "i8")
    for s in range(steps + 1):
        if s:
            t = T0 + s - 1
            bd.append_step(ks, vs, k[:, :, t:t + 1].to(DEV).contiguous(), v[:, :, t:t + 1].to(DEV).contiguous())
        if s % 4 == 0 or s == steps:
            got = view_bits(ks.read())
            assert ks._rec_blocks == ks.n_blocks
            want = O.view(gpu_archive(ks), O.BF16)
            assert got.tobytes() == np.ascontiguousarray(want).tobytes(), s
    torch.cuda.synchronize()


@pytest.mark.parametrize("fmt,raw", [("i8", "bf16"), ("bf16", "bf16"), ("f32", "f32")])
def test_crop_bitexact_then_decode_and_append(fmt, raw):
    B, H, Hq, D, R, S = 2, 2, 4, 128, 8, 3
    T = 8 * 23 + 6
    dt = torch.bfloat16 if raw == "bf16" else torch.float32
    k, v, q = syn.small_case(B, Hq, H, D, T + 12, seed=17, dtype=dt)
    for L in (T, T - 3, 8 * 20, 8 * 20 + 5, 8 * 11 + 1, 7, 0):
        note("crop", fmt, raw, L)
        ks, vs = make_streams(k[:, :, :T], v[:, :, :T], R, S, fmt, fmt, raw=raw)
        ka, va = gpu_archive(ks), gpu_archive(vs)
        ks.crop(L)
        vs.crop(L)
        torch.cuda.synchronize()
        assert ks.seq_len == L
        assert_archive_equal(gpu_archive(ks), O.crop(ka, L, FMT_NAME[bd._fmt(raw)]))
        assert_archive_equal(gpu_archive(vs), O.crop(va, L, FMT_NAME[bd._fmt(raw)]))
        # idempotent
        ks.crop(L)
        assert_archive_equal(gpu_archive(ks), O.crop(ka, L, FMT_NAME[bd._fmt(raw)]))
        if L == 0:
            continue
        # decode attention on the cropped streams
        qd = q.to(DEV)
        out = bd.decode_attention(qd, ks, vs)
        ref = O.decode_attention(syn.bf16_to_numpy(q), gpu_archive(ks), gpu_archive(vs))
        assert rel_err(out[:, :, 0].float().cpu().numpy(), ref) <= TOL
        # appending after the crop archives the boundary block from the re-exposed tail
        ko, vo = oracle_stream(gpu_archive(ks)), oracle_stream(gpu_archive(vs))
        for t in range(T, T + 12):
            kn, vn = k[:, :, t:t + 1], v[:, :, t:t + 1]
            bd.append_step(ks, vs, kn.to(DEV).contiguous(), vn.to(DEV).contiguous())
            ko.append(syn.bf16_to_numpy(kn))
            vo.append(syn.bf16_to_numpy(vn))
        torch.cuda.synchronize()
        assert_archive_equal(gpu_archive(ks), ko.archive())
        assert_archive_equal(gpu_archive(vs), vo.archive())


@pytest.mark.parametrize("fmt,idx", [("i8", [3, 3, 0, 2, 1]), ("bf16", [1, 0]), ("f32", [2, 2, 2])])
def test_select_batch_bitexact(fmt, idx):
    note("select_batch", fmt, idx)
    B, H, Hq, D, R, S = 4, 2, 8, 64, 8, 2
    T = 8 * 13 + 5
    k, v, q = syn.small_case(B, Hq, H, D, T, seed=23)
    ks, vs = make_streams(k, v, R, S, fmt, fmt)
    ks.read()                                   # a memoised view exists and is dropped
    ka, va = gpu_archive(ks), gpu_archive(vs)
    ks.select_batch(idx)
    vs.select_batch(torch.tensor(idx))
    torch.cuda.synchronize()
    assert ks.B == len(idx) and ks._rec is None
    assert_archive_equal(gpu_archive(ks), O.select_batch(ka, idx))
    assert_archive_equal(gpu_archive(vs), O.select_batch(va, idx))
    # decode on the gathered streams = decode of the gathered archives
    qg = q[idx].contiguous()
    out = bd.decode_attention(qg.to(DEV), ks, vs)
    ref = O.decode_attention(syn.bf16_to_numpy(qg), gpu_archive(ks), gpu_archive(vs))
    assert rel_err(out[:, :, 0].float().cpu().numpy(), ref) <= TOL
    # the gathered view is the gathered view
    assert view_bits(ks.read()).tobytes() == np.ascontiguousarray(O.view(ka, O.BF16)[idx]).tobytes()


def test_materialise_fullsize_128k():
    # The 128K-context workload's key archive (B=1, H=8, T=131077, R=16, S=4,
    # int8): the whole bf16 view in one call; two heads checked bit for bit.
    w = syn.WORKLOADS["long128k"]
    note("materialise fullsize", w.name)
    k, _ = syn.workload_kv_device(w, device=DEV)
    ks = bd.CodecStream(w.B, w.Hkv, w.D, w.R, w.S, fmt=w.kfmt, device=DEV)
    ks.encode(k[:, :, :w.T])
    del k
    view = ks.read()
    torch.cuda.synchronize()
    for h in (0, 5):
        got = view_bits(view[:, h:h + 1])
        want = O.view(gpu_head_archive(ks, 0, h), O.BF16)
        assert got.tobytes() == np.ascontiguousarray(want).tobytes(), h


def test_select_batch_fullsize_beam_reorder():
    # The large-batch workload (B=64, H=8, T=8192, int8 keys, bf16 values):
    # a beam reorder of all 64 rows; sampled rows checked against the source
    # archive bytes.
    w = syn.WORKLOADS["batch64_gqa8"]
    note("select_batch fullsize", w.name)
    k, v = syn.workload_kv_device(w, T=w.T + 3, device=DEV)
    ks = bd.CodecStream(w.B, w.Hkv, w.D, w.R, w.S, fmt=w.kfmt, device=DEV)
    vs = bd.CodecStream(w.B, w.Hkv, w.D, w.R, w.S, fmt=w.vfmt, device=DEV)
    ks.encode(k)
    vs.encode(v)
    del k, v
    idx = np.random.default_rng(5).integers(0, w.B, size=w.B)
    src = {(b, h): (gpu_head_archive(ks, b, h), gpu_head_archive(vs, b, h))
           for b in set(int(i) for i in idx[[0, 17, 63]]) for h in (0, 7)}
    ks.select_batch(idx)
    vs.select_batch(idx)
    torch.cuda.synchronize()
    for i in (0, 17, 63):
        for h in (0, 7):
            ka, va = src[(int(idx[i]), h)]
            assert_archive_equal(gpu_head_archive(ks, i, h), ka)
            assert_archive_equal(gpu_head_archive(vs, i, h), va)
