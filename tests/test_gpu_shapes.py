"""GPU parity at head dims other than 64, 128 and 256 (any multiple of 8 up
to 256: the kernels compute at 64, 128 or 256 columns and rows keep their own
pitch) and with up to 32 kept frequencies, through the C ABI against the
fp64 oracle: encode, materialised view, crop and batch gather bit-exact,
decode within the output tolerance, appends and the fused decode-append.
Cases include int8 rows whose head dim is 8 modulo 16 (8-byte aligned
rows), the smallest head dim (8), a head dim just past 128 (computed at 256
columns), every kept frequency of 32-token blocks, and the largest S each
format pair's decode tile holds."""

import numpy as np
import pytest
import torch

import oracle as O
from compressed_domain_attention_amd import binding as bd
from compressed_domain_attention_amd import synthetic as syn
from parity_util import FMT_NAME, TOL, assert_archive_equal, gpu_archive, make_streams, note, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda"


def view_bits(t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


ENCODE_CASES = [
    # D, R, S, fmt, raw, B, H, T
    (80, 8, 2, "i8", "bf16", 2, 2, 8 * 40 + 5),
    (96, 16, 4, "bf16", "bf16", 1, 2, 16 * 20 + 7),
    (120, 8, 3, "i8", "bf16", 1, 3, 8 * 33 + 1),       # int8 rows of 120 bytes
    (8, 4, 2, "f32", "bf16", 1, 2, 4 * 50 + 3),
    (200, 16, 5, "i8", "f32", 1, 1, 16 * 9 + 2),
    (136, 8, 8, "bf16", "f32", 1, 2, 8 * 11),
    (128, 32, 32, "i8", "bf16", 1, 2, 32 * 10 + 17),   # all 32 frequencies: one wave per block, four passes
    (80, 32, 20, "i8", "bf16", 2, 1, 32 * 6 + 3),
    (40, 24, 24, "bf16", "bf16", 1, 2, 24 * 8 + 5),
    (104, 12, 12, "png", "bf16", 1, 2, 12 * 9 + 4),
]


@pytest.mark.parametrize("D,R,S,fmt,raw,B,H,T", ENCODE_CASES)
def test_encode_bitexact_any_head_dim(D, R, S, fmt, raw, B, H, T):
    note("encode shape", D, R, S, fmt, raw, B, H, T)
    dt = torch.bfloat16 if raw == "bf16" else torch.float32
    k, _, _ = syn.small_case(B, H, H, D, T, seed=D + R + S, dtype=dt, offset_var=2.0)
    st = bd.CodecStream(B, H, D, R, S, fmt=fmt, raw_dtype=raw, device=DEV)
    st.encode(k.to(DEV))
    torch.cuda.synchronize()
    assert (st.n_blocks, st.n_tail) == (T // R, T % R)
    assert_archive_equal(gpu_archive(st), O.encode(syn.bf16_to_numpy(k), R, S, fmt))


DECODE_CASES = [
    # B, Hq, H, D, R, S, kfmt, vfmt, T, raw
    (1, 8, 2, 80, 16, 4, "i8", "i8", 16 * 300 + 5, "bf16"),
    (2, 16, 2, 96, 8, 3, "i8", "bf16", 8 * 200 + 7, "bf16"),     # eight-head groups, bf16 values on MFMA
    (1, 8, 2, 120, 8, 2, "i8", "i8", 8 * 250 + 3, "bf16"),      # int8 rows of 120 bytes
    (1, 4, 2, 72, 8, 4, "bf16", "bf16", 8 * 120 + 6, "bf16"),
    (1, 4, 1, 200, 8, 4, "f32", "f32", 8 * 60 + 2, "f32"),      # computed at 256 columns, fp32 tail
    (1, 2, 1, 8, 4, 2, "f32", "i8", 4 * 100 + 3, "bf16"),
    (1, 3, 3, 48, 8, 2, "i8", "i8", 8 * 90 + 1, "bf16"),        # one head per group
    (1, 8, 2, 128, 32, 32, "i8", "i8", 32 * 60 + 13, "bf16"),   # S = R = 32
    (1, 8, 2, 64, 32, 32, "bf16", "bf16", 32 * 40 + 9, "bf16"),
    (1, 16, 2, 96, 32, 24, "i8", "bf16", 32 * 30 + 31, "bf16"),
    (1, 4, 2, 136, 16, 16, "i8", "i8", 16 * 70 + 15, "bf16"),   # computed at 256 columns, S = 16
]


@pytest.mark.parametrize("B,Hq,H,D,R,S,kfmt,vfmt,T,raw", DECODE_CASES)
def test_decode_parity_any_head_dim(B, Hq, H, D, R, S, kfmt, vfmt, T, raw):
    note("decode shape", B, Hq, H, D, R, S, kfmt, vfmt, T, raw)
    dt = torch.bfloat16 if raw == "bf16" else torch.float32
    k, v, q = syn.small_case(B, Hq, H, D, T, seed=D * 3 + R + S, dtype=dt, offset_var=1.0)
    ks, vs = make_streams(k, v, R, S, kfmt, vfmt)
    # the output rows are padded and pre-filled: columns past D stay untouched
    obig = torch.full((B, Hq, 1, D + 8), float("nan"), dtype=torch.float32, device=DEV)
    out = obig[:, :, :, :D]
    bd.decode_attention(q.to(DEV), ks, vs, out=out)
    torch.cuda.synchronize()
    ka, va = gpu_archive(ks), gpu_archive(vs)
    assert_archive_equal(ka, O.encode(syn.bf16_to_numpy(k), R, S, kfmt))
    ref = O.decode_attention(syn.bf16_to_numpy(q), ka, va)
    assert rel_err(out.cpu().numpy()[:, :, 0], ref) <= TOL
    assert torch.isnan(obig[:, :, :, D:]).all()


def test_decode_beyond_the_tile_is_unsupported():
    # fp32 rows at head dim 200 hold four rows per decode tile: S = 5 has no kernel
    k, v, q = syn.small_case(1, 2, 1, 200, 8 * 10, seed=5, dtype=torch.float32)
    ks, vs = make_streams(k, v, 8, 5, "f32", "f32")
    with pytest.raises(bd.CodecError) as e:
        bd.decode_attention(q.to(DEV), ks, vs)
    assert e.value.status == 7        # CODEC_ERR_UNSUPPORTED


VIEW_CASES = [
    # D, R, S, fmt, raw, out, B, H, T, block_begin
    (80, 8, 2, "i8", "bf16", "bf16", 2, 2, 8 * 30 + 5, 3),
    (120, 16, 4, "bf16", "bf16", "f32", 1, 2, 16 * 12 + 15, 0),
    (64, 32, 32, "i8", "bf16", "bf16", 1, 2, 32 * 5 + 7, 1),     # more than 16 kept rows
    (8, 32, 24, "f32", "f32", "f32", 1, 3, 32 * 4 + 2, 0),
    (200, 24, 18, "i8", "f32", "bf16", 1, 1, 24 * 3 + 23, 0),
]


@pytest.mark.parametrize("D,R,S,fmt,raw,out,B,H,T,b0", VIEW_CASES)
def test_materialise_bitexact_any_head_dim(D, R, S, fmt, raw, out, B, H, T, b0):
    note("materialise shape", D, R, S, fmt, raw, out, B, H, T, b0)
    dt = torch.bfloat16 if raw == "bf16" else torch.float32
    k, _, _ = syn.small_case(B, H, H, D, T, seed=D + 2 * R + S, dtype=dt, offset_var=2.0)
    st = bd.CodecStream(B, H, D, R, S, fmt=fmt, raw_dtype=raw, device=DEV)
    st.encode(k.to(DEV))
    odt = torch.bfloat16 if out == "bf16" else torch.float32
    dst = torch.full((B, H, T + 3, D), float("nan"), dtype=odt, device=DEV)
    bd.materialise(st, dst, block_begin=b0)
    torch.cuda.synchronize()
    got = view_bits(dst)
    want = O.view(gpu_archive(st), FMT_NAME[bd._fmt(out)], block_begin=b0)
    assert got[:, :, b0 * R:T].tobytes() == np.ascontiguousarray(want).tobytes(), \
        np.argwhere(got[:, :, b0 * R:T] != want)[:5].tolist()


def test_crop_and_gather_any_head_dim():
    # int8 rows of 120 bytes with three rows per block and 33 blocks: the
    # gathered slabs are not multiples of 16 bytes
    B, H, Hq, D, R, S = 3, 2, 4, 120, 8, 3
    T = 8 * 33 + 1
    note("crop / gather shape", D, R, S)
    k, v, q = syn.small_case(B, Hq, H, D, T, seed=12)
    ks, vs = make_streams(k, v, R, S, "i8", "i8")
    ka, va = gpu_archive(ks), gpu_archive(vs)
    idx = [2, 0, 2, 1]
    ks.select_batch(idx)
    vs.select_batch(idx)
    torch.cuda.synchronize()
    assert_archive_equal(gpu_archive(ks), O.select_batch(ka, idx))
    assert_archive_equal(gpu_archive(vs), O.select_batch(va, idx))
    L = 8 * 20 + 5
    ka, va = gpu_archive(ks), gpu_archive(vs)
    ks.crop(L)
    vs.crop(L)
    torch.cuda.synchronize()
    assert_archive_equal(gpu_archive(ks), O.crop(ka, L, O.BF16))
    assert_archive_equal(gpu_archive(vs), O.crop(va, L, O.BF16))
    qg = q[idx].contiguous()
    out = bd.decode_attention(qg.to(DEV), ks, vs)
    ref = O.decode_attention(syn.bf16_to_numpy(qg), gpu_archive(ks), gpu_archive(vs))
    assert rel_err(out[:, :, 0].float().cpu().numpy(), ref) <= TOL


@pytest.mark.parametrize("fmt,R,S,Hq,H,D,T0", [
    ("i8", 8, 2, 8, 2, 80, 8 * 30 + 3),
    ("i8", 32, 32, 8, 2, 128, 32 * 6 + 30),     # block-end appends encode 32 rows in passes of eight
    ("bf16", 16, 8, 4, 2, 40, 16 * 12 + 9),
])
def test_fused_append_any_head_dim(fmt, R, S, Hq, H, D, T0):
    note("fused append shape", fmt, R, S, Hq, H, D, T0)
    B = 1
    steps = R + 5
    k, v, _ = syn.small_case(B, Hq, H, D, T0 + steps, seed=D + R)
    ka, va = make_streams(k[:, :, :T0], v[:, :, :T0], R, S, fmt, fmt)
    kb, vb = make_streams(k[:, :, :T0], v[:, :, :T0], R, S, fmt, fmt)
    for s in range(steps):
        t = T0 + s
        q = syn.gaussian((B, Hq, 1, D), 700 + s).to(DEV)
        kn, vn = k[:, :, t:t + 1].to(DEV).contiguous(), v[:, :, t:t + 1].to(DEV).contiguous()
        bd.append_step(ka, va, kn, vn)
        oa = bd.decode_attention(q, ka, va)
        ob = bd.decode_attention_append(q, kb, vb, kn, vn)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob), (s, (oa - ob).abs().max().item())
        if s in (0, R - T0 % R - 1, steps - 1):
            assert_archive_equal(gpu_archive(kb), gpu_archive(ka))
            ref = O.decode_attention(syn.bf16_to_numpy(q.cpu()), gpu_archive(kb), gpu_archive(vb))
            assert rel_err(ob[:, :, 0].float().cpu().numpy(), ref) <= TOL
    assert_archive_equal(gpu_archive(kb), O.encode(syn.bf16_to_numpy(k), R, S, fmt))
