"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Encode: codes, scales, float rows and tail bit-exact.  Decode: on the
identical archive, max over (b, hq) of ||o - o_ref||_inf / ||o_ref||_inf
<= 2e-3 (fp32 accumulation, bf16 inputs).  Sizes span several tiles and
splits with ragged ends; edge cases: empty archive (tail only), no tail,
R = 1, S = R, GQA from 1 to 16, every row format, fp32 raw tokens.
"""

import numpy as np
import pytest
import torch

import oracle as O
from compressed_domain_attention_amd import binding as bd
from compressed_domain_attention_amd import synthetic as syn
from parity_util import TOL, assert_archive_equal, gpu_archive, make_streams, note, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda"


# ------------------------------------------------------------------ encode --
ENCODE_CASES = [
    # D, R, S, fmt, raw, B, H, T
    (64, 8, 2, "f32", "bf16", 1, 2, 1027),
    (128, 8, 2, "i8", "bf16", 2, 3, 8 * 37 + 5),
    (128, 16, 4, "i8", "bf16", 1, 2, 16 * 21 + 15),
    (128, 8, 3, "bf16", "bf16", 2, 2, 8 * 40),
    (256, 8, 3, "i8", "bf16", 1, 2, 8 * 9 + 1),
    (64, 1, 1, "i8", "bf16", 1, 2, 33),
    (64, 2, 2, "f32", "f32", 2, 1, 65),
    (128, 32, 16, "i8", "f32", 1, 2, 32 * 3 + 31),
    (128, 5, 3, "i8", "bf16", 1, 1, 5 * 11 + 2),
    (64, 8, 8, "f32", "bf16", 1, 1, 8 * 6),
    (128, 8, 2, "i8", "bf16", 1, 1, 5),        # tail only
    (128, 16, 16, "i8", "bf16", 1, 2, 16 * 9 + 3),   # four passes of four rows
    (256, 16, 5, "bf16", "bf16", 2, 1, 16 * 7),      # a second pass with one row
    (128, 16, 4, "i8", "f32", 1, 2, 16 * 7 + 9),      # fp32 tokens, sixteen-token blocks
    (256, 12, 3, "bf16", "f32", 1, 1, 12 * 5 + 1),    # fp32 tokens, R = 12, three rows per pass
]


@pytest.mark.parametrize("D,R,S,fmt,raw,B,H,T", ENCODE_CASES)
def test_encode_bitexact(D, R, S, fmt, raw, B, H, T):
    note("encode", D, R, S, fmt, raw, B, H, T)
    dt = torch.bfloat16 if raw == "bf16" else torch.float32
    k, _, _ = syn.small_case(B, H, H, D, T, seed=R * 7 + S, dtype=dt, offset_var=2.0)
    st = bd.CodecStream(B, H, D, R, S, fmt=fmt, raw_dtype=raw, device=DEV)
    st.encode(k.to(DEV))
    torch.cuda.synchronize()
    assert (st.n_blocks, st.n_tail) == (T // R, T % R)
    assert_archive_equal(gpu_archive(st), O.encode(syn.bf16_to_numpy(k), R, S, fmt))


@pytest.mark.parametrize("D,R,S,fmt,T1,T2", [(128, 8, 3, "i8", 8 * 21, 8 * 13 + 6), (64, 16, 4, "bf16", 16 * 5, 16 * 2)])
def test_encode_two_calls(D, R, S, fmt, T1, T2):
    # the second call archives into slots after the first call's blocks, from
    # a view that starts T1 tokens into the tensor
    note("encode two calls", D, R, S, fmt, T1, T2)
    B, H = 2, 3
    k, _, _ = syn.small_case(B, H, H, D, T1 + T2, seed=D + R + S, dtype=torch.bfloat16, offset_var=2.0)
    kd = k.to(DEV)
    st = bd.CodecStream(B, H, D, R, S, fmt=fmt, device=DEV)
    st.encode(kd[:, :, :T1])
    st.encode(kd[:, :, T1:])
    torch.cuda.synchronize()
    assert (st.n_blocks, st.n_tail) == ((T1 + T2) // R, (T1 + T2) % R)
    assert_archive_equal(gpu_archive(st), O.encode(syn.bf16_to_numpy(k), R, S, fmt))


def test_encode_special_values():
    # zero block (scale 0, codes 0), exact ties in the quantiser, huge and tiny magnitudes
    note("encode special values")
    B, H, D, R, S = 1, 1, 64, 4, 4
    x = np.zeros((B, H, 5 * R, D), dtype=np.float32)
    x[0, 0, R:2 * R] = 1e30 * np.linspace(-1, 1, R * D, dtype=np.float32).reshape(R, D)
    x[0, 0, 2 * R:3 * R] = 1e-30 * np.linspace(-1, 1, R * D, dtype=np.float32).reshape(R, D)
    x[0, 0, 3 * R:4 * R, :] = np.arange(-127, 129, dtype=np.float32)[: R * D].reshape(R, D) / 2
    x[0, 0, 4 * R:5 * R, 0] = -0.0
    t = torch.from_numpy(x)
    for fmt in ("i8", "f32", "bf16"):
        st = bd.CodecStream(B, H, D, R, S, fmt=fmt, raw_dtype="f32", device=DEV)
        st.encode(t.to(DEV))
        torch.cuda.synchronize()
        assert_archive_equal(gpu_archive(st), O.encode(x.astype(np.float64), R, S, fmt))


# ------------------------------------------------------------------ decode --
DECODE_CASES = [
    # B, Hq, H, D, R, S, kfmt, vfmt, T, raw
    (1, 4, 2, 64, 8, 2, "f32", "f32", 1027, "bf16"),
    (2, 8, 2, 128, 8, 2, "i8", "i8", 8 * 300 + 3, "bf16"),
    (1, 8, 2, 128, 16, 4, "i8", "i8", 16 * 700 + 5, "bf16"),
    (2, 16, 2, 128, 8, 3, "i8", "bf16", 8 * 200 + 7, "bf16"),
    (1, 2, 2, 64, 8, 2, "i8", "i8", 8 * 100, "bf16"),          # G = 1, no tail
    (1, 6, 2, 128, 8, 2, "bf16", "i8", 8 * 90 + 1, "bf16"),    # G = 3
    (1, 32, 2, 128, 8, 4, "i8", "f32", 8 * 64 + 2, "bf16"),    # G = 16 -> two query groups
    (1, 4, 1, 256, 8, 3, "i8", "i8", 8 * 130 + 6, "bf16"),
    (1, 8, 1, 256, 16, 8, "bf16", "bf16", 16 * 50 + 9, "bf16"),
    (1, 4, 2, 64, 1, 1, "i8", "f32", 300, "bf16"),             # R = 1
    (1, 4, 2, 64, 8, 8, "f32", "f32", 8 * 50 + 4, "f32"),      # S = R, fp32 tokens
    (1, 8, 2, 128, 32, 16, "i8", "i8", 32 * 40 + 31, "bf16"),
    (1, 4, 2, 128, 8, 2, "i8", "i8", 7, "bf16"),               # tail only
    (1, 4, 2, 128, 8, 2, "i8", "i8", 1, "bf16"),               # one token
    (3, 24, 3, 64, 4, 1, "i8", "i8", 4 * 333 + 2, "bf16"),     # S = 1
    # bf16 value rows on the MFMA path: G = 4, 2, 1 (absent heads in an M
    # block), D = 64 (two 32-row chunks per tile), fp32 tokens, R = 32
    (1, 8, 2, 64, 8, 2, "i8", "bf16", 8 * 50 + 3, "bf16"),
    (2, 4, 2, 128, 16, 4, "bf16", "bf16", 16 * 30 + 7, "f32"),
    (1, 2, 2, 128, 8, 3, "f32", "bf16", 8 * 33, "bf16"),
    (1, 8, 2, 128, 32, 16, "i8", "bf16", 32 * 12 + 17, "bf16"),
    # S <= 2: two items per logit MFMA column when R <= 8 (R = 6, 8), the
    # plain path when R > 8
    (1, 8, 2, 128, 6, 2, "i8", "i8", 6 * 201 + 5, "bf16"),
    (3, 8, 2, 128, 16, 2, "i8", "i8", 16 * 64 + 3, "bf16"),
    # eight-head groups with S = 2 (int8 rows: two items per logit column;
    # bf16 values: plain logit path), at D = 128, 64 and 256
    (1, 16, 2, 128, 8, 2, "i8", "i8", 8 * 150 + 3, "bf16"),
    (2, 16, 2, 64, 8, 2, "i8", "i8", 8 * 400 + 5, "bf16"),    # 32-row tiles, thirteen splits
    (1, 16, 2, 256, 8, 2, "i8", "i8", 8 * 200 + 3, "bf16"),
    (1, 8, 2, 64, 16, 4, "i8", "i8", 16 * 300 + 7, "bf16"),   # D = 64, GQA 4, S = 4, several splits
    (1, 8, 2, 256, 8, 3, "i8", "bf16", 8 * 60 + 5, "bf16"),
    (2, 16, 2, 64, 8, 2, "i8", "bf16", 8 * 70 + 1, "bf16"),
    # query groups that do not divide the kv head's G heads: G = 3 runs as a
    # group of four with one absent head (the last kv head's absent head
    # would be past the query tensor), 5..7 as groups of eight, 12 and 24 as
    # eight-head groups plus a partial one; every row is read once per group
    (1, 3, 1, 128, 16, 4, "i8", "i8", 16 * 200 + 9, "bf16"),
    (1, 10, 2, 128, 8, 2, "i8", "i8", 8 * 120 + 3, "bf16"),    # G = 5
    (2, 12, 2, 64, 16, 4, "i8", "bf16", 16 * 40 + 5, "bf16"),  # G = 6
    (1, 14, 2, 128, 8, 3, "f32", "f32", 8 * 40 + 7, "f32"),    # G = 7, VALU paths
    (1, 12, 1, 128, 8, 2, "i8", "i8", 8 * 300 + 1, "bf16"),    # G = 12: 8 + 4
    (1, 24, 1, 64, 8, 2, "bf16", "i8", 8 * 50 + 2, "bf16"),    # G = 24: 8 + 8 + 8
]


@pytest.mark.parametrize("B,Hq,H,D,R,S,kfmt,vfmt,T,raw", DECODE_CASES)
def test_decode_parity(B, Hq, H, D, R, S, kfmt, vfmt, T, raw):
    note("decode", B, Hq, H, D, R, S, kfmt, vfmt, T, raw)
    dt = torch.bfloat16 if raw == "bf16" else torch.float32
    k, v, q = syn.small_case(B, Hq, H, D, T, seed=B * 13 + Hq + R, dtype=dt, offset_var=1.0)
    ks, vs = make_streams(k, v, R, S, kfmt, vfmt)
    out = bd.decode_attention(q.to(DEV), ks, vs)
    torch.cuda.synchronize()
    ka, va = gpu_archive(ks), gpu_archive(vs)
    assert_archive_equal(ka, O.encode(syn.bf16_to_numpy(k), R, S, kfmt))
    ref = O.decode_attention(syn.bf16_to_numpy(q), ka, va)
    err = rel_err(out.cpu().numpy()[:, :, 0], ref)
    assert err <= TOL, err


def test_decode_bf16_out_and_strided_views():
    note("decode bf16 out / strided q and out")
    B, Hq, H, D, R, S, T = 2, 8, 2, 128, 8, 2, 8 * 77 + 3
    k, v, q = syn.small_case(B, Hq, H, D, T, seed=3)
    ks, vs = make_streams(k, v, R, S, "i8", "i8")
    # q as a strided view: heads interleaved with padding
    qbig = torch.zeros((B, Hq, 2, D), dtype=torch.bfloat16, device=DEV)
    qbig[:, :, 1:2] = q.to(DEV)
    qv = qbig[:, :, 1:2]
    obig = torch.full((B, Hq, 3, D), float("nan"), dtype=torch.float32, device=DEV)
    ov = obig[:, :, 2:3]
    bd.decode_attention(qv, ks, vs, out=ov)
    ob = bd.decode_attention(q.to(DEV), ks, vs, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = O.decode_attention(syn.bf16_to_numpy(q), gpu_archive(ks), gpu_archive(vs))
    assert rel_err(ov.cpu().numpy()[:, :, 0], ref) <= TOL
    assert torch.isnan(obig[:, :, :2]).all()           # nothing outside the view was written
    assert rel_err(ob.float().cpu().numpy()[:, :, 0], ref) <= 2 ** -8 + TOL


def test_decode_scale_argument():
    note("decode scale")
    B, Hq, H, D, R, S, T = 1, 4, 2, 64, 8, 2, 8 * 60 + 1
    k, v, q = syn.small_case(B, Hq, H, D, T, seed=5)
    ks, vs = make_streams(k, v, R, S, "i8", "i8")
    for scale in (0.01, 0.125, 1.0, 3.0):
        out = bd.decode_attention(q.to(DEV), ks, vs, scale=scale)
        torch.cuda.synchronize()
        ref = O.decode_attention(syn.bf16_to_numpy(q), gpu_archive(ks), gpu_archive(vs), scale)
        assert rel_err(out.cpu().numpy()[:, :, 0], ref) <= TOL, scale


def test_decode_repeatable_and_workspace_reuse():
    # the workspace counters reset themselves: back-to-back calls, same bits
    note("decode repeat")
    B, Hq, H, D, R, S, T = 2, 8, 2, 128, 16, 4, 16 * 400 + 9
    k, v, q = syn.small_case(B, Hq, H, D, T, seed=6)
    ks, vs = make_streams(k, v, R, S, "i8", "i8")
    qd = q.to(DEV)
    outs = [bd.decode_attention(qd, ks, vs).clone() for _ in range(5)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


def test_one_workspace_for_calls_of_different_shapes():
    """One explicit workspace serves decodes whose (b, kv head, group) pair
    counts and split counts differ, interleaved: every result matches the
    oracle (the arrival counters must never meet another call's partials)."""
    note("decode shared workspace")
    cases = []
    for (B, Hq, H, T, seed) in ((1, 32, 8, 16 * 2000 + 3, 21), (4, 32, 8, 16 * 300 + 1, 22), (2, 8, 2, 16 * 900, 23)):
        k, v, q = syn.small_case(B, Hq, H, 128, T, seed=seed)
        ks, vs = make_streams(k, v, 16, 4, "i8", "i8")
        cases.append((q.to(DEV), ks, vs))
    need = max(bd.decode_workspace_bytes(ks, vs, q.shape[1]) for (q, ks, vs) in cases)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    refs = [O.decode_attention(syn.bf16_to_numpy(q), gpu_archive(ks), gpu_archive(vs)) for (q, ks, vs) in cases]
    for order in ((0, 1, 2), (2, 0, 1), (1, 1, 0, 2, 0)):
        for i in order:
            q, ks, vs = cases[i]
            out = bd.decode_attention(q, ks, vs, workspace=ws)
            torch.cuda.synchronize()
            assert rel_err(out.cpu().numpy()[:, :, 0], refs[i]) <= TOL, (order, i)


def test_graph_replay_matches_eager():
    """append + decode captured in a HIP graph and replayed several times
    with eager work in between: every replay equals the eager result of the
    same step (the graph holds no memset nodes; the counters self-reset)."""
    note("graph replay")
    B, Hq, H, D, R, S, T0 = 2, 8, 2, 128, 8, 2, 8 * 200 + 7
    k, v, q = syn.small_case(B, Hq, H, D, T0 + 8, seed=31)
    kd, vd, qd = k.to(DEV), v.to(DEV), q.to(DEV)
    # eager reference: append the token at T0 (completes a block), then decode
    ks, vs = make_streams(k[:, :, :T0], v[:, :, :T0], R, S, "i8", "i8", capacity=T0 // R + 4)
    bd.append_step(ks, vs, kd[:, :, T0:T0 + 1], vd[:, :, T0:T0 + 1])
    ref = bd.decode_attention(qd, ks, vs).clone()
    torch.cuda.synchronize()
    # graph: the same step on fresh streams, replayed after restoring the state
    gs_k, gs_v = make_streams(k[:, :, :T0], v[:, :, :T0], R, S, "i8", "i8", capacity=T0 // R + 4)
    snap = [t.clone() for t in (gs_k.rows, gs_k.scales, gs_k.tail, gs_v.rows, gs_v.scales, gs_v.tail)]
    n0, t0 = gs_k.n_blocks, gs_k.n_tail
    ws = torch.zeros(bd.decode_workspace_bytes(gs_k, gs_v, Hq), dtype=torch.uint8, device=DEV)
    out = torch.empty((B, Hq, 1, D), dtype=torch.float32, device=DEV)
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        bd.append_step(gs_k, gs_v, kd[:, :, T0:T0 + 1], vd[:, :, T0:T0 + 1])
        bd.decode_attention(qd, gs_k, gs_v, out=out, workspace=ws)
    for rep in range(4):
        for dst, src in zip((gs_k.rows, gs_k.scales, gs_k.tail, gs_v.rows, gs_v.scales, gs_v.tail), snap):
            dst.copy_(src)
        noise = torch.randn(1 << 20, device=DEV).sum()        # eager work between replays
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), rep
        assert float(noise) == float(noise)
    assert (gs_k.n_blocks, gs_k.n_tail) != (n0, t0)            # host counters advanced once, at capture


# ------------------------------------------------------------------ append --
@pytest.mark.parametrize("R,S,kfmt,vfmt,T0,steps", [
    (8, 3, "i8", "bf16", 8 * 10 + 5, 30),
    (16, 4, "i8", "i8", 16 * 3, 40),
    (4, 4, "f32", "f32", 0, 13),
    (1, 1, "i8", "i8", 3, 5),
])
def test_append_matches_encode_and_never_rewrites(R, S, kfmt, vfmt, T0, steps):
    note("append", R, S, kfmt, vfmt, T0, steps)
    B, Hq, H, D = 2, 8, 2, 128
    k, v, _ = syn.small_case(B, Hq, H, D, T0 + steps, seed=R + S)
    ks = bd.CodecStream(B, H, D, R, S, fmt=kfmt, device=DEV)
    vs = bd.CodecStream(B, H, D, R, S, fmt=vfmt, device=DEV)
    kd, vd = k.to(DEV), v.to(DEV)
    ks.encode(kd[:, :, :T0])
    vs.encode(vd[:, :, :T0])
    frozen = []
    for t in range(T0, T0 + steps):
        bd.append_step(ks, vs, kd[:, :, t:t + 1], vd[:, :, t:t + 1])
        assert ks.seq_len == t + 1 and vs.seq_len == t + 1
        n = ks.n_blocks
        if n > len(frozen):
            frozen.append((ks.rows[:, :, len(frozen)].clone(), None if ks.scales is None else ks.scales[:, :, len(frozen)].clone()))
        for i, (r, s) in enumerate(frozen):
            assert torch.equal(ks.rows[:, :, i], r)
            if s is not None:
                assert torch.equal(ks.scales[:, :, i], s)
        if t % 7 == 3 or t == T0 + steps - 1:
            q = syn.gaussian((B, Hq, 1, D), 1000 + t)
            out = bd.decode_attention(q.to(DEV), ks, vs)
            torch.cuda.synchronize()
            ref = O.decode_attention(syn.bf16_to_numpy(q), gpu_archive(ks), gpu_archive(vs))
            assert rel_err(out.cpu().numpy()[:, :, 0], ref) <= TOL
    # the streamed archive equals one encode of the whole sequence
    k2, v2 = make_streams(k, v, R, S, kfmt, vfmt)
    torch.cuda.synchronize()
    assert_archive_equal(gpu_archive(ks), gpu_archive(k2))
    assert_archive_equal(gpu_archive(vs), gpu_archive(v2))
    assert_archive_equal(gpu_archive(ks), O.encode(syn.bf16_to_numpy(k), R, S, kfmt))
