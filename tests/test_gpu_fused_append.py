"""codec_decode_attention_append (one launch for a decode step that appends
a token) against the two-call sequence codec_append_step +
codec_decode_attention: identical outputs bit for bit, identical archives
and tails, across block boundaries, for every row format, with one and two
query groups per kv head; and against the fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle as O
from compressed_domain_attention_amd import binding as bd
from compressed_domain_attention_amd import synthetic as syn
from parity_util import TOL, assert_archive_equal, gpu_archive, make_streams, note, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("fmt,raw,R,S,B,Hq,H,D,T0", [
    ("i8", "bf16", 8, 2, 2, 8, 2, 128, 8 * 20 + 3),
    ("i8", "bf16", 16, 4, 1, 32, 2, 128, 16 * 40),       # two query groups per kv head, empty tail at start
    ("bf16", "bf16", 8, 3, 2, 4, 2, 64, 8 * 7 + 6),
    ("f32", "f32", 4, 2, 1, 4, 1, 256, 4 * 9 + 1),
    ("png", "bf16", 8, 8, 1, 8, 2, 128, 8 * 11 + 5),
    ("i8", "bf16", 8, 2, 1, 4, 1, 128, 3),               # tail only at start
    # the benchmark's 128K-context constants (GQA 4, R = 16, S = 4, int8 keys
    # and values, five tail tokens at the start) on a shorter sequence
    ("i8", "bf16", 16, 4, 1, 32, 8, 128, 16 * 600 + 5),
])
def test_fused_equals_two_calls(fmt, raw, R, S, B, Hq, H, D, T0):
    note("fused append", fmt, raw, R, S, B, Hq, H, D, T0)
    steps = 2 * R + 3
    dt = torch.bfloat16 if raw == "bf16" else torch.float32
    k, v, _ = syn.small_case(B, Hq, H, D, T0 + steps, seed=R * 13 + S, dtype=dt)
    ka, va = make_streams(k[:, :, :T0], v[:, :, :T0], R, S, fmt, fmt, raw=raw)
    kb, vb = make_streams(k[:, :, :T0], v[:, :, :T0], R, S, fmt, fmt, raw=raw)
    for s in range(steps):
        t = T0 + s
        q = syn.gaussian((B, Hq, 1, D), 500 + s).to(DEV)
        kn, vn = k[:, :, t:t + 1].to(DEV).contiguous(), v[:, :, t:t + 1].to(DEV).contiguous()
        bd.append_step(ka, va, kn, vn)
        oa = bd.decode_attention(q, ka, va)
        ob = bd.decode_attention_append(q, kb, vb, kn, vn)
        torch.cuda.synchronize()
        assert (kb.n_blocks, kb.n_tail) == (ka.n_blocks, ka.n_tail)
        assert torch.equal(oa, ob), (s, (oa - ob).abs().max().item())
        if s in (0, R - 1, steps - 1):
            assert_archive_equal(gpu_archive(kb), gpu_archive(ka))
            assert_archive_equal(gpu_archive(vb), gpu_archive(va))
            ref = O.decode_attention(syn.bf16_to_numpy(q.cpu()), gpu_archive(kb), gpu_archive(vb))
            assert rel_err(ob[:, :, 0].float().cpu().numpy(), ref) <= TOL


@pytest.mark.parametrize("kfmt,vfmt,R,S,B,Hq,H,D,T0", [
    # the large-batch GQA-8 constants (eight-head groups, int8 keys, bf16
    # values, R = 8, S = 3; the raw tail runs after the tail wave's tiles),
    # one split per pair and several
    ("i8", "bf16", 8, 3, 2, 16, 2, 128, 8 * 150 + 2),     # one split per pair
    ("i8", "bf16", 8, 3, 1, 16, 2, 128, 8 * 600 + 1),
    # head_dim 256 and 32 kept rows (also tail after the tiles)
    ("i8", "i8", 16, 4, 1, 8, 2, 256, 16 * 70 + 3),
    ("i8", "i8", 32, 32, 1, 8, 2, 64, 32 * 9 + 5),
])
def test_fused_tail_after_tiles(kfmt, vfmt, R, S, B, Hq, H, D, T0):
    note("fused append, tail after tiles", kfmt, vfmt, R, S, B, Hq, H, D, T0)
    steps = R + 3
    k, v, _ = syn.small_case(B, Hq, H, D, T0 + steps, seed=R * 7 + S + D)
    ka, va = make_streams(k[:, :, :T0], v[:, :, :T0], R, S, kfmt, vfmt)
    kb, vb = make_streams(k[:, :, :T0], v[:, :, :T0], R, S, kfmt, vfmt)
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
            ref = O.decode_attention(syn.bf16_to_numpy(q.cpu()), gpu_archive(kb), gpu_archive(vb))
            assert rel_err(ob[:, :, 0].float().cpu().numpy(), ref) <= TOL
