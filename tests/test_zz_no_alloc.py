"""codec_decode_attention_noalloc (no workspace argument: the split partials
live in the library's per-GPU scratch array) against codec_decode_attention
with a caller workspace: identical outputs bit for bit, on two calls in a
row (the second with a smaller input), for plans with many splits and with
one split, and under a HIP graph replayed several times."""

import pytest
import torch

from compressed_domain_attention_amd import binding as bd
from compressed_domain_attention_amd import synthetic as syn
from parity_util import make_streams, note

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(B, Hq, H, D, R, S, kfmt, vfmt, T, seed):
    k, v, q = syn.small_case(B, Hq, H, D, T, seed=seed, offset_var=1.0)
    ks, vs = make_streams(k, v, R, S, kfmt, vfmt)
    return q.to(DEV), ks, vs


@pytest.mark.parametrize("first,second", [
    # many splits (one pair per kv head of a single row), then a smaller input
    ((1, 32, 8, 128, 16, 4, "i8", "i8", 16 * 3000 + 5, 1), (1, 8, 2, 128, 16, 4, "i8", "i8", 16 * 500 + 3, 2)),
    # one split per pair (256 pairs), then a smaller many-split input
    # (58 tiles per pair: 8 splits)
    ((32, 32, 8, 128, 8, 2, "i8", "i8", 8 * 400, 3), (1, 4, 2, 64, 8, 2, "i8", "bf16", 8 * 1200 + 7, 4)),
])
def test_noalloc_equals_workspace_call(first, second):
    for case in (first, second):
        note("noalloc", case)
        q, ks, vs = _case(*case)
        want = bd.decode_attention(q, ks, vs)
        out = torch.full_like(want, float("nan"))
        got = bd.decode_attention_noalloc(q, ks, vs, out=out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(got, want), (case, (got - want).abs().max().item())
        # a second call on the same scratch: the counters reset themselves
        again = bd.decode_attention_noalloc(q, ks, vs)
        torch.cuda.synchronize()
        assert torch.equal(again, want)


def test_noalloc_graph_replays():
    note("noalloc graph")
    q, ks, vs = _case(1, 32, 8, 128, 16, 4, "i8", "i8", 16 * 2000 + 9, 5)
    want = bd.decode_attention(q, ks, vs).clone()
    out = torch.empty_like(want)
    bd.decode_attention_noalloc(q, ks, vs, out=out)        # first call on the device: outside the capture
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        bd.decode_attention_noalloc(q, ks, vs, out=out)
    for rep in range(4):
        out.fill_(float("nan"))
        noise = torch.randn(1 << 20, device=DEV).sum()       # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), rep
        assert float(noise) == float(noise)
