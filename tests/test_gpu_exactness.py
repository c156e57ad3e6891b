"""GPU decode against attention on the raw tokens when nothing is dropped, and
against the oracle when the largest logits sit in the raw tail or in a block
streamed after it.

With every frequency kept (S = R) in fp32 rows, the orthonormal transform
loses only the fp32 rounding of the coefficients and of the basis (page 4
README, "Math": the DCT is orthonormal, so keeping all R rows reconstructs
the block), and the decode equals softmax attention on the raw bf16 tokens
up to fp32 arithmetic.  The raw attention here is the plain definition in
fp64, written in this file; it is not the oracle.

The raw tail is summed before the tiles by one wave of the last split
(page 4 `triton_attention.py`: every token of the tail attended exactly),
and the tiles' online softmax rescales what came before whenever the running
maximum grows (the (max, sum, acc) rule of the split kernel).  Planting the
largest key of a head in an archive block makes the maximum grow after the
tail; planting it in the tail keeps it there."""

import numpy as np
import pytest
import torch

import oracle as O
from compressed_domain_attention_amd import binding as bd
from compressed_domain_attention_amd import synthetic as syn
from parity_util import TOL, gpu_archive, make_streams, note, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda"
RAW_TOL = 1e-6   # fp32 coefficients, basis and arithmetic against fp64 on the raw tokens


def raw_attention(q, k, v):
    """softmax(q . k / sqrt(D)) v per query head, in fp64 on the raw tokens
    (query head hq reads kv head hq / (Hq / H))."""
    B, Hq, _, D = q.shape
    H = k.shape[1]
    G = Hq // H
    out = np.zeros((B, Hq, D))
    for b in range(B):
        for hq in range(Hq):
            kk, vv = k[b, hq // G], v[b, hq // G]
            s = kk @ q[b, hq, 0] / np.sqrt(D)
            p = np.exp(s - s.max())
            out[b, hq] = (p / p.sum()) @ vv
    return out


@pytest.mark.parametrize("B,Hq,H,D,R,T", [
    (1, 4, 2, 64, 8, 8 * 50 + 4),
    (1, 8, 2, 64, 16, 16 * 40 + 7),      # fp32 rows hold S <= 16 per decode tile at head_dim 64, 8 at 128
    (2, 8, 2, 128, 8, 8 * 120 + 5),
    (1, 16, 2, 96, 8, 8 * 300 + 3),      # many splits, eight-head groups, padded head_dim
])
def test_all_frequencies_fp32_rows_equal_raw_attention(B, Hq, H, D, R, T):
    note("S = R fp32 rows vs raw attention", B, Hq, H, D, R, T)
    k, v, q = syn.small_case(B, Hq, H, D, T, seed=R + D)
    ks, vs = make_streams(k, v, R, R, "f32", "f32")
    out = bd.decode_attention(q.to(DEV), ks, vs)
    torch.cuda.synchronize()
    got = out[:, :, 0].float().cpu().numpy()
    want = raw_attention(syn.bf16_to_numpy(q), syn.bf16_to_numpy(k), syn.bf16_to_numpy(v))
    err = rel_err(got, want)
    note("max relative error", err)
    assert err <= RAW_TOL, err


def planted(k, q, tokens, G):
    """K with, for every (b, kv head), the keys at `tokens` set to a multiple
    of the group's first query (their logits far above the rest)."""
    k = k.clone()
    for b in range(k.shape[0]):
        for h in range(k.shape[1]):
            qq = q[b, h * G, 0].float()
            k[b, h, tokens] = (qq * (24.0 * np.sqrt(k.shape[3]) / float(qq.dot(qq)))).to(k.dtype)
    return k


@pytest.mark.parametrize("kfmt,vfmt", [("i8", "i8"), ("i8", "bf16"), ("f32", "f32")])
@pytest.mark.parametrize("place", ["tail", "blocks"])
def test_maximum_in_the_tail_or_after_it(kfmt, vfmt, place):
    # 8 (b, kv head) pairs with one query group each, 2560 blocks of 8 tokens
    # and 8 blocks per tile: 32 splits of 10 tiles, so with a raw tail the
    # last split keeps 9 and its wave 1 runs the tail and then one tile.
    # "blocks": the first token of every block is planted, so that tile's
    # logits exceed the tail's and the tail's sums are rescaled after it;
    # "tail": one tail token is planted and holds the maximum throughout.
    B, Hq, H, D, R, S = 1, 32, 8, 128, 8, 4
    T = 8 * 2560 + 6
    tokens = [T - 3] if place == "tail" else list(range(0, 8 * 2560, 8))
    note("planted maximum", kfmt, vfmt, place, len(tokens))
    k, v, q = syn.small_case(B, Hq, H, D, T, seed=17)
    k = planted(k, q, tokens, Hq // H)
    ks, vs = make_streams(k, v, R, S, kfmt, vfmt)
    assert (ks.n_blocks, ks.n_tail) == (2560, 6)
    out = bd.decode_attention(q.to(DEV), ks, vs)
    torch.cuda.synchronize()
    ref = O.decode_attention(syn.bf16_to_numpy(q), gpu_archive(ks), gpu_archive(vs))
    assert rel_err(out[:, :, 0].float().cpu().numpy(), ref) <= TOL
