"""The layer stack (CodecLayerStack: the archives of L layers in one
allocation, one launch per step across layers) through the C ABI, against
the fp64 oracle layer by layer: prefill of all layers in one encode launch
per side, bit-exact codes, scales and tails per layer; one decode launch for
every layer within 2e-3 of each layer's oracle decode; decode steps that
append every layer's token (across block boundaries and a capacity
doubling) after a prefill done layer by layer through the per-layer views;
and a stack-wide crop and beam reorder."""

import numpy as np
import pytest
import torch

import oracle as O
from compressed_domain_attention_amd import binding as bd
from compressed_domain_attention_amd import synthetic as syn
from parity_util import TOL, assert_archive_equal, gpu_archive, note, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda"
OF = {"i8": O.I8, "bf16": O.BF16, "f32": O.F32}


def layer_tokens(L, B, Hq, H, D, T, seed, dtype=torch.bfloat16):
    """Per-layer K, V (L, B, H, T, D) and queries (L, B, Hq, 1, D) on the CPU."""
    ks, vs, qs = zip(*[syn.small_case(B, Hq, H, D, T, seed=seed + 17 * l, dtype=dtype) for l in range(L)])
    return torch.stack(ks), torch.stack(vs), torch.stack(qs)


def check_layers(stack, k, v, q, out, kfmt, vfmt, T):
    """Every layer's archive bit-exact against the oracle's encode of its T
    tokens, and its output within TOL of the oracle's decode."""
    R, S = stack.k.R, stack.k.S
    for l in range(stack.L):
        kl, vl = stack.layer(l)
        assert (kl.n_blocks, kl.n_tail) == (T // R, T % R)
        kw = O.encode(syn.bf16_to_numpy(k[l, :, :, :T]), R, S, OF[kfmt])
        vw = O.encode(syn.bf16_to_numpy(v[l, :, :, :T]), R, S, OF[vfmt])
        assert_archive_equal(gpu_archive(kl), kw)
        assert_archive_equal(gpu_archive(vl), vw)
        ref = O.decode_attention(syn.bf16_to_numpy(q[l]), kw, vw)
        err = rel_err(out[l, :, :, 0].float().cpu().numpy(), ref)
        assert err <= TOL, (l, err)


@pytest.mark.parametrize("kfmt,vfmt,L,B,Hq,H,D,R,S,T", [
    ("i8", "i8", 3, 2, 8, 2, 128, 8, 2, 8 * 40 + 5),
    ("i8", "bf16", 4, 1, 16, 2, 128, 16, 4, 16 * 300 + 9),   # five splits per pair
    ("bf16", "bf16", 2, 3, 4, 2, 64, 8, 3, 8 * 25),
])
def test_stack_prefill_and_one_launch_decode(kfmt, vfmt, L, B, Hq, H, D, R, S, T):
    note("layer stack prefill + decode", kfmt, vfmt, L, B, Hq, H, D, R, S, T)
    k, v, q = layer_tokens(L, B, Hq, H, D, T, seed=R + S)
    st = bd.CodecLayerStack(L, B, H, D, R, S, k_fmt=kfmt, v_fmt=vfmt, device=DEV)
    st.encode(k.to(DEV), v.to(DEV))
    out = st.decode(q.to(DEV))
    torch.cuda.synchronize()
    assert out.shape == (L, B, Hq, 1, D)
    check_layers(st, k, v, q, out, kfmt, vfmt, T)
    # one layer through its views gives that layer's decode too
    for l in (0, L - 1):
        ol = bd.decode_attention(q[l].to(DEV), *st.layer(l))
        ref = O.decode_attention(syn.bf16_to_numpy(q[l]), gpu_archive(st.layer(l)[0]), gpu_archive(st.layer(l)[1]))
        assert rel_err(ol[:, :, 0].float().cpu().numpy(), ref) <= TOL


def test_stack_steps_after_per_layer_prefill():
    """Prefill layer by layer through the views, then stack-wide decode steps
    that append every layer's token: blocks complete (R = 8) and the archive
    outgrows its first capacity of 16 blocks."""
    L, B, Hq, H, D, R, S = 3, 2, 8, 2, 128, 8, 2
    T0, steps = 8 * 16 + 5, 2 * 8 + 4
    note("layer stack steps", L, B, Hq, H, D, R, S, T0, steps)
    k, v, _ = layer_tokens(L, B, Hq, H, D, T0 + steps, seed=41)
    st = bd.CodecLayerStack(L, B, H, D, R, S, k_fmt="i8", device=DEV)
    for l in range(L):
        kl, vl = st.layer(l)
        kl.encode(k[l, :, :, :T0].to(DEV).contiguous())
        vl.encode(v[l, :, :, :T0].to(DEV).contiguous())
    assert st.capacity == 16
    for s in range(steps):
        t = T0 + s
        q = torch.stack([syn.gaussian((B, Hq, 1, D), 900 + 10 * s + l) for l in range(L)])
        kn = k[:, :, :, t:t + 1].to(DEV).contiguous()
        vn = v[:, :, :, t:t + 1].to(DEV).contiguous()
        out = st.decode_append(q.to(DEV), kn, vn)
        torch.cuda.synchronize()
        if s in (2, 3, 11, steps - 1):
            check_layers(st, k, v, q, out, "i8", "i8", t + 1)
    assert st.capacity == 32


def test_stack_crop_and_beam_reorder():
    L, B, Hq, H, D, R, S = 2, 3, 4, 2, 64, 8, 2
    T = 8 * 12 + 6
    note("layer stack crop + select_batch", L, B, Hq, H, D, R, S, T)
    k, v, q = layer_tokens(L, B, Hq, H, D, T, seed=5)
    st = bd.CodecLayerStack(L, B, H, D, R, S, k_fmt="i8", device=DEV)
    st.encode(k.to(DEV), v.to(DEV))
    keep = 8 * 9 + 3   # inside the archive: block 9 leaves it, its first 3 tokens become the tail
    st.crop(keep)
    idx = [2, 0, 2]
    st.select_batch(idx)
    assert st.B == 3 and st.seq_len == keep
    qq = q[:, idx]
    out = st.decode(qq.to(DEV))
    torch.cuda.synchronize()
    for l in range(L):
        for side, x in zip(st.layer(l), (k, v)):
            want = O.select_batch(O.crop(O.encode(syn.bf16_to_numpy(x[l]), R, S, O.I8), keep, O.BF16), idx)
            assert_archive_equal(gpu_archive(side), want)
        ref = O.decode_attention(syn.bf16_to_numpy(qq[l]), gpu_archive(st.layer(l)[0]), gpu_archive(st.layer(l)[1]))
        assert rel_err(out[l, :, :, 0].float().cpu().numpy(), ref) <= TOL


def test_stack_matches_separate_streams_bitwise_per_layer_call():
    """A layer's decode through its view equals the same decode on a separate
    stream holding the same tokens, bit for bit (same plan, same kernels)."""
    L, B, Hq, H, D, R, S, T = 2, 2, 8, 2, 128, 16, 4, 16 * 50 + 3
    note("layer stack view == separate stream", L, B, Hq, H, D, R, S, T)
    k, v, q = layer_tokens(L, B, Hq, H, D, T, seed=77)
    st = bd.CodecLayerStack(L, B, H, D, R, S, k_fmt="i8", device=DEV)
    st.encode(k.to(DEV), v.to(DEV))
    for l in range(L):
        ks = bd.CodecStream(B, H, D, R, S, fmt="i8", device=DEV)
        vs = bd.CodecStream(B, H, D, R, S, fmt="i8", device=DEV)
        ks.encode(k[l].to(DEV))
        vs.encode(v[l].to(DEV))
        a = bd.decode_attention(q[l].to(DEV), *st.layer(l))
        b = bd.decode_attention(q[l].to(DEV), ks, vs)
        torch.cuda.synchronize()
        assert torch.equal(a, b)
        assert np.array_equal(gpu_archive(st.layer(l)[0])["rows"], gpu_archive(ks)["rows"])
