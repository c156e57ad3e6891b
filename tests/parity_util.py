"""Helpers shared by the GPU parity tests: moving archives between the HIP
path's device tensors and the oracle's numpy form, and the error measure.
No method arithmetic lives here."""

import sys

import numpy as np
import torch

import oracle as O
from compressed_domain_attention_amd import binding as bd
from compressed_domain_attention_amd import synthetic as syn

FMT_NAME = {bd.FMT_F32: O.F32, bd.FMT_BF16: O.BF16, bd.FMT_I8: O.I8, bd.FMT_PNG: O.PNG}
TOL = 2e-3   # max over (b, hq) of ||o - o_ref||_inf / ||o_ref||_inf


def note(*a):
    """Name the case on stdout before a GPU step (survives a lost box)."""
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def rows_to_numpy(t, fmt):
    t = t.detach().cpu().contiguous()
    if fmt == bd.FMT_BF16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def gpu_archive(st):
    """The GPU stream's archive in the oracle's dict form (identical bytes)."""
    n = st.n_blocks
    rows = rows_to_numpy(st.rows[:, :, :n], st.fmt)
    scales = st.scales[:, :, :n].detach().cpu().numpy() if st.fmt == bd.FMT_I8 else None
    tail = syn.bf16_to_numpy(st.tail[:, :, :st.n_tail])
    return dict(fmt=FMT_NAME[st.fmt], R=st.R, S=st.S, rows=rows, scales=scales, tail=tail, n_blocks=n)


def gpu_head_archive(st, b, h):
    """One (b, kv head) of the GPU stream's archive in the oracle's dict form,
    shaped as a batch of one with one head."""
    n = st.n_blocks
    rows = rows_to_numpy(st.rows[b:b + 1, h:h + 1, :n], st.fmt)
    scales = st.scales[b:b + 1, h:h + 1, :n].detach().cpu().numpy() if st.fmt == bd.FMT_I8 else None
    tail = syn.bf16_to_numpy(st.tail[b:b + 1, h:h + 1, :st.n_tail].cpu())
    return dict(fmt=FMT_NAME[st.fmt], R=st.R, S=st.S, rows=rows, scales=scales, tail=tail, n_blocks=n)


def assert_archive_equal(got, want, blocks=None):
    """Bit-exact rows / scales / tail (optionally only for listed (b, h, n))."""
    if blocks is None:
        assert got["rows"].shape == want["rows"].shape, (got["rows"].shape, want["rows"].shape)
        assert got["rows"].tobytes() == np.ascontiguousarray(want["rows"]).tobytes(), \
            f"rows differ at {np.argwhere(got['rows'] != want['rows'])[:5].tolist()}"
        if want["scales"] is not None:
            assert got["scales"].tobytes() == np.ascontiguousarray(want["scales"]).tobytes(), "scales differ"
        assert np.array_equal(got["tail"], want["tail"]), "tail differs"
    else:
        for (b, h, n) in blocks:
            assert got["rows"][b, h, n].tobytes() == want["rows"][b, h, n].tobytes(), (b, h, n)
            if want["scales"] is not None:
                assert got["scales"][b, h, n].tobytes() == want["scales"][b, h, n].tobytes(), (b, h, n)


def rel_err(got, ref):
    """Per (b, hq): ||got - ref||_inf / ||ref||_inf; returns the max."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return float((num / den).max())


def make_streams(k, v, R, S, kfmt, vfmt, dev="cuda", raw=None, capacity=0):
    raw = raw or ("bf16" if k.dtype == torch.bfloat16 else "f32")
    B, H, T, D = k.shape
    ks = bd.CodecStream(B, H, D, R, S, fmt=kfmt, raw_dtype=raw, device=dev, capacity=capacity)
    vs = bd.CodecStream(B, H, D, R, S, fmt=vfmt, raw_dtype=raw, device=dev, capacity=capacity)
    ks.encode(k.to(dev))
    vs.encode(v.to(dev))
    return ks, vs
