"""Parity at the full sizes of the five synthetic workloads, through the C ABI
and in the launch configuration the benchmark times (the decode plan is a
function of the shapes only).  The oracle recomputes sampled (batch, kv head)
pairs one at a time: encoded rows and scales bit-exact, every query head of
a sampled pair within the 2e-3 output tolerance.  Inputs are drawn on the
device (synthetic.workload_kv_device), the oracle gets the same bf16 bytes."""

import numpy as np
import pytest
import torch

import oracle as O
from compressed_domain_attention_amd import binding as bd
from compressed_domain_attention_amd import synthetic as syn
from parity_util import TOL, assert_archive_equal, gpu_head_archive, note, rel_err

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")


def encode_streams(w, k, v, capacity=0):
    ks = bd.CodecStream(w.B, w.Hkv, w.D, w.R, w.S, fmt=w.kfmt, device=DEV, capacity=capacity)
    vs = bd.CodecStream(w.B, w.Hkv, w.D, w.R, w.S, fmt=w.vfmt, device=DEV, capacity=capacity)
    ks.encode(k[:, :, :w.T])
    vs.encode(v[:, :, :w.T])
    return ks, vs


def check_encode(w, st, x, fmt, heads, T):
    for (b, h) in heads:
        want = O.encode(syn.bf16_to_numpy(x[b:b + 1, h:h + 1, :T]), w.R, w.S, fmt)
        assert_archive_equal(gpu_head_archive(st, b, h), want)


def check_decode(w, q, out, ks, vs, heads):
    """Every query head of the sampled kv heads against the oracle."""
    G = w.G
    qn = syn.bf16_to_numpy(q)
    for (b, h) in heads:
        ka, va = gpu_head_archive(ks, b, h), gpu_head_archive(vs, b, h)
        ref = O.decode_attention(qn[b:b + 1, h * G:(h + 1) * G], ka, va)
        got = out[b:b + 1, h * G:(h + 1) * G, 0].float().cpu().numpy()
        err = rel_err(got, ref)
        assert err <= TOL, ((b, h), err)


def sample_heads(w, n, seed):
    rng = np.random.default_rng(seed)
    allp = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    if n >= len(allp):
        return allp
    idx = rng.choice(len(allp), size=n, replace=False)
    return [allp[i] for i in sorted(idx)]


@pytest.mark.parametrize("name,n_enc,n_dec", [
    ("tiny", 2, 2),
    ("llama8b_layer", 8, 64),
    ("long128k", 2, 8),
    ("batch64_gqa8", 4, 6),
])
def test_fullsize_encode_and_decode(name, n_enc, n_dec):
    w = syn.WORKLOADS[name]
    note("fullsize", name)
    k, v = syn.workload_kv_device(w, device=DEV)
    ks, vs = encode_streams(w, k, v)
    torch.cuda.synchronize()
    assert ks.n_blocks == w.n_blocks and ks.n_tail == w.n_tail
    enc = sample_heads(w, n_enc, 11)
    check_encode(w, ks, k, w.kfmt, enc, w.T)
    check_encode(w, vs, v, w.vfmt, enc, w.T)
    q = syn.workload_query(w, 0).to(DEV)
    out = bd.decode_attention(q, ks, vs)
    torch.cuda.synchronize()
    check_decode(w, q, out, ks, vs, sample_heads(w, n_dec, 12))


def test_fullsize_streaming():
    """64 append + decode steps from T = 32760 (a block archived every 8
    steps), as in the benchmark's step; decode checked at three steps, and
    the final archive equal to encoding the whole sequence at once."""
    w = syn.WORKLOADS["stream64"]
    note("fullsize", w.name)
    k, v = syn.workload_kv_device(w, device=DEV)
    ks, vs = encode_streams(w, k, v, capacity=(w.T + w.steps) // w.R + 1)
    heads = sample_heads(w, 4, 13)
    for s in range(w.steps):
        t = w.T + s
        bd.append_step(ks, vs, k[:, :, t:t + 1], v[:, :, t:t + 1])
        if s in (0, 31, w.steps - 1):
            q = syn.workload_query(w, s).to(DEV)
            out = bd.decode_attention(q, ks, vs)
            torch.cuda.synchronize()
            check_decode(w, q, out, ks, vs, heads)
    torch.cuda.synchronize()
    T1 = w.T + w.steps
    assert ks.n_blocks * w.R + ks.n_tail == T1
    check_encode(w, ks, k, w.kfmt, heads[:2], T1)
    check_encode(w, vs, v, w.vfmt, heads[:2], T1)
