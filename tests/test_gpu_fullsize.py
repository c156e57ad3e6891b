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
from parity_util import TOL, assert_archive_equal, gpu_archive, gpu_head_archive, note, rel_err

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
    """64 decode steps from T = 32760 through codec_decode_attention_append
    (the benchmark's step: the token is appended inside the decode launch,
    and a block is archived every 8 steps).  The decode is checked against
    the oracle at steps 1, 7, 8, 9, 16 and 64 for four sampled kv heads, and
    at every step for one kv head in each of batch rows 0 and 31; the final
    archive equals encoding the whole sequence at once."""
    w = syn.WORKLOADS["stream64"]
    note("fullsize fused streaming", w.name)
    k, v = syn.workload_kv_device(w, device=DEV)
    ks, vs = encode_streams(w, k, v, capacity=(w.T + w.steps) // w.R + 1)
    heads = sample_heads(w, 4, 13)
    rng = np.random.default_rng(17)
    every = [(0, int(rng.integers(w.Hkv))), (w.B - 1, int(rng.integers(w.Hkv)))]
    out = torch.empty((w.B, w.Hq, 1, w.D), dtype=torch.float32, device=DEV)
    for s in range(1, w.steps + 1):
        t = w.T + s - 1
        q = syn.workload_query(w, s).to(DEV)
        bd.decode_attention_append(q, ks, vs, k[:, :, t:t + 1], v[:, :, t:t + 1], out=out)
        torch.cuda.synchronize()
        assert ks.n_blocks * w.R + ks.n_tail == t + 1
        pairs = every + (heads if s in (1, 7, 8, 9, 16, 64) else [])
        check_decode(w, q, out, ks, vs, pairs)
    T1 = w.T + w.steps
    check_encode(w, ks, k, w.kfmt, heads[:2], T1)
    check_encode(w, vs, v, w.vfmt, heads[:2], T1)


def test_fullsize_long_context_fused_steps():
    """The benchmarked call at its own shape: 35 steps of
    codec_decode_attention_append on the 128K-context workload (five tail
    tokens at the start, so blocks complete at steps 11 and 27), checked
    against the oracle at steps 1, 11, 12, 27 and 35 on two kv heads."""
    w = syn.WORKLOADS["long128k"]
    steps = 2 * w.R + 3
    note("fullsize fused steps", w.name, steps)
    k, v = syn.workload_kv_device(w, T=w.T + steps, device=DEV)
    ks, vs = encode_streams(w, k, v, capacity=(w.T + steps) // w.R + 1)
    heads = sample_heads(w, 2, 19)
    out = torch.empty((w.B, w.Hq, 1, w.D), dtype=torch.float32, device=DEV)
    for s in range(1, steps + 1):
        t = w.T + s - 1
        q = syn.workload_query(w, s).to(DEV)
        bd.decode_attention_append(q, ks, vs, k[:, :, t:t + 1], v[:, :, t:t + 1], out=out)
        if s in (1, 11, 12, 27, steps):
            torch.cuda.synchronize()
            assert ks.n_blocks * w.R + ks.n_tail == t + 1
            check_decode(w, q, out, ks, vs, heads)
    torch.cuda.synchronize()
    check_encode(w, ks, k, w.kfmt, heads[:1], w.T + steps)


def _ns_from_workspace(nbytes, pairs, GS, D):
    """Split count of a decode from its workspace size: a 256 KiB counter
    region, then (max, sum) pairs (256-byte aligned) and the D-wide
    partial accumulators, each per (pair, split, head)."""
    for ns in range(1, 257):
        ml = -(-(pairs * ns * GS * 8) // 256) * 256
        if 262144 + ml + pairs * ns * GS * D * 4 == nbytes:
            return ns
    raise AssertionError(f"workspace size {nbytes} matches no split count")


def test_split_count_invariance():
    """The same (batch row, kv head) archives decoded with 32, 4 and 1
    splits (batch of 1, 8 and 32 rows: the split count follows the number
    of (row, head) pairs): batch row 0 agrees with the oracle and across the
    three within the output tolerance."""
    B0, Hq, H, D, R, S, T = 1, 32, 8, 128, 16, 4, 16 * 2000 + 5
    note("split count invariance", T)
    k4, v4, _ = syn.small_case(4, Hq, H, D, T, seed=41, offset_var=2.0)
    k, v = k4.repeat(8, 1, 1, 1), v4.repeat(8, 1, 1, 1)     # 32 rows; row 0 is the same everywhere
    q = syn.gaussian((32, Hq, 1, D), 4102)
    outs, nss = [], []
    for B in (1, 8, 32):
        ks, vs = bd.CodecStream(B, H, D, R, S, fmt="i8", device=DEV), bd.CodecStream(B, H, D, R, S, fmt="i8", device=DEV)
        ks.encode(k[:B].to(DEV))
        vs.encode(v[:B].to(DEV))
        nss.append(_ns_from_workspace(bd.decode_workspace_bytes(ks, vs, Hq), B * H, 4, D))
        out = bd.decode_attention(q[:B].to(DEV), ks, vs)
        torch.cuda.synchronize()
        outs.append(out[:B0, :, 0].float().cpu().numpy())
        if B == 1:
            ref = O.decode_attention(syn.bf16_to_numpy(q[:1]), gpu_archive(ks), gpu_archive(vs))
    assert nss == [32, 4, 1], nss
    for o in outs:
        assert rel_err(o, ref) <= TOL
    for o in outs[1:]:
        assert rel_err(o, outs[0]) <= TOL
