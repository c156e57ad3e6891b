"""GPU parity of PNG mode (anchor + first-order deltas, README "Math", PNG
item) through the C ABI: rows bit-exact against the oracle, the lossless
round trip through the materialised view, decode attention within the 2e-3
tolerance (and, the tier being lossless, against attention on the raw
tokens), and appends across block boundaries."""

import numpy as np
import pytest
import torch

import oracle as O
from compressed_domain_attention_amd import binding as bd
from compressed_domain_attention_amd import synthetic as syn
from parity_util import TOL, assert_archive_equal, gpu_archive, make_streams, note, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [
    # D, R, raw, B, Hq, H, T
    (128, 8, "bf16", 2, 8, 2, 8 * 41 + 5),
    (64, 16, "bf16", 1, 4, 2, 16 * 19 + 15),
    (256, 4, "f32", 1, 2, 2, 4 * 30 + 1),
    (128, 1, "bf16", 1, 4, 4, 37),
    (128, 8, "bf16", 1, 16, 1, 8 * 300),
]


@pytest.mark.parametrize("D,R,raw,B,Hq,H,T", CASES)
def test_png_encode_view_decode(D, R, raw, B, Hq, H, T):
    note("png", D, R, raw, B, Hq, H, T)
    dt = torch.bfloat16 if raw == "bf16" else torch.float32
    k, v, q = syn.small_case(B, Hq, H, D, T, seed=5 * R + D, dtype=dt)
    ks, vs = make_streams(k, v, R, R, "png", "png")
    torch.cuda.synchronize()
    kx, vx = syn.bf16_to_numpy(k), syn.bf16_to_numpy(v)
    ka, va = gpu_archive(ks), gpu_archive(vs)
    assert_archive_equal(ka, O.encode(kx, R, R, O.PNG))
    assert_archive_equal(va, O.encode(vx, R, R, O.PNG))
    # the view equals the oracle's bit for bit; for bf16 tokens it gives the
    # tokens back exactly (the lossless tier), for fp32 tokens the fp32
    # rounding of the deltas leaves an error of a few ulp
    view = ks.read()
    torch.cuda.synchronize()
    vw = view.cpu()
    want = O.view(ka, O.BF16 if raw == "bf16" else O.F32)
    if raw == "bf16":
        assert np.array_equal(vw.view(torch.int16).numpy().view(np.uint16), want)
        assert torch.equal(vw, k)
    else:
        assert np.array_equal(vw.numpy(), want)
        assert np.abs(vw.numpy() - kx).max() <= 1e-5 * np.abs(kx).max()
    # decode attention: oracle on the identical archive, and raw attention
    out = bd.decode_attention(q.to(DEV), ks, vs)
    got = out[:, :, 0].float().cpu().numpy()
    qn = syn.bf16_to_numpy(q)
    ref = O.decode_attention(qn, ka, va)
    assert rel_err(got, ref) <= TOL
    raw_ref = O.attention(qn[:, :, 0], kx, vx, D ** -0.5)
    assert rel_err(got, raw_ref) <= TOL


def test_png_append_across_blocks():
    note("png append")
    B, Hq, H, D, R = 2, 8, 2, 128, 8
    T0, steps = 8 * 6 + 2, 30
    k, v, q = syn.small_case(B, Hq, H, D, T0 + steps, seed=71)
    ks, vs = make_streams(k[:, :, :T0], v[:, :, :T0], R, R, "png", "png")
    ko, vo = O.Stream(R, R, O.PNG), O.Stream(R, R, O.PNG)
    ko.append(syn.bf16_to_numpy(k[:, :, :T0]))
    vo.append(syn.bf16_to_numpy(v[:, :, :T0]))
    for t in range(T0, T0 + steps):
        bd.append_step(ks, vs, k[:, :, t:t + 1].to(DEV).contiguous(), v[:, :, t:t + 1].to(DEV).contiguous())
        ko.append(syn.bf16_to_numpy(k[:, :, t:t + 1]))
        vo.append(syn.bf16_to_numpy(v[:, :, t:t + 1]))
    torch.cuda.synchronize()
    assert_archive_equal(gpu_archive(ks), ko.archive())
    assert_archive_equal(gpu_archive(vs), vo.archive())
    out = bd.decode_attention(q.to(DEV), ks, vs)
    ref = O.decode_attention(syn.bf16_to_numpy(q), ko.archive(), vo.archive())
    assert rel_err(out[:, :, 0].float().cpu().numpy(), ref) <= TOL
