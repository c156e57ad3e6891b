"""Pins for the fp64 oracle, against facts the pages and mathematics fix.

None of these re-type the oracle's own formula: each compares it with a
closed form, a library routine, a hand-worked value, an invariant, or a
figure printed on the pages (tests/golden/).
"""

import math
import os

import numpy as np
import pytest
import scipy.fft
import torch

import oracle as O
from compressed_domain_attention_amd import synthetic as syn


# ---------------------------------------------------------------- basis ----
@pytest.mark.parametrize("R", [1, 2, 3, 4, 5, 8, 12, 16, 32])
def test_basis_rows_orthonormal(R):
    # README "Math": the analysis rows are orthonormal.
    M = O.dct_basis_f64(R, R)
    assert np.abs(M @ M.T - np.eye(R)).max() <= 1e-14
    M32 = O.dct_basis_f32(R, R).astype(np.float64)
    assert np.abs(M32 @ M32.T - np.eye(R)).max() <= 4 * R * 2.0 ** -24


def test_basis_closed_forms():
    # R = 1: the transform is the identity.
    assert O.dct_basis_f64(1, 1).tolist() == [[1.0]]
    # R = 2: the normalised Haar pair (sum and difference over sqrt 2).
    h = 0.7071067811865476          # 1/sqrt(2), correctly rounded
    M2 = O.dct_basis_f64(2, 2)
    np.testing.assert_allclose(M2, [[h, h], [h, -h]], rtol=0, atol=2e-16)
    # R = 4, frequency 1: sqrt(1/2) cos(k pi/8) for k = 1, 3, 5, 7;
    # cos(pi/8) = sqrt(2 + sqrt 2) / 2 = 0.92387953251128674,
    # cos(3 pi/8) = sqrt(2 - sqrt 2) / 2 = 0.38268343236508978.
    c1, c3 = 0.92387953251128674 * h, 0.38268343236508978 * h
    np.testing.assert_allclose(O.dct_basis_f64(4, 2)[1], [c1, c3, -c3, -c1], rtol=0, atol=4e-16)
    # the constant row has all entries 1/sqrt(R)
    for R in (3, 8, 16):
        np.testing.assert_allclose(O.dct_basis_f64(R, 1)[0], np.full(R, 1 / math.sqrt(R)), rtol=0, atol=2.3e-16)


def _f32_rne_bits(x):
    """fp32 bit pattern of a positive exact value (decimal.Decimal), rounded
    to nearest with ties to even, by integer arithmetic on the scaled value."""
    from decimal import Decimal
    e = 0
    while x >= 2:
        x, e = x / 2, e + 1
    while x < 1:
        x, e = x * 2, e - 1
    scaled = x * (Decimal(2) ** 23)
    fl = int(scaled)
    frac = scaled - fl
    mant = fl + (1 if frac > Decimal("0.5") or (frac == Decimal("0.5") and fl % 2) else 0)
    if mant == 1 << 24:
        mant, e = mant >> 1, e + 1
    return ((e + 127) << 23) | (mant - (1 << 23))


def test_basis_f32_rounding_by_hand():
    # Reading 2: the codec's basis is the fp64 basis rounded to nearest fp32.
    # At R = 4, frequency 1, the exact entries are sqrt(1/2) cos(pi/8) =
    # sqrt((2 + sqrt 2) / 8) = 0.6532814824381882639... and sqrt(1/2)
    # cos(3 pi/8) = sqrt((2 - sqrt 2) / 8) = 0.2705980500730984921...; their
    # nearest fp32 values are 0x3f273d75 and 0x3e8a8bd4, while truncation
    # gives 0x3f273d74 and 0x3e8a8bd3, so a chopped or otherwise misrounded
    # basis fails here (R = 2's 1/sqrt 2 rounds the same both ways).
    from decimal import Decimal, getcontext
    getcontext().prec = 60
    r2 = Decimal(2).sqrt()
    exact = [((2 + r2) / 8).sqrt(), ((2 - r2) / 8).sqrt()]
    assert [_f32_rne_bits(x) for x in exact] == [0x3F273D75, 0x3E8A8BD4]
    got = O.dct_basis_f32(4, 2)[1].view(np.uint32).tolist()
    assert got == [0x3F273D75, 0x3E8A8BD4, 0xBE8A8BD4, 0xBF273D75]
    # every entry of the R = 8 and R = 16 bases against the exact value from
    # fifty-digit arithmetic, rounded by hand (cos from its Taylor series)
    def cos_dec(xn, xd):
        # cos(pi * xn / xd) in Decimal: pi from Machin's formula
        def arctan_inv(k):
            t, s, n, sign = Decimal(1) / k, Decimal(0), 1, 1
            pw = Decimal(1) / k
            while True:
                term = pw / n
                if term < Decimal(10) ** -58:
                    return s + sign * term
                s += sign * term
                pw /= k * k
                n += 2
                sign = -sign
        pi = 16 * arctan_inv(5) - 4 * arctan_inv(239)
        x = pi * xn / xd
        tot, term, k = Decimal(1), Decimal(1), 0
        while abs(term) > Decimal(10) ** -58:
            term = -term * x * x / ((2 * k + 1) * (2 * k + 2))
            tot += term
            k += 1
        return tot
    for R in (8, 16):
        M = O.dct_basis_f32(R, R)
        for j in range(R):
            cj = (Decimal(1) / R).sqrt() if j == 0 else (Decimal(2) / R).sqrt()
            for i in range(R):
                v = cj * cos_dec((2 * i + 1) * j, 2 * R)
                bits = _f32_rne_bits(abs(v)) if v != 0 else 0
                want = bits | (0x80000000 if v < 0 else 0)
                assert int(M[j, i].view(np.uint32)) == want, (R, j, i)


@pytest.mark.parametrize("R,S", [(2, 1), (3, 2), (8, 2), (8, 8), (12, 5), (16, 4)])
def test_projection_equals_scipy_dct(R, S):
    # The lowest S outputs of the orthonormal DCT-II of each block.
    rng = np.random.default_rng(R * 100 + S)
    x = rng.standard_normal((3, 5 * R, 7))
    ref = scipy.fft.dct(x.reshape(3, 5, R, 7), type=2, norm="ortho", axis=2)[:, :, :S, :]
    M = O.dct_basis_f64(R, S)
    got = np.einsum("ji,bnid->bnjd", M, x.reshape(3, 5, R, 7))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-13)
    # and the codec's fp32-basis projection is within the basis rounding
    C = O.project_blocks(x, R, S)
    bound = R * 2.0 ** -24 * np.abs(x).max() * 1.01
    assert np.abs(C - ref).max() <= bound


# ---------------------------------------------------------------- encode ---
def test_projection_by_hand_r2():
    # R = 2, D = 1, block [1, 3]: c0 = 4 * fp32(1/sqrt 2), c1 = -2 * fp32(1/sqrt 2);
    # fp32(1/sqrt 2) = 0.707106769084930419921875, so the fp32 rows are
    # 2.8284270763397216796875 and -1.4142135381698608398437500.
    arc = O.encode(np.array([[1.0], [3.0]]), 2, 2, O.F32)
    assert arc["rows"].shape == (1, 2, 1)
    assert arc["rows"][0, 0, 0] == np.float32(2.8284270763397216796875)
    assert arc["rows"][0, 1, 0] == np.float32(-1.41421353816986083984375)
    # one kept frequency: just the block mean times sqrt 2
    arc1 = O.encode(np.array([[1.0], [3.0], [5.0]]), 2, 1, O.F32)
    assert arc1["n_blocks"] == 1 and arc1["tail"].tolist() == [[5.0]]


def test_all_frequencies_is_lossless():
    # README "Math": keeping all R rows is lossless per block (up to the fp32
    # rounding of the basis entries).
    rng = np.random.default_rng(1)
    for R in (2, 8, 16):
        x = rng.standard_normal((2, 3, 4 * R, 16))
        xh = O.reconstruct(O.project_blocks(x, R, R), R)
        assert np.abs(xh - x).max() <= 4 * R * 2.0 ** -24 * np.abs(x).max()


def test_parseval_when_all_kept():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((6 * 8, 32))
    C = O.project_blocks(x, 8, 8)
    e_x = (x.reshape(6, 8, 32) ** 2).sum(axis=(1, 2))
    e_c = (C ** 2).sum(axis=(1, 2))
    np.testing.assert_allclose(e_c, e_x, rtol=1e-6)


def test_quality_monotone_in_kept_frequencies():
    # The reconstruction error can only shrink as more frequencies are kept.
    k, _, _ = syn.small_case(1, 1, 1, 32, 8 * 64, rho=0.95, seed=3)
    x = syn.bf16_to_numpy(k)[0, 0]
    errs = []
    for S in range(1, 9):
        xh = O.reconstruct(O.project_blocks(x, 8, S), 8)
        errs.append(np.linalg.norm(xh - x))
    assert all(errs[i + 1] <= errs[i] + 1e-9 for i in range(7))
    assert errs[-1] <= 1e-5 * np.linalg.norm(x)


def test_k2_cosine_on_correlated_signal():
    # README test list: k = 2 keeps cosine similarity above 0.99 on a
    # smooth autocorrelated signal (parity unpinned beyond this bound).
    k, _, _ = syn.small_case(2, 2, 2, 64, 2048, rho=0.99, seed=4)
    x = syn.bf16_to_numpy(k)
    xh = O.reconstruct(O.project_blocks(x, 8, 2), 8)
    cos = (xh * x).sum() / np.linalg.norm(xh) / np.linalg.norm(x)
    assert cos > 0.99


def test_quantiser_by_hand():
    # scale = fp32(1.27 / 127) = fp32(0.01) = 0.00999999977648258209228515625
    # 0.5 / s = 50.0000011..., -1.27 / s = -127.0000028..., 1.27 / s likewise.
    codes, s = O.quantize_rows(np.array([[0.5, -1.27, 0.0, 1.27]]))
    assert s.tolist() == [np.float32(0.00999999977648258209228515625)]
    assert codes.tolist() == [[50, -127, 0, 127]]
    # ties go to even: scale exactly 1.0 (absmax 127)
    codes, s = O.quantize_rows(np.array([[127.0, 2.5, -3.5, 0.5, -0.5, 1.5, -126.5]]))
    assert s.tolist() == [1.0]
    assert codes.tolist() == [[127, 2, -4, 0, 0, 2, -126]]
    # an all-zero row: scale 0, codes 0
    codes, s = O.quantize_rows(np.zeros((1, 5)))
    assert s.tolist() == [0.0] and codes.tolist() == [[0] * 5]


def test_quantiser_invariants():
    rng = np.random.default_rng(5)
    C = rng.standard_normal((40, 3, 64)) * rng.uniform(1e-3, 1e3, size=(40, 3, 1))
    C[0, 1] = 0.0
    codes, s = O.quantize_rows(C)
    assert codes.dtype == np.int8 and s.dtype == np.float32
    assert np.abs(codes.astype(int)).max() <= 127
    nz = s > 0
    assert (np.abs(codes.astype(int)).max(axis=-1)[nz] == 127).all()
    err = np.abs(C - codes.astype(np.float64) * s.astype(np.float64)[..., None])
    assert (err <= s.astype(np.float64)[..., None] / 2 * (1 + 2.0 ** -40)).all()


def test_dequantize_int8_within_half_a_step():
    # Reading 6 through O.dequantize: each code times ITS OWN row's scale is
    # within half a quantisation step of the coefficient.  Rows of one block
    # and of neighbouring blocks differ in magnitude by up to 10^6, so a scale
    # taken from the wrong row, block or axis misses by orders of magnitude.
    rng = np.random.default_rng(8)
    mag = 10.0 ** rng.uniform(-3, 3, size=(2, 3, 9, 5, 1))
    C = rng.standard_normal((2, 3, 9, 5, 48)) * mag
    codes, s = O.quantize_rows(C)
    got = O.dequantize(codes, s, O.I8)
    assert got.shape == C.shape
    half = s.astype(np.float64)[..., None] / 2
    assert (np.abs(got - C) <= half * (1 + 2.0 ** -40)).all()
    # and the steps really are per row: every row's error is at most its
    # own half step although the steps differ by up to 10^6 between rows
    assert s.max() / s.min() > 1e3


def _int8_token_error_bound(X, R):
    """Bound on |x_hat - x| per token for an int8 archive keeping all S = R
    frequencies, from scipy's orthonormal DCT (independent of the oracle):
    x_hat - x = M32^T e + (M32^T M32 - I) x with |e_j| <= s_j / 2, s_j the
    row scale max_d |c_j| / 127 (fp32 rounding: the factor 1 + 2^-20);
    the second term is below 8 R 2^-24 max |x| of the block.  Tail tokens
    are exact.  Returns (..., T) bounds."""
    T, D = X.shape[-2], X.shape[-1]
    n = T // R
    blocks = X[..., :n * R, :].reshape(*X.shape[:-2], n, R, D)
    C = scipy.fft.dct(blocks, type=2, norm="ortho", axis=-2)
    s = np.abs(C).max(axis=-1) / 127 * (1 + 2.0 ** -20)
    Mabs = np.abs(scipy.fft.dct(np.eye(R), type=2, norm="ortho", axis=0))   # |M[j, i]|
    b = np.einsum("ji,...nj->...ni", Mabs, s / 2) + 8 * R * 2.0 ** -24 * np.abs(blocks).max(axis=(-1, -2))[..., None]
    return np.concatenate([b.reshape(*X.shape[:-2], n * R), np.zeros((*X.shape[:-2], T - n * R))], axis=-1)


@pytest.mark.parametrize("R", [4, 8, 16])
def test_int8_all_frequencies_reconstruction_bound(R):
    # README "Math" (K = r is lossless) with int8 rows: the reconstruction
    # differs from the tokens only by the quantisation, within the bound above.
    k, _, _ = syn.small_case(2, 2, 2, 24, 12 * R + 3, seed=R + 60)
    K = syn.bf16_to_numpy(k)
    got = O.materialise(O.encode(K, R, R, O.I8))
    bound = _int8_token_error_bound(K, R)
    assert (np.abs(got - K) <= bound[..., None]).all()
    assert np.abs(got - K).max() > 0       # the bound is not vacuous: quantisation is visible


@pytest.mark.parametrize("R,D", [(8, 16), (4, 16), (16, 16)])
def test_int8_all_frequencies_attention_bound(R, D):
    # An int8 archive with all frequencies against textbook attention on the
    # raw tokens (torch SDPA, fp64).  Per token, |dk|, |dv| are bounded as in
    # the previous pin; then |dz_t| <= scale sum_d |q_d| |dk_t| <= delta, the
    # softmax weights move by a factor within exp(+-2 delta), so
    #   |out' - out|_inf <= max_t |dv_t| + (exp(2 delta) - 1) * max_d (max_t v - min_t v) / 2
    # (the weights of both sums total 1, so v may be centred).  The softmax
    # scale 0.02 keeps delta small enough for the bound to be tight.
    scale = 0.02
    k, v, q = syn.small_case(1, 2, 1, D, 12 * R + 3, seed=77)
    K, V, qn = (syn.bf16_to_numpy(t) for t in (k, v, q))
    got = O.decode_attention(qn, O.encode(K, R, R, O.I8), O.encode(V, R, R, O.I8), scale)
    ref = _sdpa_ref(qn[:, :, 0], K, V, scale)
    bK, bV = _int8_token_error_bound(K, R), _int8_token_error_bound(V, R)
    for hq in range(2):
        delta = (scale * np.abs(qn[0, hq, 0]).sum() * bK[0, 0]).max()
        centre = ((V[0, 0].max(axis=0) - V[0, 0].min(axis=0)) / 2).max()
        bound = bV[0, 0].max() + (math.exp(2 * delta) - 1) * centre
        err = np.abs(got[0, hq] - ref[0, hq]).max()
        assert err <= bound, (hq, err, bound)
        assert bound < 0.1 * np.abs(V).max()


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(6)
    v = (rng.standard_normal(10000) * 10.0 ** rng.uniform(-30, 30, 10000)).astype(np.float32)
    # exact ties and near-ties on both sides
    v[:4] = np.array([1.00390625, 1.01171875, -1.00390625, 1.0039063], dtype=np.float32)
    ours = O.f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (ours == ref).all()


@pytest.mark.parametrize("fmt", [O.F32, O.BF16, O.I8])
def test_causal_invariant_stream_equals_batch(fmt):
    # README "Causal-safety design" and cache.py ``append``: only complete
    # blocks are archived, never rewritten; token-by-token appends give the
    # same bytes as encoding the whole prefix at once.
    R, S = 8, 3
    k, _, _ = syn.small_case(2, 2, 2, 16, 5 * R + 3, seed=8)
    x = syn.bf16_to_numpy(k)
    st = O.Stream(R, S, fmt)
    seen = []
    for t in range(x.shape[-2]):
        st.append(x[..., t:t + 1, :])
        a = st.archive()
        for i, old in enumerate(seen):
            assert np.array_equal(a["rows"][..., i, :, :], old)
        if a["n_blocks"] > len(seen):
            seen.append(a["rows"][..., len(seen), :, :].copy())
    full = O.encode(x, R, S, fmt)
    a = st.archive()
    assert np.array_equal(a["rows"], full["rows"])
    if fmt == O.I8:
        assert np.array_equal(a["scales"], full["scales"])
    assert np.array_equal(a["tail"], full["tail"]) and a["tail"].shape[-2] == 3


# ------------------------------------------------------------- attention ---
def _sdpa_ref(q, K, V, scale):
    """torch fp64 CPU scaled_dot_product_attention with kv heads repeated."""
    G = q.shape[1] // K.shape[1]
    Kt = torch.from_numpy(np.repeat(K, G, axis=1))
    Vt = torch.from_numpy(np.repeat(V, G, axis=1))
    qt = torch.from_numpy(q[:, :, None, :])
    out = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=scale)
    return out[:, :, 0, :].numpy()


def test_attention_matches_torch_sdpa():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((2, 6, 24))
    K = rng.standard_normal((2, 3, 77, 24)) * 3
    V = rng.standard_normal((2, 3, 77, 24))
    np.testing.assert_allclose(O.attention(q, K, V, 0.3), _sdpa_ref(q, K, V, 0.3), rtol=0, atol=1e-12)


def test_attention_by_hand():
    # T = 3 tokens, D = 2, scale 1: logits 0, 1, 2.
    q = np.array([[[1.0, 0.0]]])
    K = np.array([[[[0.0, 0.0], [1.0, 0.0], [2.0, 0.0]]]])
    V = np.array([[[[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]]]])
    e = math.e
    den = 1 + e + e * e
    want = [(1 + e * e) / den, (e + e * e) / den]
    np.testing.assert_allclose(O.attention(q, K, V, 1.0)[0, 0], want, rtol=0, atol=1e-15)


def test_coefficient_domain_identity():
    # README "Materialization-free decode attention": with K_block = A S,
    # q . K[p] = (q . S^T) A[p] and out = (p A) S.  Computed here directly in
    # the coefficient domain and compared with the oracle's materialised path.
    R, S, D, G = 8, 3, 16, 2
    k, v, q = syn.small_case(1, 2 * G, 2, D, 9 * R + 5, seed=10)
    ka = O.encode(syn.bf16_to_numpy(k), R, S, O.I8)
    va = O.encode(syn.bf16_to_numpy(v), R, S, O.BF16)
    qn = syn.bf16_to_numpy(q)[:, :, 0, :]
    scale = D ** -0.5
    A = O.dct_basis_f32(R, S).astype(np.float64).T       # R x S synthesis
    Kc = ka["rows"].astype(np.float64) * ka["scales"].astype(np.float64)[..., None]
    Vc = O.bf16_bits_to_f64(va["rows"])
    out = np.empty_like(qn)
    for hq in range(2 * G):
        h = hq // G
        sj = Kc[0, h] @ qn[0, hq]                         # (n, S)
        z = np.concatenate([(sj @ A.T).reshape(-1), ka["tail"][0, h] @ qn[0, hq]]) * scale
        p = np.exp(z - z.max())
        nb = Kc.shape[2]
        w = p[: nb * R].reshape(nb, R) @ A                # (n, S)
        acc = np.einsum("ns,nsd->d", w, Vc[0, h]) + p[nb * R:] @ va["tail"][0, h]
        out[0, hq] = acc / p.sum()
    got = O.decode_attention(qn, ka, va, scale)
    np.testing.assert_allclose(got, out, rtol=0, atol=1e-12)


@pytest.mark.parametrize("kfmt,vfmt,T", [(O.I8, O.I8, 8 * 9 + 5), (O.I8, O.BF16, 8 * 12), (O.F32, O.I8, 8 * 3 + 7),
                                         (O.PNG, O.PNG, 8 * 5 + 2)])
def test_split_combine_equals_materialised(kfmt, vfmt, T):
    # README "Materialization-free decode attention": attending in the
    # coefficient domain (never building K or V) equals attending to the
    # reconstruction; triton_attention.py's split over block ranges and its
    # (max, sum, acc) combine leave the result unchanged for any split count,
    # including splits that hold no block (ns > n) and the raw tail.
    R = 8
    S = R if kfmt == O.PNG else 3
    k, v, q = syn.small_case(2, 6, 2, 16, T, seed=T)
    K, V, qn = (syn.bf16_to_numpy(t) for t in (k, v, q))
    ka, va = O.encode(K, R, S, kfmt), O.encode(V, R, S, vfmt)
    ref = O.decode_attention(qn, ka, va, 0.3)
    n = T // R
    for ns in (1, 2, 3, n, n + 4):
        np.testing.assert_allclose(O.decode_attention_split(qn, ka, va, 0.3, ns), ref, rtol=0, atol=1e-12)


def test_split_combine_tail_only_and_by_hand():
    # no complete block: the last (only non-empty) split holds the tail
    k, v, q = syn.small_case(1, 2, 1, 16, 5, seed=3)
    K, V, qn = (syn.bf16_to_numpy(t) for t in (k, v, q))
    ka, va = O.encode(K, 8, 2, O.I8), O.encode(V, 8, 2, O.I8)
    for ns in (1, 4):
        np.testing.assert_allclose(O.decode_attention_split(qn, ka, va, None, ns), _sdpa_ref(qn[:, :, 0], K, V, 0.25),
                                   rtol=0, atol=1e-12)
    # R = S = 1 identity codec, three tokens, two splits of one block and a
    # tail: logits 0, 1, 2 (q = 1, keys 0, 1, 2), values 1, 0, 0 -> 1 / (1 + e + e^2)
    e = math.e
    arch = lambda x: dict(fmt=O.F32, R=1, S=1, rows=np.array(x[:2], dtype=np.float32).reshape(1, 1, 2, 1, 1),
                          scales=None, tail=np.array(x[2:], dtype=np.float64).reshape(1, 1, 1, 1), n_blocks=2)
    got = O.decode_attention_split(np.ones((1, 1, 1)), arch([0.0, 1.0, 2.0]), arch([1.0, 0.0, 0.0]), 1.0, 2)
    assert abs(got[0, 0, 0] - 1 / (1 + e + e * e)) <= 1e-15


def test_identity_codec_equals_plain_attention():
    # R = 1, S = 1, fp32 rows: the basis is [1] and bf16 values are exact in
    # fp32, so the archive holds the keys/values themselves.
    k, v, q = syn.small_case(2, 4, 2, 32, 50, seed=11)
    K, V, qn = (syn.bf16_to_numpy(t) for t in (k, v, q))
    got = O.decode_attention(qn, O.encode(K, 1, 1, O.F32), O.encode(V, 1, 1, O.F32), 0.2)
    np.testing.assert_allclose(got, _sdpa_ref(qn[:, :, 0], K, V, 0.2), rtol=0, atol=1e-12)


def test_tail_only_is_plain_attention():
    k, v, q = syn.small_case(1, 2, 1, 16, 5, seed=12)
    K, V, qn = (syn.bf16_to_numpy(t) for t in (k, v, q))
    ka, va = O.encode(K, 8, 2, O.I8), O.encode(V, 8, 2, O.I8)
    assert ka["n_blocks"] == 0
    np.testing.assert_allclose(O.decode_attention(qn, ka, va), _sdpa_ref(qn[:, :, 0], K, V, 16 ** -0.5),
                               rtol=0, atol=1e-12)


def test_all_frequencies_attention_close_to_raw():
    k, v, q = syn.small_case(1, 4, 2, 32, 8 * 20 + 3, seed=13)
    K, V, qn = (syn.bf16_to_numpy(t) for t in (k, v, q))
    got = O.decode_attention(qn, O.encode(K, 8, 8, O.F32), O.encode(V, 8, 8, O.F32))
    ref = _sdpa_ref(qn[:, :, 0], K, V, 32 ** -0.5)
    assert np.abs(got - ref).max() <= 1e-5 * np.abs(ref).max()


def test_gqa_equals_repeated_heads():
    R, S = 8, 2
    k, v, q = syn.small_case(1, 6, 2, 16, 8 * 7, seed=14)
    K, V, qn = (syn.bf16_to_numpy(t) for t in (k, v, q))
    got = O.decode_attention(qn, O.encode(K, R, S, O.I8), O.encode(V, R, S, O.I8))
    Kr, Vr = np.repeat(K, 3, axis=1), np.repeat(V, 3, axis=1)
    ref = O.decode_attention(qn, O.encode(Kr, R, S, O.I8), O.encode(Vr, R, S, O.I8))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-13)


def test_sampled_heads_match_full():
    R, S = 8, 3
    k, v, q = syn.small_case(2, 8, 2, 16, 8 * 5 + 2, seed=15)
    K, V, qn = (syn.bf16_to_numpy(t) for t in (k, v, q))
    ka, va = O.encode(K, R, S, O.I8), O.encode(V, R, S, O.BF16)
    full = O.decode_attention(qn, ka, va, 0.25)
    part = O.decode_attention_heads(qn, ka, va, 0.25, [(0, 0), (1, 7), (1, 3)])
    for (b, hq), o in part.items():
        np.testing.assert_allclose(o, full[b, hq], rtol=0, atol=1e-14)


# --------------------------------------------------------------- storage ---
def _read_table(path):
    rows = []
    for line in open(path):
        line = line.split("#")[0].strip()
        if line:
            rows.append(line.split())
    return rows


def test_storage_matches_printed_tables(golden_dir):
    for row in _read_table(os.path.join(golden_dir, "storage_tables.txt")):
        kind, fmt = row[0], row[1]
        S, D = int(row[2]), int(row[3])
        R = 8
        if kind == "ratio":
            raw_b, pct, dec = int(row[4]), float(row[5]), int(row[6])
            n = 1000
            comp = O.storage_bytes(n, S, D, fmt, 0, raw_b)
            raw = n * R * D * raw_b
            assert abs(100.0 * comp / raw - pct) <= 0.5 * 10.0 ** -dec + 1e-9, row
        else:
            BH, seq, mb, ratio = int(row[4]), int(row[5]), float(row[6]), float(row[7])
            n, t = seq // R, seq % R
            comp = 2 * BH * O.storage_bytes(n, S, D, fmt, t, 4)
            raw = 2 * BH * seq * D * 4
            assert abs(comp / 2 ** 20 - mb) <= 0.05 + 1e-9, row
            assert abs(comp / raw - ratio) <= 0.005 + 1e-9, row


# ------------------------------------------------ view / crop / batch gather ----
def _bf16_values(x):
    return O.bf16_bits_to_f64(O.f32_to_bf16_bits(np.asarray(x, dtype=np.float32)))


def _f32_archive(x, R, S):
    return O.encode(np.asarray(x, dtype=np.float32).astype(np.float64), R, S, O.F32)


@pytest.mark.parametrize("R", [1, 2, 4, 8, 16])
def test_view_all_frequencies_returns_tokens(R):
    # S = R with fp32 rows: the orthonormal inverse gives the tokens back up
    # to the fp32 rounding of rows and basis (a transposed basis or a wrong
    # sum would miss by O(1)).
    rng = np.random.default_rng(R)
    x = rng.standard_normal((2, 3, 5 * R + 3, 8)).astype(np.float32)
    a = _f32_archive(x, R, R)
    v = O.view(a, O.F32)
    assert v.shape == x.shape and v.dtype == np.float32
    err = np.abs(v.astype(np.float64) - x).max()
    assert err <= 4 * R * 2.0 ** -24 * np.abs(x).max() + 1e-7
    # the raw tail comes back verbatim
    nR = (x.shape[-2] // R) * R
    assert np.array_equal(v[..., nR:, :], x[..., nR:, :])


@pytest.mark.parametrize("R,S", [(8, 2), (16, 4), (12, 5)])
def test_view_equals_scipy_idct_of_kept_rows(R, S):
    # Block synthesis = inverse orthonormal DCT-II (scipy's type-2 'ortho'
    # inverse) of the kept rows padded with zeros.
    rng = np.random.default_rng(R + S)
    x = rng.standard_normal((1, 1, 4 * R, 6))
    a = _f32_archive(x, R, S)
    rows = a["rows"].astype(np.float64)                      # (1,1,4,S,6)
    pad = np.zeros((1, 1, 4, R, 6))
    pad[..., :S, :] = rows
    ref = scipy.fft.idct(pad, type=2, norm="ortho", axis=3).reshape(1, 1, 4 * R, 6)
    v = O.view(a, O.F32).astype(np.float64)
    assert np.abs(v - ref).max() <= 8 * R * 2.0 ** -24 * (np.abs(rows).max() + 1)


def test_view_identity_codec_is_exact():
    # R = S = 1: M = [1], the view is the stored rows bit for bit.
    x = np.random.default_rng(3).standard_normal((2, 2, 9, 8)).astype(np.float32)
    a = _f32_archive(x, 1, 1)
    assert np.array_equal(O.view(a, O.F32), x)


@pytest.mark.parametrize("fmt", [O.F32, O.BF16, O.I8])
def test_view_prefix_is_append_only(fmt):
    # Causal-safety design: the decoded prefix never changes as tokens are
    # appended, and decoding only the blocks since block k gives the same
    # values as the full decode from token k*R on (the memoised read).
    R, S = 8, 3
    x = _bf16_values(np.random.default_rng(5).standard_normal((2, 2, 70, 16)))
    st = O.Stream(R, S, fmt)
    st.append(x[..., :37, :])
    v1 = O.view(st.archive(), O.BF16)
    st.append(x[..., 37:, :])
    a2 = st.archive()
    v2 = O.view(a2, O.BF16)
    assert np.array_equal(v2[..., :32, :], v1[..., :32, :])
    assert np.array_equal(O.view(a2, O.BF16, block_begin=3), v2[..., 24:, :])


def test_crop_cases_by_hand():
    R, S = 4, 4                                   # lossless, fp32 rows
    x = np.arange(2 * 1 * 14 * 2, dtype=np.float64).reshape(2, 1, 14, 2) / 8.0
    a = _f32_archive(x, R, S)                     # 3 blocks + 2 tail tokens
    # into the raw tail: plain truncation
    c = O.crop(a, 13, O.F32)
    assert c["n_blocks"] == 3 and np.array_equal(c["tail"], x[..., 12:13, :])
    # at a block boundary: archive prefix verbatim, empty tail
    c = O.crop(a, 8, O.F32)
    assert c["n_blocks"] == 2 and c["tail"].shape[-2] == 0
    assert np.array_equal(c["rows"], a["rows"][..., :2, :, :])
    # into the archive: the boundary block's tokens come back (lossless here)
    c = O.crop(a, 6, O.F32)
    assert c["n_blocks"] == 1 and c["tail"].shape[-2] == 2
    np.testing.assert_allclose(c["tail"], x[..., 4:6, :], rtol=0, atol=1e-5)
    # nothing left
    c = O.crop(a, 0, O.F32)
    assert c["n_blocks"] == 0 and c["tail"].shape[-2] == 0
    with pytest.raises(ValueError):
        O.crop(a, 15, O.F32)


@pytest.mark.parametrize("fmt", [O.BF16, O.I8])
def test_crop_is_path_independent_and_idempotent(fmt):
    # README / cache.py: a crop never re-compresses the history, so repeated
    # crops are idempotent and crops compose: crop(crop(a, L1), L2) = crop(a, L2).
    R, S = 8, 2
    x = _bf16_values(np.random.default_rng(9).standard_normal((2, 2, 45, 16)))
    a = O.encode(x, R, S, fmt)
    for L1 in (45, 40, 37, 16, 9):
        c1 = O.crop(a, L1, O.BF16)
        c11 = O.crop(c1, L1, O.BF16)
        for k in ("rows", "tail"):
            assert np.array_equal(c11[k], c1[k])
        for L2 in range(0, L1 + 1, 3):
            d1, d2 = O.crop(c1, L2, O.BF16), O.crop(a, L2, O.BF16)
            assert d1["n_blocks"] == d2["n_blocks"]
            for k in ("rows", "scales", "tail"):
                if d1[k] is not None:
                    assert np.array_equal(d1[k], d2[k]), (L1, L2, k)
    # the re-exposed tail is the view of the same tokens, in the raw format
    c = O.crop(a, 21, O.BF16)
    assert np.array_equal(O.f32_to_bf16_bits(c["tail"]), O.view(a, O.BF16)[..., 16:21, :])


def test_select_batch_invariants():
    R, S = 8, 2
    x = _bf16_values(np.random.default_rng(11).standard_normal((4, 2, 30, 16)))
    a = O.encode(x, R, S, O.I8)
    same = O.select_batch(a, [0, 1, 2, 3])
    for k in ("rows", "scales", "tail"):
        assert np.array_equal(same[k], a[k])
    # gathering commutes with decoding: the view of a gathered archive is the
    # gathered view (and so is the archive of gathered tokens)
    idx = [3, 3, 0, 2, 1]
    g = O.select_batch(a, idx)
    assert np.array_equal(O.view(g, O.BF16), O.view(a, O.BF16)[idx])
    e = O.encode(x[idx], R, S, O.I8)
    for k in ("rows", "scales", "tail"):
        assert np.array_equal(g[k], e[k])


# ------------------------------------------------------------- PNG mode ----
def test_png_rows_by_hand():
    # README "Math", PNG item: the anchor x_0, then deltas x_i - x_{i-1}.
    x = np.array([1.0, 3.0, 2.0, 2.0, 5.0, 4.0, 4.5, -1.0, 7.0]).reshape(1, 1, 9, 1)
    a = O.encode(x, 4, 4, O.PNG)
    assert a["rows"].dtype == np.float32 and a["n_blocks"] == 2
    assert a["rows"][0, 0, :, :, 0].tolist() == [[1, 2, -1, 0], [5, -1, 0.5, -5.5]]
    assert a["tail"][0, 0, :, 0].tolist() == [7.0]
    with pytest.raises(ValueError):
        O.encode(x, 4, 2, O.PNG)
    # the synthesis undoes the analysis exactly (cumulative sum of the deltas)
    for R in (1, 2, 8, 16):
        assert np.array_equal(O.png_synthesis(R) @ O.png_analysis(R), np.eye(R))


@pytest.mark.parametrize("R", [1, 4, 8, 16])
def test_png_is_lossless_on_bf16_tokens(R):
    # The lossless tier: bf16 tokens come back bit for bit through the view
    # (deltas of bf16 values of similar magnitude are exact in fp32).
    x = syn.bf16_to_numpy(syn.ar1_sequence(2, 3, 7 * R + 3, 32, 0.95, seed=R))
    a = O.encode(x, R, R, O.PNG)
    v = O.view(a, O.BF16)
    assert np.array_equal(v, O.f32_to_bf16_bits(x.astype(np.float32)))
    # and attention over the archive is attention over the raw tokens
    q = np.random.default_rng(R).standard_normal((2, 6, 32))
    got = O.decode_attention(q, a, a)
    ref = O.attention(q, x, x, 32 ** -0.5)
    assert np.abs(got - ref).max() <= 1e-12


def test_png_delta_variance_collapse():
    # README "Math": autocorrelation collapses the variance of first-order
    # deltas; for a stationary AR(1), Var(delta) / Var(x) = 2 (1 - rho).
    rho = 0.95
    x = syn.bf16_to_numpy(syn.ar1_sequence(1, 4, 8 * 4096, 64, rho, seed=3))
    a = O.encode(x, 8, 8, O.PNG)
    deltas = a["rows"][..., 1:, :].astype(np.float64)
    ratio = deltas.var() / x.var()
    assert abs(ratio - 2 * (1 - rho)) <= 0.01
