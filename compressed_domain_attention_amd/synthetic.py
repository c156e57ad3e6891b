"""Seeded synthetic workloads: shapes and random inputs only.

This module is the one piece shared by the HIP path's tests/benchmark and
the CPU oracle.  It holds none of the method's arithmetic: it describes
workload shapes and draws sequence-correlated keys/values and queries.

Key/value recipe.  The pages measure on real post-RoPE caches of models
whose weights are not available here, so a stationary AR(1) process along
the sequence axis stands in for them: per independent channel (b, h, d)
    x_0 ~ N(0, 1 / (1 - rho^2)),   x_t = rho * x_{t-1} + eps_t,  eps ~ N(0, 1)
optionally plus a per-channel offset ~ N(0, offset_var) constant along the
sequence.  Values are drawn in float64, rounded to float32, then to bf16
(round to nearest even); the same bf16 bytes feed both sides.  Queries are
N(0, 1) rounded to bf16.  Seeds: 1000 * workload_index + stream, stream
K=0, V=1, q=2, offsets=3, with the batch row as a second seed word.
"""

from dataclasses import dataclass, field

import numpy as np
import torch

STREAM_K, STREAM_V, STREAM_Q, STREAM_OFF = 0, 1, 2, 3


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    B: int
    Hq: int
    Hkv: int
    D: int
    T: int
    R: int
    S: int
    kfmt: str
    vfmt: str
    rho: float
    offset_var: float = 0.0
    steps: int = 0          # decode steps appended one token at a time
    encode: bool = False    # the workload includes encoding the prefill
    raw_dtype: str = "bf16"
    notes: str = field(default="", compare=False)

    @property
    def G(self):
        return self.Hq // self.Hkv

    @property
    def n_blocks(self):
        return self.T // self.R

    @property
    def n_tail(self):
        return self.T % self.R


# The five workloads: tiny parity case, a Llama-3-8B-shaped layer, a 128K
# split-K context, a large-batch GQA-8 case with its prefill encode, and a
# steady-state stream of 64 single-token decode steps.
WORKLOADS = {
    "tiny": Workload("tiny", 1, B=1, Hq=4, Hkv=2, D=64, T=1027, R=8, S=2,
                     kfmt="f32", vfmt="f32", rho=0.95),
    "llama8b_layer": Workload("llama8b_layer", 2, B=8, Hq=32, Hkv=8, D=128, T=4096, R=8, S=2,
                              kfmt="i8", vfmt="i8", rho=0.95),
    "long128k": Workload("long128k", 3, B=1, Hq=32, Hkv=8, D=128, T=131077, R=16, S=4,
                         kfmt="i8", vfmt="i8", rho=0.98, offset_var=2.0),
    "batch64_gqa8": Workload("batch64_gqa8", 4, B=64, Hq=64, Hkv=8, D=128, T=8192, R=8, S=3,
                             kfmt="i8", vfmt="bf16", rho=0.9, encode=True),
    "stream64": Workload("stream64", 5, B=32, Hq=32, Hkv=8, D=128, T=32760, R=8, S=2,
                         kfmt="i8", vfmt="i8", rho=0.95, steps=64),
    # PNG mode (anchor + fp32 deltas, R = S = 8) at the shape of the README's
    # coefficient-domain table: B=1, Hkv=8, Hq=16, D=64, 65 536 tokens.
    "png64k": Workload("png64k", 6, B=1, Hq=16, Hkv=8, D=64, T=65536, R=8, S=8,
                       kfmt="png", vfmt="png", rho=0.95),
}


def _rng(seed, b=0):
    return np.random.Generator(np.random.PCG64([int(seed), int(b)]))


def to_bf16(x):
    """float64/float32 numpy array -> torch bfloat16 CPU tensor (RNE)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def ar1_sequence(B, H, T, D, rho, seed, offset_var=0.0, offset_seed=None, dtype=torch.bfloat16):
    """(B, H, T, D) CPU tensor of AR(1) sequences along T (bf16, or float32
    rounded from float64 when dtype is torch.float32).

    Generated one batch row at a time to bound host memory.
    """
    from scipy.signal import lfilter

    out = torch.empty((B, H, T, D), dtype=dtype)
    sd = 1.0 / np.sqrt(1.0 - rho * rho) if rho < 1 else 1.0
    for b in range(B):
        g = _rng(seed, b)
        x0 = g.standard_normal((H, 1, D)) * sd
        if T > 1:
            eps = g.standard_normal((H, T - 1, D))
            # the filter runs along the last axis (contiguous): same values, faster
            rest = lfilter([1.0], [1.0, -rho], np.ascontiguousarray(eps.transpose(0, 2, 1)), axis=-1,
                           zi=rho * x0.transpose(0, 2, 1))[0].transpose(0, 2, 1)
            x = np.concatenate([x0, rest], axis=1)
        else:
            x = x0[:, :T]
        if offset_var:
            go = _rng(offset_seed if offset_seed is not None else seed + 1, b)
            x = x + go.standard_normal((H, 1, D)) * np.sqrt(offset_var)
        out[b] = to_bf16(x) if dtype == torch.bfloat16 else torch.from_numpy(x.astype(np.float32))
    return out


def gaussian(shape, seed, scale=1.0):
    """N(0, scale^2) bf16 CPU tensor."""
    return to_bf16(_rng(seed).standard_normal(shape) * scale)


def workload_kv(w, T=None):
    """(K, V) bf16 CPU tensors (B, Hkv, T, D) for workload `w`.

    T defaults to the workload's prefill length plus its decode steps, so a
    streaming workload gets its future tokens from the same sequences.
    """
    T = (w.T + w.steps) if T is None else T
    k = ar1_sequence(w.B, w.Hkv, T, w.D, w.rho, 1000 * w.index + STREAM_K,
                     w.offset_var, 1000 * w.index + STREAM_OFF)
    v = ar1_sequence(w.B, w.Hkv, T, w.D, w.rho, 1000 * w.index + STREAM_V,
                     w.offset_var, 1000 * w.index + STREAM_OFF + 10)
    return k, v


def ar1_sequence_device(B, H, T, D, rho, seed, offset_var=0.0, offset_seed=None, device="cuda"):
    """(B, H, T, D) bf16 device tensor of the same AR(1) process, drawn on the
    device (torch Philox generator seeded with `seed`; offsets from
    `offset_seed`) for the full-size workloads, where host generation is slow.

    The recurrence is evaluated exactly in float64 in chunks of L steps: inside
    a chunk y = P e with P[i][j] = rho^(i-j) (i >= j), then the carried state
    adds rho^(i+1) * x_end(previous chunk).
    """
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed))
    sd = 1.0 / np.sqrt(1.0 - rho * rho) if rho < 1 else 1.0
    x0 = torch.randn((B, H, 1, D), generator=g, device=dev, dtype=torch.float64) * sd
    L = 256
    n_rest = T - 1
    C = (n_rest + L - 1) // L
    out = torch.empty((B, H, T, D), dtype=torch.bfloat16, device=dev)
    out[:, :, 0:1] = x0.to(torch.float32).to(torch.bfloat16)
    if n_rest > 0:
        i = torch.arange(L, device=dev, dtype=torch.float64)
        P = torch.tril(torch.pow(torch.tensor(rho, dtype=torch.float64, device=dev), i[:, None] - i[None, :]))
        carry_pow = torch.pow(torch.tensor(rho, dtype=torch.float64, device=dev), i + 1)   # rho^(i+1)
        state = x0[:, :, 0, :]                                     # (B, H, D)
        if offset_var:
            go = torch.Generator(device=dev)
            go.manual_seed(int(offset_seed if offset_seed is not None else seed + 1))
            off = torch.randn((B, H, 1, D), generator=go, device=dev, dtype=torch.float64) * np.sqrt(offset_var)
            out[:, :, 0:1] = (x0 + off).to(torch.float32).to(torch.bfloat16)
        else:
            off = None
        for c in range(C):
            n = min(L, n_rest - c * L)
            e = torch.randn((B, H, n, D), generator=g, device=dev, dtype=torch.float64)
            y = torch.matmul(P[:n, :n], e)                         # (B, H, n, D), zero initial state
            y += carry_pow[:n, None] * state[:, :, None, :]
            state = y[:, :, n - 1, :]
            if off is not None:
                y = y + off
            out[:, :, 1 + c * L:1 + c * L + n] = y.to(torch.float32).to(torch.bfloat16)
    return out


def workload_kv_device(w, T=None, device="cuda"):
    """(K, V) bf16 device tensors (B, Hkv, T, D) for workload `w`, drawn on
    the device (see ar1_sequence_device)."""
    T = (w.T + w.steps) if T is None else T
    k = ar1_sequence_device(w.B, w.Hkv, T, w.D, w.rho, 1000 * w.index + STREAM_K,
                            w.offset_var, 1000 * w.index + STREAM_OFF, device)
    v = ar1_sequence_device(w.B, w.Hkv, T, w.D, w.rho, 1000 * w.index + STREAM_V,
                            w.offset_var, 1000 * w.index + STREAM_OFF + 10, device)
    return k, v


def workload_query(w, step=0):
    """(B, Hq, 1, D) bf16 query; `step` selects the query of a decode step."""
    return gaussian((w.B, w.Hq, 1, w.D), 1000 * w.index + STREAM_Q + 100 * step)


def small_case(B, Hq, Hkv, D, T, rho=0.95, seed=7, offset_var=0.0, dtype=torch.bfloat16):
    """Ad-hoc small K, V (bf16 or float32) and bf16 q CPU tensors for tests."""
    k = ar1_sequence(B, Hkv, T, D, rho, seed * 10 + STREAM_K, offset_var, seed * 10 + STREAM_OFF, dtype)
    v = ar1_sequence(B, Hkv, T, D, rho, seed * 10 + STREAM_V, offset_var, seed * 10 + STREAM_OFF + 5, dtype)
    q = gaussian((B, Hq, 1, D), seed * 10 + STREAM_Q)
    return k, v, q


def bf16_to_numpy(t):
    """bf16 / float32 torch tensor -> float64 numpy array holding the same values."""
    return t.detach().to("cpu").to(torch.float32).numpy().astype(np.float64)
