"""Benchmark: compressed-domain decode attention on one MI355X.

Default workload: the 128K-context layer (B=1, Hq=32, Hkv=8, D=128,
T=131072+5, R=16, S=4, int8 K and V rows).  A step is one decode step of a
stack of LAYERS such layers, each with its own archive at its own address
(8 x 69 MB exceeds the 256 MB MALL, so HBM is what is measured): per layer,
append the new token's K/V and attend (codec_decode_attention_append: the
decode launch takes the token itself, and a separate append launch archives
a block every R steps).  Each step is captured once
as a HIP graph and the graphs are replayed in order.

Prints one JSON line.  value = compressed-KV GB/s: algorithmic decode bytes
of all layers and timed steps / wall time of the timed steps.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import compressed_domain_attention_amd as cda  # noqa: E402
from compressed_domain_attention_amd import synthetic as syn  # noqa: E402

HBM_PEAK_GBS = 8000.0
EB = {"f32": 4, "bf16": 2, "i8": 1, "png": 4}


def decode_bytes(w, n_blocks, n_tail):
    """Algorithmic bytes of one decode call: rows + scales of both archives,
    the raw tail, q (bf16) and out (fp32)."""
    per_bh = n_blocks * w.S * (w.D * EB[w.kfmt] + (4 if w.kfmt == "i8" else 0)) \
        + n_blocks * w.S * (w.D * EB[w.vfmt] + (4 if w.vfmt == "i8" else 0)) \
        + 2 * n_tail * w.D * EB[w.raw_dtype]
    return w.B * w.Hkv * per_bh + w.B * w.Hq * w.D * (2 + 4)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("decode_impl.h", "internal.h", "basis.h", "basis_dev.h"):
        h.update(open(os.path.join(ROOT, "compressed_domain_attention_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def arith_note(w):
    """How each contraction of the workload's row formats is computed."""
    k = ("keys: int8 x int8 MFMA (query as int8 digits), products summed exactly in int32"
         if w.kfmt == "i8" else "keys: fp32 VALU FMAs")
    v = {"i8": "values: int8 x int8 MFMA (weights as int8 digits), products summed exactly in int32",
         "bf16": "values: bf16 MFMA (weights as three bf16 terms), products exact in fp32",
         }.get(w.vfmt, "values: fp32 VALU FMAs")
    return f"{k}; {v}; fp32 softmax, scaling and accumulation"


def load_traffic(workload):
    """HBM traffic per decode launch from the committed counter summary, if it
    was taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", f"decode_{workload}_traffic.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("traffic_bytes_per_launch")


CALIB_ELEMS = 64 << 20      # fp32 elements of the calibration copy (256 MiB read + 256 MiB written)


def profile_run(w, n):
    """Launch sequence for rocprofv3 counter passes: one decode of the
    workload (eager, so every launch is its own dispatch) n times, then a
    plain elementwise copy of known size n times to calibrate the counters."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    k, v = syn.workload_kv_device(w, T=w.T, device=dev)
    q = syn.workload_query(w, 0).to(dev)
    ks = cda.CodecStream(w.B, w.Hkv, w.D, w.R, w.S, fmt=w.kfmt, device=dev)
    vs = cda.CodecStream(w.B, w.Hkv, w.D, w.R, w.S, fmt=w.vfmt, device=dev)
    ks.encode(k)
    vs.encode(v)
    del k, v
    out = torch.empty((w.B, w.Hq, 1, w.D), dtype=torch.float32, device=dev)
    ws = torch.zeros(cda.decode_workspace_bytes(ks, vs, w.Hq), dtype=torch.uint8, device=dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    a = torch.ones(CALIB_ELEMS, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(n):
        flush.fill_(1)                      # the archive is read from HBM, not the MALL
        cda.decode_attention(q, ks, vs, out=out, workspace=ws)
    for _ in range(n):
        torch.neg(a, out=b)                 # reads and writes CALIB_ELEMS * 4 bytes
    torch.cuda.synchronize()
    print(f"# profile run done: {n} decodes, {n} calibration copies", flush=True)


def traffic_summary(w, fetch_csv, write_csv, command):
    """HBM bytes per decode launch from two rocprofv3 --pmc runs (FETCH_SIZE,
    WRITE_SIZE; KiB per dispatch), each scaled by what the same counter reads
    for the calibration copy of known size.  Writes the committed summary."""
    import csv
    import statistics

    def per_kernel(path, counter):
        vals = {"decode": [], "copy": []}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            if "decode_kernel" in name:
                vals["decode"].append(float(r["Counter_Value"]))
            elif "neg_kernel" in name:
                vals["copy"].append(float(r["Counter_Value"]))
        return {key: statistics.median(x) if x else None for key, x in vals.items()}

    f = per_kernel(fetch_csv, "FETCH_SIZE")
    wr = per_kernel(write_csv, "WRITE_SIZE")
    calib = CALIB_ELEMS * 4
    f_factor = calib / (f["copy"] * 1024.0)
    w_factor = calib / (wr["copy"] * 1024.0)
    fetch_b = f["decode"] * 1024.0 * f_factor
    write_b = wr["decode"] * 1024.0 * w_factor
    d = {"workload": w.name, "kernel": "decode_kernel", "kernel_source_hash": kernel_source_hash(),
         "fetch_kib_per_launch": f["decode"], "write_kib_per_launch": wr["decode"],
         "copy_fetch_kib": f["copy"], "copy_write_kib": wr["copy"], "copy_bytes_each_way": calib,
         "fetch_factor": f_factor, "write_factor": w_factor,
         "traffic_bytes_per_launch": fetch_b + write_b,
         "algorithmic_bytes_per_launch": decode_bytes(w, w.n_blocks, w.n_tail), "command": command}
    path = os.path.join(ROOT, "profiles", f"decode_{w.name}_traffic.json")
    with open(path, "w") as fh:
        json.dump(d, fh, indent=1)
    print(json.dumps(d, indent=1))


def view_bytes(w, fmt, n_blocks, n_tail, out_bytes=2):
    """Algorithmic bytes of one full materialised view of a stream: rows (+
    scales) and tail read, every token written in the view format."""
    per_bh = n_blocks * w.S * (w.D * EB[fmt] + (4 if fmt == "i8" else 0)) + n_tail * w.D * 2 \
        + (n_blocks * w.R + n_tail) * w.D * out_bytes
    return w.B * w.Hkv * per_bh


def archive_ops(w, streams, dev, rounds=3):
    """Timings of the structural archive operations on the workload's
    streams (each layer's key stream, rotated so reads come from HBM):
    the full bf16 materialised view (codec_materialise from block 0) and a
    batch gather of every row (codec_select_batch, reversed order)."""
    L = len(streams)
    ks0 = streams[0][0]
    n, t = ks0.n_blocks, ks0.n_tail
    views = [torch.empty((w.B, w.Hkv, n * w.R + t, w.D), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    for li in range(L):
        cda.materialise(streams[li][0], views[li], block_begin=0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(rounds):
        for li in range(L):
            cda.materialise(streams[li][0], views[li], block_begin=0)
    e1.record()
    torch.cuda.synchronize()
    v_us = e0.elapsed_time(e1) * 1e3 / (rounds * L)
    vb = view_bytes(w, w.kfmt, n, t)
    del views
    # gather: every batch row, reversed, of each layer's key stream into new buffers
    idx = list(range(w.B))[::-1]
    gb = 2 * (w.B * w.Hkv * (n * w.S * (w.D * EB[w.kfmt] + (4 if w.kfmt == "i8" else 0)) + w.R * w.D * 2))
    g_ms = []
    for li in range(L):
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        streams[li][0].select_batch(idx)
        b.record()
        torch.cuda.synchronize()
        g_ms.append(a.elapsed_time(b))
    g_us = float(np.median(g_ms)) * 1e3
    return {"materialise": {"kernel": "view_kernel", "avg_us": round(v_us, 3), "bytes": vb,
                            "GBps": round(vb / (v_us * 1e-6) / 1e9, 2),
                            "hbm_peak_fraction": round(vb / (v_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                            "what": "whole bf16 view of one layer's key archive (all blocks + tail)"},
            "select_batch": {"kernel": "gather_kernel", "avg_us_incl_alloc": round(g_us, 3), "bytes": gb,
                             "GBps": round(gb / (g_us * 1e-6) / 1e9, 2),
                             "what": "all batch rows of one layer's key stream, reversed, into new buffers"}}


def read_ceiling(per_launch, L, dev, cap_stream, rounds=4):
    """The streaming-read ceiling for this size: one plain read of
    `per_launch` bytes (the decode's algorithmic bytes) per launch, rotating
    over L buffers at their own addresses like the decode's layers, captured
    in a graph and timed with events on the capture stream; the fastest of
    several grid sizes (codec_measure_read: 16-byte loads, sixteen requested
    together per thread)."""
    nbytes = -(-per_launch // 16) * 16
    bufs = [torch.ones(nbytes, dtype=torch.uint8, device=dev) for _ in range(L)]
    sink = torch.empty(65536, dtype=torch.int32, device=dev)
    best = None
    for wg in (256, 512, 1024, 2048, 4096):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap_stream):
            for _ in range(rounds):
                for b in bufs:
                    cda.measure_read(b, sink, wg)
        with torch.cuda.stream(cap_stream):
            g.replay()
            e_a, e_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e_a.record(cap_stream)
            for _ in range(5):
                g.replay()
            e_b.record(cap_stream)
        torch.cuda.synchronize()
        us = e_a.elapsed_time(e_b) * 1e3 / (5 * rounds * L)
        if best is None or us < best[0]:
            best = (us, wg)
    del bufs
    us, wg = best
    return {"kernel": "read_kernel", "avg_launch_us": round(us, 3), "bytes": nbytes, "workgroups": wg,
            "GBps": round(nbytes / (us * 1e-6) / 1e9, 2),
            "what": f"one plain read of the decode's algorithmic bytes per launch, {L} buffers rotated, graph-timed; "
                    f"fastest of 256..4096 workgroups"}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, k, v, q, budget_s=12.0, budget_1t_s=5.0):
    """The fp64 oracle on the host cores, on a bounded sample: whole-sequence
    decode attention of one kv head (with its G query heads) at a time,
    cycling over the kv heads until the time budget is spent (the archives
    are encoded once, outside the timed part).  BLAS threads are set to the
    cores this process may run on; a second, shorter sample runs on one
    thread.  Returns the JSON object."""
    import oracle as O
    from threadpoolctl import threadpool_limits
    cores = len(os.sched_getaffinity(0))
    R, S = w.R, w.S
    n = w.T // R
    per_head = n * S * (w.D * EB[w.kfmt] + (4 if w.kfmt == "i8" else 0) + w.D * EB[w.vfmt]
                        + (4 if w.vfmt == "i8" else 0)) + 2 * (w.T % R) * w.D * 2 + w.G * w.D * 6
    heads = [(b, h) for b in range(w.B) for h in range(w.Hkv)][:16]
    qn = syn.bf16_to_numpy(q)[:, :, 0]
    scale = w.D ** -0.5
    # the archives of the sample, encoded by the oracle: timed as the oracle's
    # prefill encode (bf16 tokens read, rows, scales and raw tail written)
    enc_bytes = sum(w.T * w.D * 2 + n * S * (w.D * EB[f] + (4 if f == "i8" else 0)) + (w.T % R) * w.D * 2
                    for f in (w.kfmt, w.vfmt))
    arch = []
    t_enc = 0.0
    with threadpool_limits(limits=cores):
        for (b, h) in heads:
            kx = syn.bf16_to_numpy(k[b:b + 1, h:h + 1, :w.T])
            vx = syn.bf16_to_numpy(v[b:b + 1, h:h + 1, :w.T])
            t1 = time.perf_counter()
            ka, va = O.encode(kx, R, S, w.kfmt), O.encode(vx, R, S, w.vfmt)
            t_enc += time.perf_counter() - t1
            arch.append((b, h, ka, va))

    def run(budget):
        done, t_used = 0, 0.0
        while t_used < budget:
            b, h, ka, va = arch[done % len(arch)]
            qs = qn[b:b + 1, h * w.G:(h + 1) * w.G]
            t1 = time.perf_counter()
            O.decode_attention(qs, ka, va, scale)
            t_used += time.perf_counter() - t1
            done += 1
        return done, t_used

    with threadpool_limits(limits=cores):
        done, t_used = run(budget_s)
    with threadpool_limits(limits=1):
        done1, t_used1 = run(budget_1t_s)
    return {"value": round(done * per_head / t_used / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "threads_setting": f"BLAS threads = len(os.sched_getaffinity(0)) = {cores}", "cpu_model": cpu_model(),
            "value_1_thread": round(done1 * per_head / t_used1 / 1e9, 4),
            "encode": {"value": round(len(arch) * enc_bytes / t_enc / 1e9, 4), "unit": "GB/s",
                       "sample": f"oracle encode of the K and V sequences of {len(arch)} kv heads ({w.T} tokens "
                                 f"each) on {cores} threads, {t_enc:.1f}s"},
            "sample": f"{done} whole-archive decodes ({w.T} tokens, one kv head with its {w.G} query heads each), "
                      f"cycling over {len(arch)} of the {w.B * w.Hkv} kv heads; fp64 numpy; "
                      f"{t_used:.1f}s of oracle time on {cores} threads, then {done1} decodes in {t_used1:.1f}s "
                      f"on 1 thread"}


def graph_time_us(fn, stream, rounds=4, reps=5):
    """Average time of one fn() call: fn captured `rounds` times into one HIP
    graph on `stream`, the graph replayed `reps` times, timed with events on
    that stream."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(rounds):
            fn()
    with torch.cuda.stream(stream):
        g.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / (reps * rounds)


def shape_timing(spec, dev):
    """Graph-timed decode launch for a shape outside the named workloads:
    spec = "B,Hq,Hkv,D,T,R,S,kfmt,vfmt" (AR(1) rho 0.95 keys and values drawn
    on the device, N(0,1) query), layers rotated for at least 512 MiB of
    archives (at least 2, at most 64)."""
    f = spec.split(",")
    B, Hq, H, D, T, R, S = (int(x) for x in f[:7])
    kf, vf = f[7], f[8]
    k = syn.ar1_sequence_device(B, H, T, D, 0.95, 11, device=dev)
    v = syn.ar1_sequence_device(B, H, T, D, 0.95, 12, device=dev)
    q = syn.gaussian((B, Hq, 1, D), 13).to(dev)
    ks = cda.CodecStream(B, H, D, R, S, fmt=kf, device=dev)
    vs = cda.CodecStream(B, H, D, R, S, fmt=vf, device=dev)
    ks.encode(k)
    vs.encode(v)
    layers = [(ks, vs)]
    eb = {"i8": 1, "bf16": 2, "f32": 4}
    n, t = ks.n_blocks, ks.n_tail
    per = B * H * n * S * (D * (eb[kf] + eb[vf]) + 4 * ((kf == "i8") + (vf == "i8"))) \
        + 2 * B * H * t * D * 2 + B * Hq * D * (2 + 4)
    L = min(64, max(2, -(-(512 << 20) // per)))
    for _ in range(L - 1):
        a = cda.CodecStream(B, H, D, R, S, fmt=kf, device=dev)
        b = cda.CodecStream(B, H, D, R, S, fmt=vf, device=dev)
        a.encode(k)
        b.encode(v)
        layers.append((a, b))
    del k, v
    out = torch.empty((B, Hq, 1, D), dtype=torch.float32, device=dev)
    ws = torch.zeros(cda.decode_workspace_bytes(*layers[0], Hq) + 4096, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def fn():
        for a, b in layers:
            cda.decode_attention(q, a, b, out=out, workspace=ws)
    us = graph_time_us(fn, torch.cuda.Stream()) / L
    return {"shape": {"B": B, "Hq": Hq, "Hkv": H, "D": D, "T": T, "R": R, "S": S, "k_rows": kf, "v_rows": vf},
            "layers_rotated": L, "avg_launch_us": round(us, 2), "algorithmic_bytes_per_launch": per,
            "GBps": round(per / us / 1e3, 1), "hbm_peak_fraction": round(per / us / 1e3 / HBM_PEAK_GBS, 4)}


def layer_launch_bound(w, L, dev):
    """What one launch per step across L layers could save at most: L decode
    launches (one per layer's archive, as a model runs them) against one
    launch over the same bytes (the L layers in one CodecLayerStack, which a
    model cannot use for a step: each layer's query needs the previous
    layer's output), and the fixed cost of one launch: the intercept of the
    launch time against the context length (full, half and quarter length
    keep the same split count), i.e. launch, prologue, tail, merge and
    combine, the part that a resident multi-layer kernel could hide."""
    cs = torch.cuda.Stream()
    k, v = syn.workload_kv_device(w, T=w.T, device=dev)
    q = syn.workload_query(w, 0).to(dev)

    def make(kk, vv, B, T):
        ks = cda.CodecStream(B, w.Hkv, w.D, w.R, w.S, fmt=w.kfmt, device=dev)
        vs = cda.CodecStream(B, w.Hkv, w.D, w.R, w.S, fmt=w.vfmt, device=dev)
        ks.encode(kk[:, :, :T])
        vs.encode(vv[:, :, :T])
        return ks, vs

    layers = [make(k, v, w.B, w.T) for _ in range(L)]
    stack = cda.CodecLayerStack(L, w.B, w.Hkv, w.D, w.R, w.S, k_fmt=w.kfmt, v_fmt=w.vfmt, device=dev)
    stack.encode(torch.stack([k] * L), torch.stack([v] * L))
    merged = (stack.k, stack.v)
    lengths = [w.T, w.T // 2, w.T // 4]
    shorter = {T: [make(k, v, w.B, T) for _ in range(L)] for T in lengths[1:]}
    qm = torch.stack([q] * L)
    outs = [torch.empty((w.B, w.Hq, 1, w.D), dtype=torch.float32, device=dev) for _ in range(L)]
    om = torch.empty((L, w.B, w.Hq, 1, w.D), dtype=torch.float32, device=dev)
    need = max(cda.decode_workspace_bytes(*layers[0], w.Hq), cda.decode_workspace_bytes(*merged, w.Hq))
    ws = torch.zeros(need + 4096, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def per_layer(group):
        def fn():
            for li, (ks, vs) in enumerate(group):
                cda.decode_attention(q, ks, vs, out=outs[li], workspace=ws)
        return fn

    t_layers = graph_time_us(per_layer(layers), cs)
    t_merged = graph_time_us(lambda: stack.decode(qm, out=om, workspace=ws), cs)
    per_len = [t_layers / L] + [graph_time_us(per_layer(shorter[T]), cs) / L for T in lengths[1:]]
    slope, intercept = np.polyfit(np.array(lengths, dtype=np.float64), np.array(per_len), 1)
    return {"workload": w.name, "layers": L, "per_layer_launches_us": round(t_layers, 2),
            "one_merged_launch_us": round(t_merged, 2), "saving_bound_us": round(t_layers - t_merged, 2),
            "saving_bound_frac": round(1 - t_merged / t_layers, 4),
            "launch_us_by_tokens": {str(T): round(t, 3) for T, t in zip(lengths, per_len)},
            "fixed_cost_per_launch_us": round(float(intercept), 3),
            "us_per_million_tokens": round(float(slope) * 1e6, 3),
            "bytes_per_layer": decode_bytes(w, layers[0][0].n_blocks, layers[0][0].n_tail)}


def layer_stack_timing(w, kd, vd, L, q, dev, stream, per_layer_us):
    """One step's decode of all L layers as one launch (CodecLayerStack: the
    L layers' archives in one allocation, layers folded into the batch axis),
    graph-timed, beside L per-layer launches of the same archives.  The one
    launch needs every layer's query at once."""
    st = cda.CodecLayerStack(L, w.B, w.Hkv, w.D, w.R, w.S, k_fmt=w.kfmt, v_fmt=w.vfmt, device=dev,
                             capacity=w.T // w.R + 1)
    for l in range(L):
        kl, vl = st.layer(l)
        kl.encode(kd[:, :, :w.T])
        vl.encode(vd[:, :, :w.T])
    qs = torch.stack([q] * L)
    out = torch.empty((L, w.B, w.Hq, 1, w.D), dtype=torch.float32, device=dev)
    st.decode(qs, out=out)   # sizes and caches the workspace before the capture
    torch.cuda.synchronize()
    t = graph_time_us(lambda: st.decode(qs, out=out), stream)
    per_layer_bytes = decode_bytes(w, st.layer(0)[0].n_blocks, st.layer(0)[0].n_tail)
    res = {"layers": L, "one_launch_us": round(t, 2), "per_layer_launches_us": round(per_layer_us * L, 2),
           "GBps": round(L * per_layer_bytes / (t * 1e-6) / 1e9, 2),
           "frac": round(L * per_layer_bytes / (t * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
           "what": "CodecLayerStack.decode: every layer's decode in one launch (all queries given at once)"}
    del st
    torch.cuda.empty_cache()
    return res


PHASES = ["start", "query converted", "raw tail done", "tile loop done", "waves merged", "partial published",
          "arrival counted", "output written"]


def timeline(w, L, dev, reps=6):
    """Per-wave phase times of one cold decode launch, from the measurement
    build (CDATTN_LIBRARY=compressed_domain_attention_amd/timeline/libcdattn.so):
    the other L - 1 layers are decoded first, so layer 0's archive comes from
    HBM, then one launch of layer 0 writes its stamps.  Times are microseconds
    after the first wave's start; min / median / max over the waves that
    reached each phase, then the median of those over the repetitions."""
    k, v = syn.workload_kv_device(w, T=w.T, device=dev)
    q = syn.workload_query(w, 0).to(dev)
    layers = []
    for _ in range(L):
        ks = cda.CodecStream(w.B, w.Hkv, w.D, w.R, w.S, fmt=w.kfmt, device=dev)
        vs = cda.CodecStream(w.B, w.Hkv, w.D, w.R, w.S, fmt=w.vfmt, device=dev)
        ks.encode(k[:, :, :w.T])
        vs.encode(v[:, :, :w.T])
        layers.append((ks, vs))
    del k, v
    out = torch.empty((w.B, w.Hq, 1, w.D), dtype=torch.float32, device=dev)
    ws = torch.zeros(cda.decode_workspace_bytes(*layers[0], w.Hq), dtype=torch.uint8, device=dev)
    buf = torch.zeros(4096 * 8 * 8, dtype=torch.int64, device=dev)
    per_rep = []
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    for _ in range(reps):
        cda.timeline_set(None)
        for ks, vs in layers[1:]:
            cda.decode_attention(q, ks, vs, out=out, workspace=ws)
        buf.zero_()
        torch.cuda.synchronize()
        cda.timeline_set(buf)
        cda.decode_attention(q, *layers[0], out=out, workspace=ws)
        torch.cuda.synchronize()
        cda.timeline_set(None)
        t = buf.view(4096, 8, 8).cpu().numpy()
        live = t[:, :, 0] > 0
        nwg = int(live.any(axis=1).sum())
        t = t[:nwg].astype(np.float64)
        t0 = t[:, :, 0][t[:, :, 0] > 0].min()
        rel = np.where(t > 0, (t - t0) * 0.01, np.nan)      # 100 MHz ticks -> us
        stats = {}
        for i, name in enumerate(PHASES):
            col = rel[:, :, i]
            col = col[~np.isnan(col)]
            if col.size:
                stats[name] = [float(col.min()), float(np.median(col)), float(col.max())]
        loop = rel[:, :, 3]
        by_mod8 = [float(np.nanmax(loop[g::8])) for g in range(min(8, nwg))]
        halves = [float(np.nanmean(loop[:, :4])), float(np.nanmean(loop[:, 4:]))]
        # dispatch rounds: workgroups in start order, one CU's worth each
        order = np.argsort(np.nanmin(rel[:, :, 0], axis=1))
        per_wg = {"workgroup start": np.nanmin(rel[:, :, 0], axis=1),
                  "query converted (median of its waves)": np.nanmedian(rel[:, :, 1], axis=1),
                  "last tile loop of the workgroup": np.nanmax(rel[:, :, 3], axis=1),
                  "output written (or partial published)": np.nanmax(rel[:, :, 5:8], axis=(1, 2))}
        rounds = []
        for r0 in range(0, nwg, n_cu):
            idx = order[r0:r0 + n_cu]
            rounds.append({k: [float(np.nanmin(x[idx])), float(np.nanmedian(x[idx])), float(np.nanmax(x[idx]))]
                           for k, x in per_wg.items()})
        loop_time = [float(np.nanmean(loop[:, :4] - rel[:, :4, 1])), float(np.nanmean(loop[:, 4:] - rel[:, 4:, 1]))]
        per_rep.append((stats, by_mod8, halves, nwg, rounds, loop_time))
    names = [n for n in PHASES if all(n in r[0] for r in per_rep)]
    phase = {n: [round(float(np.median([r[0][n][j] for r in per_rep])), 2) for j in range(3)] for n in names}
    return {"workload": w.name, "layers_rotated": L, "launches": reps, "workgroups": per_rep[0][3],
            "phase_us_min_median_max": phase,
            "tile_loop_end_max_by_workgroup_index_mod_8_us":
                [round(float(np.median([r[1][g] for r in per_rep])), 2) for g in range(len(per_rep[0][1]))],
            "tile_loop_end_mean_waves_0_3_vs_4_7_us":
                [round(float(np.median([r[2][j] for r in per_rep])), 2) for j in range(2)],
            "tile_loop_time_mean_waves_0_3_vs_4_7_us":
                [round(float(np.median([r[5][j] for r in per_rep])), 2) for j in range(2)],
            "rounds_of_one_workgroup_per_cu": [
                {k: [round(float(np.median([r[4][i][k][j] for r in per_rep])), 2) for j in range(3)]
                 for k in per_rep[0][4][i]} for i in range(len(per_rep[0][4]))]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="long128k", choices=sorted(syn.WORKLOADS))
    ap.add_argument("--layers", type=int, default=0,
                    help="layers rotated per step (default: enough for 512 MiB of archives, twice the MALL; 8 to 64)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", type=int, default=0, metavar="N",
                    help="launch sequence for rocprofv3 counter passes: N decodes and N calibration copies")
    ap.add_argument("--timeline", action="store_true",
                    help="per-wave phase times of one cold decode launch (needs the measurement build)")
    ap.add_argument("--layer-launch-bound", action="store_true",
                    help="time L per-layer decode launches against one launch over the same bytes, and print that")
    ap.add_argument("--shape", metavar="B,Hq,Hkv,D,T,R,S,KFMT,VFMT",
                    help="graph-time the decode launch of one shape outside the named workloads, and print that")
    ap.add_argument("--traffic", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "COMMAND"),
                    help="summarise two rocprofv3 --pmc runs into profiles/decode_<workload>_traffic.json")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    w = syn.WORKLOADS[args.workload]
    if args.layers <= 0:
        args.layers = min(64, max(8, -(-(512 << 20) // decode_bytes(w, w.n_blocks, w.n_tail))))
    if args.traffic:
        traffic_summary(w, *args.traffic)
        return
    if args.profile:
        profile_run(w, args.profile)
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.shape:
        print(json.dumps(shape_timing(args.shape, dev)), flush=True)
        return
    if args.layer_launch_bound:
        print(json.dumps(layer_launch_bound(w, args.layers, dev)), flush=True)
        return
    if args.timeline:
        print(json.dumps(timeline(w, args.layers, dev)), flush=True)
        return
    L, K, W = args.layers, args.steps, args.warmup
    extra = K + W
    print(f"# generating {w.name}: B={w.B} Hkv={w.Hkv} T={w.T}+{extra} D={w.D}", file=sys.stderr, flush=True)
    k, v = syn.workload_kv_device(w, T=w.T + extra, device=dev)
    kd, vd = k, v
    queries = [syn.workload_query(w, s).to(dev) for s in range(extra)]
    cap = (w.T + extra) // w.R + 1

    # ---- prefill: encode every layer's archive (timed; a2/a3)
    streams = []
    enc_ms = []
    for _ in range(L):
        ks = cda.CodecStream(w.B, w.Hkv, w.D, w.R, w.S, fmt=w.kfmt, device=dev, capacity=cap)
        vs = cda.CodecStream(w.B, w.Hkv, w.D, w.R, w.S, fmt=w.vfmt, device=dev, capacity=cap)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        ks.encode(kd[:, :, :w.T])
        vs.encode(vd[:, :, :w.T])
        e1.record()
        torch.cuda.synchronize()
        enc_ms.append(e0.elapsed_time(e1))
        streams.append((ks, vs))
    n0, t0 = streams[0][0].n_blocks, streams[0][0].n_tail
    enc_bytes = 2 * w.B * w.Hkv * (w.T * w.D * 2) + sum(
        w.B * w.Hkv * n0 * w.S * (w.D * EB[f] + (4 if f == "i8" else 0)) for f in (w.kfmt, w.vfmt)) \
        + 2 * w.B * w.Hkv * t0 * w.D * 2

    outs = [torch.empty((w.B, w.Hq, 1, w.D), dtype=torch.float32, device=dev) for _ in range(L)]
    ws = torch.zeros(max(cda.decode_workspace_bytes(ks, vs, w.Hq) for ks, vs in streams) * 2 + 4096,
                     dtype=torch.uint8, device=dev)

    # ---- capture one graph per step (append + decode for every layer)
    print(f"# capturing {extra} step graphs x {L} layers", file=sys.stderr, flush=True)
    graphs, step_bytes, step_qtok = [], [], []
    cap_stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    for s in range(extra):
        g = torch.cuda.CUDAGraph()
        nb = ntl = 0
        with torch.cuda.graph(g, stream=cap_stream):
            for li, (ks, vs) in enumerate(streams):
                # append the step's token and attend, in one call (one launch
                # unless the token completes a block)
                cda.decode_attention_append(queries[s], ks, vs, kd[:, :, w.T + s:w.T + s + 1],
                                            vd[:, :, w.T + s:w.T + s + 1], out=outs[li], workspace=ws)
                nb, ntl = ks.n_blocks, ks.n_tail
        graphs.append(g)
        step_bytes.append(L * decode_bytes(w, nb, ntl))
        step_qtok.append(L * w.B * w.Hq * (nb * w.R + ntl))

    for s in range(W):
        graphs[s].replay()
    torch.cuda.synchronize()
    t_a, t_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_a.record()
    for s in range(W, W + K):
        graphs[s].replay()
    t_b.record()
    torch.cuda.synchronize()
    elapsed_ms = t_a.elapsed_time(t_b)
    total_bytes = sum(step_bytes[W:])
    gbs = total_bytes / (elapsed_ms * 1e-3) / 1e9
    qtok = sum(step_qtok[W:]) / (elapsed_ms * 1e-3)

    # ---- dominant kernel: average decode launch duration.  A graph of decode
    # launches only (every layer, several rounds) is replayed on the capture
    # stream and timed with events recorded on that stream.
    print("# timing decode launches", file=sys.stderr, flush=True)
    rounds = 4
    qd = queries[-1]
    gd = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gd, stream=cap_stream):
        for _ in range(rounds):
            for li, (ks, vs) in enumerate(streams):
                cda.decode_attention(qd, ks, vs, out=outs[li], workspace=ws)
    with torch.cuda.stream(cap_stream):
        gd.replay()
        e_a, e_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e_a.record(cap_stream)
        for _ in range(5):
            gd.replay()
        e_b.record(cap_stream)
    torch.cuda.synchronize()
    avg_s = e_a.elapsed_time(e_b) * 1e-3 / (5 * rounds * L)
    per_launch = decode_bytes(w, streams[0][0].n_blocks, streams[0][0].n_tail)
    achieved = per_launch / avg_s / 1e9
    traffic = load_traffic(w.name)
    print("# timing one decode launch over the layer stack", file=sys.stderr, flush=True)
    stack = layer_stack_timing(w, kd, vd, L, qd, dev, cap_stream, avg_s * 1e6)
    ops = archive_ops(w, streams, dev)
    print("# timing the streaming-read ceiling", file=sys.stderr, flush=True)
    ceiling = read_ceiling(per_launch, L, dev, cap_stream)

    res = {
        "metric": "decode-attn compressed-KV GB/s + query-heads*tokens/s at 1 GPU; % of HBM peak",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(elapsed_ms / K, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32",
        "arith": arith_note(w), "data": "synthetic AR(1) KV drawn on the device (seeded), N(0,1) q",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "T0": w.T,
                   "R": w.R, "S": w.S, "k_rows": w.kfmt, "v_rows": w.vfmt, "layers_rotated": L,
                   "step": "per layer: codec_decode_attention_append (append + decode), HIP graph per step"},
        "query_head_tokens_per_s": round(qtok, 1),
        "hbm_peak_fraction": round(gbs / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "decode_kernel", "avg_launch_us": round(avg_s * 1e6, 3),
                     "algorithmic_bytes_per_launch": per_launch},
        "read_ceiling": {**ceiling, "decode_frac_of_ceiling": round(achieved / ceiling["GBps"], 4)},
        "encode": {"avg_ms": round(float(np.mean(enc_ms[1:] or enc_ms)), 4),
                   "bytes": enc_bytes,
                   "GBps": round(enc_bytes / (float(np.mean(enc_ms[1:] or enc_ms)) * 1e-3) / 1e9, 2)},
        "layer_stack": stack,
        **ops,
    }
    if not args.no_cpu_baseline:
        print("# timing the oracle on the host cores", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w, k, v, queries[0].cpu())
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
