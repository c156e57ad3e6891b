"""Build libcdattn.so in-tree with hipcc for gfx950 (run on any host; no GPU needed).

    python -m compressed_domain_attention_amd.build
"""

import concurrent.futures as cf
import os
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libcdattn.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "encode.hip", "archive.hip", "scratch.hip", "measure.hip"] + [f"decode_{k}_{v}.hip" for k in ("i8", "bf16", "f32") for v in ("i8", "bf16", "f32")]

# Packed fp32 VALU ops are disabled for all device code.
# Leading scalar kernel arguments are preloaded into SGPRs at wave launch
# (the compiler keeps a loading entry for firmware without the feature).
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-kernarg-preload-count=16",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-Wno-unused-command-line-argument"]


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    t0 = time.time()
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{errs}")
    return obj, time.time() - t0


def build(verbose=True, jobs=None):
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, SOURCES))
    if verbose:
        for (obj, dt) in results:
            print(f"  compiled {os.path.basename(obj)} in {dt:.1f}s", flush=True)
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *[o for o, _ in results], "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"  linked {LIB}", flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
