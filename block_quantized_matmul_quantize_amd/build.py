"""Build libqmm.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

    python -m block_quantized_matmul_quantize_amd.build

Object files go to _build/ at the repository root; the shared library lands next to this file.
Device code is compiled with packed fp32 instructions disabled (-packed-fp32-ops) and without
fast-math, so the q8_1 division, rounding and fp16 conversions are the IEEE operations.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libqmm.so")
PROBE_LIB = os.path.join(HERE, "libqmm_probe.so")   # measurement probes for bench.py (include/qmm_probe.h)
SOURCES = ["quantize.hip", "mmvq.hip", "mmvq_stream.hip", "mmvq_dot4.hip", "mmq.hip", "moe.hip", "f16act.hip",
           "noalloc.hip", "repack.hip", "api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          f"-I{os.path.join(ROOT, 'include')}"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-rdc", "-munsafe-fp-atomics"]


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [HIPCC, "-x", "hip", *DEVICE, *COMMON, "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, *COMMON, "-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr).strip()
    # hipcc's host pass does not know the packed-fp32 feature flag; that warning is harmless
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln and "is not a recognized feature" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n" + "\n".join(lines))
    if lines and verbose:
        print("\n".join(lines))
    return obj


def _link(objs, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + ["probe.hip"]
    jobs = min(len(srcs), max(1, (os.cpu_count() or 2)), 8)
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    _link(objs[:-1], LIB, verbose)
    _link(objs[-1:], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
