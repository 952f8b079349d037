"""Host-side hygiene on the CPU (no GPU is used or needed):

* the q8_1 scale shortcut (one multiply and an fma correction instead of amax / 127) checked over
  every positive finite fp32 amax, and shown to fail with the correction dropped;
* the CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer, every entry point
  driven on small inputs with exactly sized buffers;
* the library's host code (C ABI, argument checks, workspace layouts, planner, launch wrappers)
  built with the same sanitizers -- the sanitizers on the host pass only, the device code
  compiled as usual -- and driven through every entry point; launches fail for want of a device.
  The driver refuses to run (skip) when a GPU is visible, since it passes fake device pointers.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CDIR = os.path.join(ROOT, "tests", "c")
CSRC = os.path.join(ROOT, "block_quantized_matmul_quantize_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"
# sanitizer flags for hipcc apply to the host compilation only (-Xarch_host before each)
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return r.returncode, r.stdout + r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_q8_1_scale_shortcut_exhaustive(tmp_path):
    src = os.path.join(CDIR, "q8_1_scale_exhaustive.c")
    exe, planted = str(tmp_path / "q81"), str(tmp_path / "q81_planted")
    base = ["gcc", "-O2", "-mfma", "-ffp-contract=off", "-fopenmp", src, "-lm"]
    assert _run(base + ["-o", exe])[0] == 0
    assert _run(base + ["-DPLANT_NO_CORRECTION", "-o", planted])[0] == 0
    rc, out = _run([exe], timeout=300)
    assert rc == 0 and "mismatches 0" in out, out
    checked = int(out.split()[1])
    assert checked > 1_600_000_000          # about 200 binades of 2^23 values
    rc, out = _run([planted], timeout=300)
    assert rc != 0 and "mismatches 0" not in out, out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    rc, out = _run(["gcc", "-O1", "-g", "-std=c99", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-fopenmp", os.path.join(ROOT, "oracle", "qmm_oracle.c"),
                    os.path.join(CDIR, "oracle_sanitize.c"), "-o", exe, "-lm"])
    assert rc == 0, out
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", OMP_NUM_THREADS="4")
    rc, out = _run([exe], env=env, timeout=300)
    assert rc == 0 and out.strip().endswith("ok"), out


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain not installed")
def test_abi_host_code_under_address_and_ub_sanitizers(tmp_path):
    from block_quantized_matmul_quantize_amd.build import SOURCES
    srcs = list(SOURCES)   # every translation unit of libqmm

    def compile_one(name):
        obj = str(tmp_path / (os.path.splitext(name)[0] + ".o"))
        cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
               f"-I{os.path.join(ROOT, 'include')}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               *HOST_SAN, "-c", os.path.join(CSRC, name), "-o", obj]
        rc, out = _run(cmd)
        assert rc == 0, out
        return obj

    with ThreadPoolExecutor(min(8, os.cpu_count() or 2)) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv = str(tmp_path / "drv.o")
    rc, out = _run([HIPCC, "-x", "hip", "--offload-host-only", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
                    f"-I{os.path.join(ROOT, 'include')}", *HOST_SAN, "-c", os.path.join(CDIR, "abi_sanitize.cpp"),
                    "-o", drv])
    assert rc == 0, out
    exe = str(tmp_path / "abi_san")
    rc, out = _run([CLANG, "-fsanitize=address,undefined", *objs, drv, "-o", exe, "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib", "-lpthread"])
    assert rc == 0, out
    rc, out = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"), timeout=300)
    if out.startswith("skip"):
        pytest.skip(out.strip())
    assert rc == 0 and out.strip().endswith("ok"), out
