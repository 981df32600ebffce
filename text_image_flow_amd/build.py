"""Build liblens.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

    python -m text_image_flow_amd.build        # or build() from Python

Objects go to _build/ at the repository root; the shared library is written
next to this file, where the binding loads it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "liblens.so")
BUILD = os.path.join(ROOT, "_build")
SOURCES = ("api.hip", "gemm.hip", "attention.hip", "elementwise.hip")
ARCH = os.environ.get("LENS_OFFLOAD_ARCH", "gfx950")
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 instructions off: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable", "-Wno-unused-result",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build liblens.so)")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; harmless
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{err}")
    return err


# per-source extra flags: the attention kernel keeps its MFMA accumulators in
# VGPRs (the softmax reads them with VALU instructions every tile)
EXTRA = {"attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []
    jobs = []
    for s in SOURCES:
        o = os.path.join(BUILD, s.replace(".hip", ".o"))
        objs.append(o)
        jobs.append([cc, *FLAGS, *EXTRA.get(s, []), "-c", os.path.join(CSRC, s), "-o", o])
    with ThreadPoolExecutor(len(jobs)) as ex:
        for msg in ex.map(_run, jobs):
            if verbose and msg.strip():
                print(msg, file=sys.stderr)
    tmp = OUT + ".tmp"
    _run([cc, *FLAGS, "-shared", *objs, "-o", tmp])
    os.replace(tmp, OUT)
    return OUT


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the same
# sources (device code unchanged: every sanitizer flag applies to the host
# pass only), for running the C-ABI argument tests on the CPU under the
# sanitizers.  Load it with the ASan runtime preloaded (asan_runtime()).
SAN_OUT = os.path.join(BUILD, "asan", "liblens_asan.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-shared-libasan", "-g"]


def asan_runtime() -> str:
    """Path of the shared ASan runtime of the compiler that builds the library."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "lib", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return r.stdout.strip()


def build_sanitized() -> str:
    d = os.path.dirname(SAN_OUT)
    os.makedirs(d, exist_ok=True)
    cc = hipcc()
    objs, jobs = [], []
    for s in SOURCES:
        o = os.path.join(d, s.replace(".hip", ".o"))
        objs.append(o)
        jobs.append([cc, *FLAGS, *SAN_FLAGS, *EXTRA.get(s, []), "-c", os.path.join(CSRC, s), "-o", o])
    with ThreadPoolExecutor(len(jobs)) as ex:
        list(ex.map(_run, jobs))
    _run([cc, *FLAGS, *SAN_FLAGS, "-shared", *objs, "-o", SAN_OUT])
    return SAN_OUT


if __name__ == "__main__":
    print(build(verbose=True))
