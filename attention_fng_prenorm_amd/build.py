"""Build libfng.so (the HIP kernels + C ABI) in-tree for gfx950.

Usage:  python -m attention_fng_prenorm_amd.build   (or build_library() from Python)
Objects go to _build/ at the repo root; the library lands next to this file.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libfng.so")
SOURCES = ["fng_api.cpp", "fng_gemm.hip", "fng_fulln.hip", "fng_norm.hip", "fng_attention.hip", "fng_fna.hip",
           "fng_fna_bwd.hip"]
ARCH = "gfx950"

# packed-fp32 ops are disabled for all device code; -O3 must not form
# v_pk_{add,mul,fma}_f32 on its own.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"--offload-arch={ARCH}",
          "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def _compile(src, obj):
    cmd = [_hipcc(), *COMMON, *DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-6000:]}")
    # the host pass warns that it does not know the packed-fp32 feature: harmless
    warn = "\n".join(ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln)
    return warn


def build_library(verbose=True):
    bdir = os.path.join(ROOT, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = [os.path.join(bdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        warns = list(ex.map(_compile, SOURCES, objs))
    for s, w in zip(SOURCES, warns):
        if w.strip() and verbose:
            print(f"[build] {s}:\n{w}", file=sys.stderr)
    tmp = OUT + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-4000:]}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"[build] wrote {OUT}", file=sys.stderr)
    return OUT


if __name__ == "__main__":
    build_library()
