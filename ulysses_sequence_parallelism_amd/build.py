"""Build libusp.so in-tree with hipcc for gfx950.

Usage: python -m ulysses_sequence_parallelism_amd.build [-v]

Every call recompiles (objects under _build/, the library under _lib/).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libusp.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3",
    "-std=c++17",
    f"--offload-arch={ARCH}",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Wno-unused-variable",
    # keep the compiler from forming packed-fp32 VALU ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
SOURCES = ["capi.hip", "trace.hip", "permute.hip", "kmajor.hip", "attn_f32.hip", "attn_fwd_bf16.hip",
           "attn_bwd_bf16.hip", "merge.hip", "splits.hip"]
# The matrix-core attention kernels never produce a NaN (masked scores are
# -inf, and every difference of two infinities is guarded), so they are built
# without NaN semantics: the row max then compiles to v_max3_f32 directly
# instead of first quieting every input. Infinities keep their meaning.
EXTRA = {"attn_fwd_bf16.hip": ["-fno-honor-nans"], "attn_bwd_bf16.hip": ["-fno-honor-nans"]}


def _compile(src: str, verbose: bool) -> str:
    out = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines()
            if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    return out


def build(verbose: bool = False) -> str:
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(OBJ, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    workers = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8")))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    # a kernel whose host launch stub was not emitted shows up only as an
    # undefined symbol of the library's own namespace: fail the build on it
    nm = shutil.which("nm")
    if nm:
        und = subprocess.run([nm, "-D", "--undefined-only", tmp], capture_output=True, text=True).stdout
        own = [ln.split()[-1] for ln in und.splitlines() if "_ZN3usp" in ln]
        if own:
            os.remove(tmp)
            raise RuntimeError("libusp.so has undefined internal symbols: " + ", ".join(own))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
