"""Builds libswa.so (the C-ABI library with its HIP kernels) for gfx950, in-tree.

    python -m decode_attention_fixed_amd.build

Every translation unit is compiled by hipcc for --offload-arch=gfx950 with
packed-fp32 instruction selection switched off, then linked into
decode_attention_fixed_amd/libswa.so next to this file.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libswa.so")

SOURCES = ["swa_api.cpp", "pager_api.cpp", "blocks_api.cpp", "append_rope.hip", "decode.hip", "decode_mfma.hip", "decode_shared.hip",
           "prefill.hip", "pager.hip", "positions.hip", "stream_read.hip"]
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libswa")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-xhip")
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    # the host pass does not know the gfx950-only feature name; drop that noise
    noise = "is not a recognized feature for this target"
    rest = "\n".join(ln for ln in res.stderr.splitlines() if noise not in ln).strip()
    if rest and verbose:
        print(rest, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libswa.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as pool:
        objs = list(pool.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    # -z defs: an unresolved symbol (say a kernel stub that the host pass did
    # not emit) fails the link instead of the first dlopen.
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
