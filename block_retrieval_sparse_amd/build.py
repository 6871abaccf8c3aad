"""Build libbrs.so (gfx950) in-tree with hipcc.

    python block_retrieval_sparse_amd/build.py

Each source is compiled to an object under ``_build/`` in parallel, then
linked into ``block_retrieval_sparse_amd/libbrs.so``.  Packed-fp32 code
generation is turned off for all device code.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbrs.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "memory.hip", "score.hip", "topk.hip", "attn_decode.hip", "attn_prefill.hip",
           "mass.hip", "prune.hip", "measure.hip", "offload.hip"]

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-x", "hip",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is expected
    noise = "is not a recognized feature for this target"
    msg = "\n".join(line for line in (r.stdout + r.stderr).splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    # every kernel and function of the library must be defined in it: a host
    # stub the compiler silently failed to emit shows up as an undefined brs::
    # symbol, which would only fail when the library is loaded
    r = subprocess.run(["nm", "-C", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [line.strip() for line in r.stdout.splitlines() if "brs::" in line]
    if missing:
        raise RuntimeError("libbrs.so leaves library symbols undefined:\n" + "\n".join(missing[:20]))
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
