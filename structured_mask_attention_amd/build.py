"""Build libmars.so (HIP for gfx950) in-tree: ``python -m structured_mask_attention_amd.build``.

Each source is compiled to an object under ``_build/`` in parallel with hipcc, then linked
into ``structured_mask_attention_amd/libmars.so``.  Always rebuilds.  Warnings are errors
(-Wall -Wextra -Werror); the compiler's messages are printed whether or not it succeeds.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmars.so")
SOURCES = ["mars_api.cpp", "attn_fwd.hip", "attn_bwd.hip", "decode.hip", "accept.hip", "mask_kernels.hip", "kv_commit.hip", "shifted_ce.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Werror",
    # Packed fp32 VALU ops stay off: the compiler would otherwise form them from float code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
# Kernel sources only: their inputs are finite, so max/min need no NaN quieting (saves
# canonicalising moves).  The host-side argument checks (mars_api.cpp) must see NaN, so they
# are built without it.
KERNEL_FLAGS = ["-fno-honor-nans"]
# The host pass of every file reports that it does not know the packed-fp32 target feature
# (it only applies to the device pass); that one notice is not printed.
_HOST_FEATURE_NOTICE = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"


def _messages(r) -> str:
    lines = (r.stdout + r.stderr).splitlines()
    return "\n".join(l for l in lines if l.strip() and l.strip() != _HOST_FEATURE_NOTICE)


def _compile(src: str) -> tuple[str, str]:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    extra = KERNEL_FLAGS if src.endswith(".hip") else []
    cmd = [HIPCC, *CFLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = _messages(r)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    return obj, msg


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = []
    for src, (obj, msg) in zip(SOURCES, results):
        objs.append(obj)
        if msg:
            print(f"[{src}]\n{msg}", file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = _messages(r)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{msg}")
    if msg:
        print(f"[link]\n{msg}", file=sys.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
