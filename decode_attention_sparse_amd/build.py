"""Build libsdkv.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m decode_attention_sparse_amd.build  (or build() from Python).
Every call recompiles: each source to an object (in parallel), then one link.
The library lands next to this file; objects go to _build/ beside it.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsdkv.so")
SOURCES = ["api.hip", "decode.hip", "topk.hip", "encode.hip", "noalloc.hip"]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-result",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    return "hipcc"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr).strip()
    # the host compiler pass does not know the device-only feature flag
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(lines))
    if lines and verbose:
        print("\n".join(lines))


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    inc = ["-I", os.path.join(HERE, "..", "include")]
    srcs = list(SOURCES)
    objs = [os.path.join(OBJ, os.path.splitext(s)[0] + ".o") for s in srcs]
    cmds = [[hipcc(), *FLAGS, *inc, "-c", os.path.join(CSRC, s), "-o", o]
            for s, o in zip(srcs, objs)]
    with ThreadPoolExecutor(max_workers=min(len(cmds), 8)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
