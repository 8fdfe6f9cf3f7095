"""Build libtreeattn.so (and the small libmfmaceiling.so that bench.py
--mfma-ceiling uses) for gfx950 with hipcc (in-tree, no JIT cache).

    python -m shared_prompt_tree_amd.build
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIBDIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIBDIR, "libtreeattn.so")
CEILING_LIB = os.path.join(LIBDIR, "libmfmaceiling.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["attn_fwd.hip", "attn_bwd.hip", "aux_kernels.hip", "tree_attn_api.cpp"]
CEILING_SOURCES = ["mfma_ceiling.hip"]
LIBRARIES = {LIB: SOURCES, CEILING_LIB: CEILING_SOURCES}
# Packed float32 VALU instructions are kept out of the device code.
FLAGS = ["-x", "hip", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-Wno-unused-command-line-argument"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("command failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
    return r


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link the shared libraries.
    Returns the path of libtreeattn.so."""
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(BUILD, src + ".o")
        _run([HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose:
            print("compiled", src, flush=True)
        return obj

    every = [src for srcs in LIBRARIES.values() for src in srcs]
    with ThreadPoolExecutor(max_workers=min(len(every), os.cpu_count() or 1)) as ex:
        objs = dict(zip(every, ex.map(compile_one, every)))
    for lib, srcs in LIBRARIES.items():
        tmp = lib + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp,
              *(objs[src] for src in srcs)])
        os.replace(tmp, lib)
        if verbose:
            print("linked", lib, flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
