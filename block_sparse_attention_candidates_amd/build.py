"""Builds libdynrad.so (the C ABI of include/dynrad.h) for gfx950 with hipcc.

    python -m block_sparse_attention_candidates_amd.build

Objects go to block_sparse_attention_candidates_amd/_build/, the library to
block_sparse_attention_candidates_amd/libdynrad.so (in-tree, so it travels with
the source tree). Always recompiles.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libdynrad.so")
SOURCES = ["api.cpp", "candidates.hip", "score_select.hip", "attention.hip", "groups.hip", "token_select.hip",
           "static_select.hip", "proxy.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable", "-Wno-inline-asm",
    # packed fp32 VALU ops stay off: plain scalar fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# attention: inputs are finite (bf16 activations); without NaN semantics the
# compiler drops the canonicalising copies in front of every float max. Its
# machine scheduler runs the iterative ILP strategy: the same arithmetic and
# bitwise the same outputs, measured 2-4% faster than the default order
# (dense and dynamic-threshold launches, 1-2% static-ratio).
EXTRA = {"attention.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False) -> str:
    bdir = os.path.join(PKG, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([HIPCC, *COMMON, *EXTRA.get(src, []), "-c", os.path.join(PKG, "csrc", src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(4, len(cmds))) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
