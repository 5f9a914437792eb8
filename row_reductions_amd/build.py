"""Builds liblr.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

    python row_reductions_amd/build.py

(run as a script: it does not import the package, whose import loads the
library it is about to replace).

Objects go to ``_build/`` at the repository root; the shared library is
written next to this file, where the Python binding loads it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblr.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed-FP32 VALU instructions (v_pk_add/mul/fma_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    # the first nine kernel arguments (the row-addressing fields every
    # kernel entry takes ahead of its KArgs, csrc/lr_entry.hpp) arrive
    # preloaded in scalar registers at wave launch
    "-mllvm", "-amdgpu-kernarg-preload-count=9",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]

# Per-source extra flags.  The ordered-fold kernels must round every
# operation on its own and use IEEE division and square root.
ORDERED_FLAGS = ["-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt"]
TREE_OPS = ["softmax", "cross_entropy", "rmsnorm", "layernorm", "add_layernorm", "row_sum", "row_minmax"]
EXTRA = {"k_ordered.hip": ORDERED_FLAGS, "k_ordered_lane.hip": ORDERED_FLAGS}
EXTRA.update({f"k_tree_{op}.hip": ORDERED_FLAGS for op in TREE_OPS})

SOURCES = [
    "lr_abi.cpp",
    "lr_planner.cpp",
    "lr_noalloc.hip",
    "k_softmax.hip",
    "k_rmsnorm.hip",
    "k_layernorm.hip",
    "k_cross_entropy.hip",
    "k_add_layernorm.hip",
    "k_row_sum.hip",
    "k_row_minmax.hip",
    "k_copy_rows.hip",
    "k_ordered.hip",
    "k_ordered_lane.hip",
    *[f"k_tree_{op}.hip" for op in TREE_OPS],
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *COMMON, *EXTRA.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every source and link liblr.so.  Returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
