"""Build libsa.so (the C-ABI library) from the HIP sources for gfx950.

Run as ``python -m indexer_routed_sparse_amd.build`` or call ``build()``. Every
source is compiled with hipcc for gfx950 only, objects in parallel, then linked
into ``indexer_routed_sparse_amd/libsa.so`` next to this file. A second library,
``libsa_debug.so``, links the same kernels with an entry-point layer built with
SA_DEBUG_CHECKS: its calls validate index values and sequence offsets on the device
first and return SA_ERR_SHAPE when one is out of range (and synchronise the stream
to do so).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libsa.so")
OUT_DEBUG = os.path.join(HERE, "libsa_debug.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["sa_api.hip", "sa_noalloc.hip", "sa_checks.hip", "topk_select.hip", "sparse_mla.hip",
           "sparse_mla_bwd.hip", "indexer.hip", "indexer_kl.hip", "block_gqa.hip", "block_gqa_bwd.hip", "routes.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# Per-source extra flags. indexer.hip: the generic indexer's score MFMAs accumulate in
# VGPRs rather than AGPRs, so its epilogue (ReLU, head weight, head sum) reads the scores
# without an AGPR-to-VGPR copy each (4-7 % on the block-routed indexer; the 64-head
# kernel issues its MFMAs by inline asm and is unaffected).
EXTRA = {"indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(job) -> str:
    src, tag, extra = job
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + tag + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = [(src, "", EXTRA.get(src, [])) for src in SOURCES] + [("sa_api.hip", "_debug", ["-DSA_DEBUG_CHECKS"])]
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, jobs))
    release, debug_api = objs[:len(SOURCES)], objs[len(SOURCES)]
    _link(release, OUT)
    _link([debug_api] + release[1:], OUT_DEBUG)
    if verbose:
        print(f"built {OUT} and {OUT_DEBUG}")
    return OUT


if __name__ == "__main__":
    build()
    sys.exit(0)
