"""Build libkda.so (gfx950 HIP kernels + the C ABI) in-tree with hipcc.

    python -m gated_delta_rule_log2_amd.build

Every translation unit is compiled for gfx950 only, with packed-fp32 code
generation turned off, into _build/, then linked next to this file; the linked
code is scanned for misplaced spill stores (codecheck.py) before it is installed.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIBRARY = os.path.join(HERE, "libkda.so")
SOURCES = [
    "kda_abi.cpp", "kda_dispatch.hip", "kda_plan_gate.hip",
    "kda_intra_c64_bf16.hip", "kda_intra_c64_f32.hip", "kda_intra_c32_bf16.hip", "kda_intra_c32_f32.hip",
    "kda_recur_c64_bf16.hip", "kda_recur_c64_f32.hip", "kda_recur_c32_bf16.hip", "kda_recur_c32_f32.hip",
    "kda_recurrent.hip", "kda_backward.hip", "kda_noalloc.hip",
    "kda_bwd_chunk_bf16.hip", "kda_bwd_chunk_f32.hip",
]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build_library(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(os.cpu_count() or 4, 16, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIBRARY + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    # spill stores placed under a region's exec mask at a join (codecheck.py) give wrong
    # reloads at run time; such a build is refused before it replaces the library
    from . import codecheck
    findings = codecheck.check_library(tmp)
    if findings:
        os.remove(tmp)
        raise RuntimeError("spill stores under a narrowed exec mask in the built code:\n" + "\n".join(findings))
    os.replace(tmp, LIBRARY)
    if verbose:
        print(f"built {LIBRARY}")
    return LIBRARY


if __name__ == "__main__":
    build_library(verbose=True)
    sys.exit(0)
