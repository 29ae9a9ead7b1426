"""Build libsage_attn.so (the attention path) and libsage_probe.so (the
micro-benchmarks bench.py --mfma-probe runs) in-tree with hipcc for gfx950.

Usage: python -m quantized_attention_qk_amd.build   (or call build()).
Every call recompiles all sources.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libsage_attn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
PROBE_PATH = os.path.join(PKG, "libsage_probe.so")

ARCH = "gfx950"
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC",
    # no packed-FP32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]
SOURCES = {
    # prepass decisions must be reproducible bit for bit: no FP contraction
    "prepass.hip": ["-ffp-contract=off"],
    "attn_fwd.hip": ["-ffp-contract=off"],
    # the attention kernel's variants, one translation unit per (d, P~V mode)
    **{f"attn_fwd_d{d}_{pv}.hip": ["-ffp-contract=off"]
       for d in (64, 128) for pv in ("fp16", "fp8", "int8")},
    "smooth_q.hip": ["-ffp-contract=off"],
    "ref_rows.hip": [],
    "sage_api.cpp": [],
    "sage_noalloc.hip": [],
}
PROBE_SOURCES = {"probe.hip": []}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD_DIR, src + ".o")
    cmd = [hipcc(), *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs: list[str], path: str) -> None:
    tmp = path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, path)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = {**SOURCES, **PROBE_SOURCES}
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        objs = dict(zip(jobs, ex.map(lambda kv: _compile(*kv), jobs.items())))
    _link([objs[s] for s in SOURCES], LIB_PATH)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_PATH)
    if verbose:
        print(f"built {LIB_PATH} and {PROBE_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
