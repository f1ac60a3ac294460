"""Build libcsa.so, the gfx950 HIP library behind include/csa.h, and
libcsa_probe.so, the measurement helper that bench.py's stream-read workload
uses (not part of the C ABI).

    python -m long_context_sparse_compress_amd.build

Every source is compiled with hipcc for gfx950 only, -O3, without fast-math,
and with packed fp32 instructions disabled.  Objects go to _build/ next to
this file; the libraries are written in-tree next to this file.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libcsa.so")
SOURCES = ["capi.cpp", "compress.hip", "indexer.hip", "topk.hip", "attention.hip", "rope.hip", "pool.hip"]
PROBE_SOURCES = ["probe/stream_read.hip"]
PROBE_LIB = os.path.join(HERE, "libcsa_probe.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-x", "hip",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-ffp-contract=fast", "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
            "-Wno-unused-command-line-argument"]


# Per-source extra flags.  The indexer's epilogue takes ReLU of MFMA results,
# which are never NaN for the finite inputs it accepts (NaN inputs are
# unsupported): without NaN semantics fmaxf(x, 0) is one v_max_f32 instead of
# a NaN-quieting canonicalize plus the max.  MFMA results are taken in VGPRs
# (not AGPRs) because every one of them feeds VALU work straight away.
EXTRA = {"indexer.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0].replace("/", "_") + ".o")
    cmd = [hipcc()] + flags() + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs: list[str], lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    try:
        build()
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
