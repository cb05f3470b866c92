"""Build libpa.so (the C-ABI library) in-tree with hipcc for gfx950.

    python -m paged_kv_cache_103_amd.build        # or __graft_entry__.build()

Every source under csrc/ is compiled for gfx950 with packed-fp32 vector
instructions disabled, then linked into paged_kv_cache_103_amd/lib/libpa.so.
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
BUILD = os.path.join(PKG, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libpa.so")
PEAKS_LIB = os.path.join(LIBDIR, "libpa_peaks.so")

ARCH = "gfx950"
SOURCES = ["pa_api.cpp", "pa_check.cpp", "pa_blocks.cpp", "reshape_and_cache.hip", "copy_blocks.hip", "decode.hip", "decode_mfma.hip",
           "sparse_select.hip", "merge_lse.hip", "mla_decode.hip", "prefill_bf16.hip", "noalloc.hip"]
# the achievable-peak probes bench.py runs beside the path (a library of their own)
PEAKS_SOURCES = ["peaks.hip"]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else (shutil.which("hipcc") or "hipcc")


def compile_flags() -> list[str]:
    return [
        "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
        # keep the compiler from emitting packed fp32 vector ops
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
        "-Wall", "-Wno-unused-result",
    ]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = [] if src.endswith(".hip") else ["-x", "hip"]
    cmd = [hipcc()] + compile_flags() + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs: list[str], out: str) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    srcs = SOURCES + PEAKS_SOURCES
    workers = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PEAKS_LIB)
    if verbose:
        print(f"built {LIB} and {PEAKS_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
