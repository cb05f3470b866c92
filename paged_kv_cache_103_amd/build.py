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


# Host sources of libpa.so: argument checking, plans, the block manager.
HOST_SOURCES = ["pa_api.cpp", "pa_check.cpp", "pa_blocks.cpp"]
SAN_LIB = os.path.join(BUILD, "libpa_host_sanitized.so")


def asan_runtime() -> str:
    """The AddressSanitizer runtime of hipcc's clang (preloaded into the
    Python process that loads the sanitized library)."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    base = os.path.join(rocm, "llvm", "lib", "clang")
    for ver in sorted(os.listdir(base), reverse=True) if os.path.isdir(base) else []:
        cand = os.path.join(base, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(cand):
            return cand
    raise FileNotFoundError("libclang_rt.asan-x86_64.so not found under " + base)


def build_host_sanitized() -> str:
    """libpa with its host sources built under AddressSanitizer and
    UndefinedBehaviorSanitizer (host code only: the GPU objects are the
    regular ones), for the CPU tests of the host logic. Returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = [f for f in compile_flags() if f != "-O3"] + ["-O1", "-g"] + san

    def one(src: str) -> str:
        obj = os.path.join(BUILD, "san_" + os.path.splitext(src)[0] + ".o")
        cmd = [hipcc()] + flags + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        return obj

    gpu_objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES if s not in HOST_SOURCES]
    if not all(os.path.exists(o) for o in gpu_objs):
        build()
    with ThreadPoolExecutor(len(HOST_SOURCES)) as ex:
        host_objs = list(ex.map(one, HOST_SOURCES))
    tmp = SAN_LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-o", tmp] + host_objs + gpu_objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
