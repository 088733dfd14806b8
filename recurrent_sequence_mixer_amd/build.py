"""Build libdn.so (HIP kernels for gfx950 + the C-ABI host library) in-tree.

    python -m recurrent_sequence_mixer_amd.build

Each source is compiled to an object under _build/ in parallel, then linked
into recurrent_sequence_mixer_amd/libdn.so.  Every call recompiles.  The
checking build libdn_debug.so (-DDN_DEBUG: every kernel's LDS starts as NaN)
is built the same way from objects under _build/debug/.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdn.so")
ARCH = "gfx950"

SOURCES = ["dn_api.cpp", "decode_step.hip", "gain_prep.hip", "chunk_fwd.hip", "chunk_fwd_ws.hip",
           "segment_combine.hip", "segment_stats.hip", "chunk_bwd.hip", "pad.hip", "token_fwd.hip"]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"--offload-arch={ARCH}",
    # no packed-fp32 instructions on the device
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libdn.so")
    return path


def _compile(src: str, outdir: str = BUILD, extra=()) -> str:
    obj = os.path.join(outdir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{r.stderr}")
    return obj


def link(objs, lib: str, extra=()) -> str:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking {os.path.basename(lib)} failed:\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


def _build_variant(outdir: str, lib: str, extra=(), verbose: bool = False) -> str:
    os.makedirs(outdir, exist_ok=True)
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, outdir, extra), SOURCES))
    link(objs, lib)
    if verbose:
        print(f"built {lib}")
    return lib


def build(verbose: bool = False) -> str:
    return _build_variant(BUILD, LIB, (), verbose)


def build_debug(verbose: bool = False) -> str:
    """libdn_debug.so: the same sources with -DDN_DEBUG (LDS poisoned with NaN)."""
    return _build_variant(os.path.join(BUILD, "debug"), os.path.join(PKG, "libdn_debug.so"),
                          ("-DDN_DEBUG",), verbose)


if __name__ == "__main__":
    build(verbose=True)
    build_debug(verbose=True)
    sys.exit(0)
