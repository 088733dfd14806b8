"""libdn_hostasan.so: libdn.so with its host code (the C-ABI layer,
dn_api.cpp) compiled under AddressSanitizer and the device kernels as in
the release build (the sanitizer flags apply to the host pass only).  The
CPU test suite loads it in a child process with the sanitizer runtime
preloaded and runs the ABI checks through it.  Needs the release objects
under _build/ (build.build() first).
"""
from __future__ import annotations

import os
import subprocess

from recurrent_sequence_mixer_amd import build as b

LIB = os.path.join(b.PKG, "libdn_hostasan.so")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def runtime() -> str:
    """The sanitizer runtime of the compiler hipcc drives (for LD_PRELOAD)."""
    r = subprocess.run([b.hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                       text=True)
    path = r.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        import glob
        found = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
        path = found[-1] if found else ""
    return path


def build_hostasan(verbose: bool = False) -> str:
    outdir = os.path.join(b.BUILD, "hostasan")
    os.makedirs(outdir, exist_ok=True)
    api = b._compile("dn_api.cpp", outdir, SAN)
    objs = [api] + [os.path.join(b.BUILD, os.path.splitext(s)[0] + ".o") for s in b.SOURCES
                    if s != "dn_api.cpp"]
    b.link(objs, LIB, ["-shared-libsan", "-fsanitize=address"])
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build_hostasan(verbose=True)
