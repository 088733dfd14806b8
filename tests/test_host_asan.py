"""The host code of the library (argument validation, aliasing checks,
workspace layouts, dispatch: dn_api.cpp) under AddressSanitizer: the ABI
tests run in a child process against libdn_hostasan.so (built by
__graft_entry__.build()) with the sanitizer runtime preloaded.  CPU only: the
ABI tests launch nothing."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "recurrent_sequence_mixer_amd")


def test_abi_checks_under_address_sanitizer():
    from recurrent_sequence_mixer_amd import build_hostasan
    lib = build_hostasan.LIB
    if not os.path.exists(lib):
        pytest.skip("libdn_hostasan.so is not built (__graft_entry__.build() builds it)")
    if os.environ.get("LD_PRELOAD"):
        pytest.skip("another library is preloaded; the sanitizer runtime has to come first")
    rt = build_hostasan.runtime()
    assert rt, "no AddressSanitizer runtime next to the compiler"
    env = dict(os.environ, LD_PRELOAD=rt, DN_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0")
    # the child checks that it runs the sanitized library with the runtime in
    # place, then runs the ABI tests through it
    probe = ("import os; from recurrent_sequence_mixer_amd import dn; dn.lib(); "
             "maps = open('/proc/self/maps').read(); "
             "assert 'libdn_hostasan.so' in maps and 'asan' in maps, 'not sanitized'")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and "AddressSanitizer" not in r.stderr, (r.stdout[-2000:], r.stderr[-3000:])
