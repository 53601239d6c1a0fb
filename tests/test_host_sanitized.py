"""The host-side argument checks of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

The library's host code (validation, status strings, workspace queries and
launch set-up of every entry point) is rebuilt with both sanitizers; the ABI
host tests then run in a child process that preloads the sanitizer runtime
and loads that build instead of the release one.  Any sanitizer report ends
the child with a non-zero status.
"""

import os
import subprocess
import sys

from moe_decoder_step_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_host_checks_clean_under_asan_and_ubsan():
    lib = B.build_sanitized()
    rt = B.sanitizer_runtime()
    assert os.path.isfile(rt), rt
    env = dict(os.environ)
    env.update({
        "MOESTEP_LIB": lib,
        "LD_PRELOAD": rt,
        # the interpreter itself is not leak-clean; everything else aborts
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    probe = ("import ctypes, moe_decoder_step_amd._lib as L; lib = L.load(); "
             "assert L.LIB_PATH.endswith('libmoestep_san.so'); "
             "ctypes.CDLL(None).__asan_init; ctypes.CDLL(None).__ubsan_handle_add_overflow; print('sanitized')")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "sanitized" in r.stdout, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "tests/test_abi_host.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
