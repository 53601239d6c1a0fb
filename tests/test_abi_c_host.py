"""The ABI from plain C, without a GPU: include/moestep.h is valid C99 and
C++11, and the C client (tests/c_client/verify_pass.c, built with the
library) links against libmoestep.so and sees the documented version, status
strings and error codes of bad arguments."""

import os
import subprocess

from moe_decoder_step_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moestep.h")


def test_header_is_plain_c99_and_cpp11():
    for cmd in (["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only", "-x", "c", HEADER],
                ["g++", "-std=c++11", "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only", "-x", "c++",
                 HEADER]):
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def test_c_client_host_checks():
    assert os.path.exists(B.C_CLIENT), "the C client is built with the library (python -m moe_decoder_step_amd.build)"
    r = subprocess.run([B.C_CLIENT, "host"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host checks ok" in r.stdout
