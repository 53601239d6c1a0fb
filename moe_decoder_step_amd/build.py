"""Build libmoestep.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m moe_decoder_step_amd.build            # the library (and the C client of its ABI)
    python -m moe_decoder_step_amd.build sanitize   # host ASan + UBSan build

Each source compiles to an object under moe_decoder_step_amd/_build/ (in
parallel), then one link produces moe_decoder_step_amd/libmoestep.so; gcc
then builds tests/c_client/verify_pass, a plain C client of the ABI.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoestep.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["abi.hip", "pack.hip", "route.hip", "permute.hip", "swiglu.hip", "gemm.hip", "combine.hip", "lmhead.hip",
           "verify.hip", "attention.hip", "noalloc.hip", "errors.hip", "validate.cpp"]

# Packed-fp32 VALU ops are switched off for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [HIPCC, f"--offload-arch={ARCH}", *COMMON, *DEVICE_FLAGS, *extra, "-c", path, "-o", obj]
    else:
        cmd = ["g++", *COMMON, *extra, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


# Host-sanitizer build: the host side of every source with AddressSanitizer
# and UndefinedBehaviorSanitizer (device code unchanged), for running the
# host-side checks of the ABI on the CPU.  Linked with the LLVM driver against
# its shared sanitizer runtime, which the Python process preloads.
SAN_BUILD = os.path.join(HERE, "_build_san")
SAN_LIB = os.path.join(SAN_BUILD, "libmoestep_san.so")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN_HOST = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def _compile_san(src: str) -> str:
    obj = os.path.join(SAN_BUILD, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        host = [f for flag in SAN_HOST for f in ("-Xarch_host", flag)]
        cmd = [HIPCC, f"--offload-arch={ARCH}", *COMMON, *DEVICE_FLAGS, *host, "-c", path, "-o", obj]
    else:
        cmd = [CLANGXX, *COMMON, *SAN_HOST, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build_sanitized(verbose: bool = False) -> str:
    """Compile the host side of every source with ASan + UBSan into
    _build_san/libmoestep_san.so; returns its path."""
    os.makedirs(SAN_BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile_san, SOURCES))
    cmd = [CLANGXX, "-shared", "-fPIC", *SAN_HOST, "-shared-libsan", *objs, "-L/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,/opt/rocm/lib", "-o", SAN_LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


def sanitizer_runtime() -> str:
    """Path of the LLVM shared ASan runtime the sanitized library needs preloaded."""
    r = subprocess.run([CLANGXX, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return r.stdout.strip()


# The plain C client of the ABI (tests/c_client): C99 with HIP's C runtime
# API, linked against the in-tree libmoestep.so (found next to it at run time).
C_CLIENT_SRC = os.path.join(ROOT, "tests", "c_client", "verify_pass.c")
C_CLIENT = os.path.join(ROOT, "tests", "c_client", "verify_pass")


def build_c_client(verbose: bool = False) -> str:
    """Compile tests/c_client/verify_pass.c with gcc; returns the binary's path."""
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-O2", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           f"-I{os.path.join(ROOT, 'include')}", C_CLIENT_SRC, f"-L{HERE}", "-lmoestep", "-L/opt/rocm/lib",
           "-lamdhip64", "-Wl,-rpath,$ORIGIN/../../moe_decoder_step_amd", "-Wl,-rpath,/opt/rocm/lib",
           "-o", C_CLIENT]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"C client build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {C_CLIENT}")
    return C_CLIENT


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile every source for gfx950 and link libmoestep.so, then the C
    client of the ABI; returns the library's path."""
    os.makedirs(BUILD, exist_ok=True)
    extra = list(extra or [])
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    build_c_client(verbose)
    return LIB


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "sanitize":
        build_sanitized(verbose=True)
    else:
        build(verbose=True)
    sys.exit(0)
