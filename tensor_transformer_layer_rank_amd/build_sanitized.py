"""Host-sanitizer build of libtpshard.

    python -m tensor_transformer_layer_rank_amd.build_sanitized [--run-tests]

The C-ABI front end (csrc/api.cpp: argument validation, shape limits, size and workspace
arithmetic, dispatch) is compiled by g++ with AddressSanitizer and UndefinedBehaviorSanitizer
(host code only: api.cpp holds no device code) and linked with the unchanged kernel objects
of the regular build into _build/sanitized/libtpshard_san.so. The sanitizer runtimes are not linked in:
they are preloaded into the Python process that loads the library (sanitized_env()), and
TPSHARD_LIB points the package at it. --run-tests runs tests/test_abi_host.py that way; any
sanitizer report aborts the run.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys

from . import build as _build

SAN_DIR = os.path.join(_build.BUILD, "sanitized")
SAN_LIB = os.path.join(SAN_DIR, "libtpshard_san.so")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def _gxx() -> str:
    g = shutil.which("g++")
    if not g:
        raise RuntimeError("g++ not found")
    return g


def runtimes() -> list[str]:
    """Paths of the GCC AddressSanitizer and UBSan runtimes (empty if not installed)."""
    out = []
    for name in ("libasan.so", "libubsan.so"):
        r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
        p = r.stdout.strip()
        if r.returncode != 0 or not os.path.isabs(p) or not os.path.exists(p):
            return []
        out.append(p)
    return out


def sanitized_env(base: dict | None = None) -> dict:
    env = dict(os.environ if base is None else base)
    env["LD_PRELOAD"] = " ".join(runtimes() + ([env["LD_PRELOAD"]] if env.get("LD_PRELOAD") else []))
    # leak checking would report the HIP runtime's process-lifetime allocations
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["TPSHARD_LIB"] = SAN_LIB
    return env


def build() -> str:
    """Compile api.cpp with the sanitizers and link it with the regular kernel objects."""
    objs = [os.path.join(_build.BUILD, os.path.splitext(s)[0] + ".o") for s in _build.SOURCES if s != "api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        _build.build()
    os.makedirs(SAN_DIR, exist_ok=True)
    api_o = os.path.join(SAN_DIR, "api.o")
    cmd = [_gxx(), "-std=c++17", "-O1", "-g", "-fPIC", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           f"-I{_build.INCLUDE}", f"-I{_build.CSRC}", *SAN_FLAGS, "-c", os.path.join(_build.CSRC, "api.cpp"),
           "-o", api_o]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # the kernel objects carry gfx950 code, so the device link stays the regular one; the
    # sanitizer symbols of the rebuilt api.o resolve against the preloaded runtimes
    tmp = SAN_LIB + ".tmp"
    cmd = [_build.hipcc(), f"--offload-arch={_build.ARCH}", "-shared", "-fPIC", api_o, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


def run_host_tests() -> subprocess.CompletedProcess:
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
           os.path.join(_build.ROOT, "tests", "test_abi_host.py")]
    return subprocess.run(cmd, cwd=_build.ROOT, env=sanitized_env(), capture_output=True, text=True, timeout=900)


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--run-tests", action="store_true")
    a = ap.parse_args()
    print(f"built {build()}")
    if a.run_tests:
        r = run_host_tests()
        print(r.stdout[-3000:], r.stderr[-3000:])
        sys.exit(r.returncode)
