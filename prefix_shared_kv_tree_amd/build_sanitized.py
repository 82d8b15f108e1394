"""Build the host library (prefix tree, planner, C ABI) with AddressSanitizer
and UndefinedBehaviorSanitizer, for running the CPU test suite under them.

    python -m prefix_shared_kv_tree_amd.build_sanitized

The kernels are not part of this build: the launch interface comes from
``csrc/launch_stubs.cpp`` (every launch reports that no device is present),
so only host code is instrumented and the library is for CPU tests only.
It lands in ``_build/sanitized/libpkvt_san.so``; point the binding at it with
``PKVT_LIB`` and preload the sanitizer runtime into the Python process
(``run_env`` gives the environment):

    PKVT_LIB=_build/sanitized/libpkvt_san.so \\
    LD_PRELOAD=$(g++ -print-file-name=libasan.so) \\
    ASAN_OPTIONS=detect_leaks=0 UBSAN_OPTIONS=print_stacktrace=1 \\
    python -m pytest tests -m "not gpu" -p no:cacheprovider
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(ROOT, "_build", "sanitized")
LIB = os.path.join(OUT, "libpkvt_san.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

SOURCES = ["tree.cpp", "plan.cpp", "capi.cpp", "launch_stubs.cpp"]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer"]
FLAGS = ["-O1", "-g", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter",
         "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{INCLUDE}", f"-I{CSRC}"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("sanitized build step failed:\n" + " ".join(cmd) + "\n" + r.stdout)


def build() -> str:
    os.makedirs(OUT, exist_ok=True)
    objs = [os.path.join(OUT, s + ".o") for s in SOURCES]
    jobs = [["g++", *FLAGS, *SAN, "-c", os.path.join(CSRC, s), "-o", o]
            for s, o in zip(SOURCES, objs)]
    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        list(ex.map(_run, jobs))
    tmp = LIB + ".tmp"
    _run(["g++", "-shared", *SAN, *objs, f"-L{ROCM}/lib", "-lamdhip64",
          f"-Wl,-rpath,{ROCM}/lib", "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


def runtime() -> str:
    """Path of the AddressSanitizer runtime the library was linked against."""
    return subprocess.run(["g++", "-print-file-name=libasan.so"], stdout=subprocess.PIPE,
                          text=True, check=True).stdout.strip()


def run_env(base=None) -> dict:
    """Environment for a Python process that loads the sanitized library."""
    env = dict(os.environ if base is None else base)
    env["PKVT_LIB"] = LIB
    env["LD_PRELOAD"] = runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return env


if __name__ == "__main__":
    print("built", build())
    sys.exit(0)
