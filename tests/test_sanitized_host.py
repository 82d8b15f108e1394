"""The host library (prefix tree, planner, C ABI) built with AddressSanitizer
and UndefinedBehaviorSanitizer runs the C-ABI and planner CPU tests clean.

The sanitized build (prefix_shared_kv_tree_amd/build_sanitized.py) leaves
the kernels out; the tests run in a child Python process that preloads the
sanitizer runtime and loads that library through PKVT_LIB.  Any sanitizer
report aborts the child, failing this test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_TESTS = ["tests/test_capi_tree.py", "tests/test_capi_token_tree.py",
              "tests/test_decode_trace.py", "tests/test_prefill_plan.py"]


def test_host_library_under_asan_and_ubsan():
    from prefix_shared_kv_tree_amd import build_sanitized as S
    try:
        lib = S.build()
    except (OSError, RuntimeError) as e:          # pragma: no cover - toolchain missing
        pytest.skip(f"sanitized build unavailable: {e}")
    env = S.run_env()
    probe = subprocess.run(
        [sys.executable, "-c", "from prefix_shared_kv_tree_amd import binding as B; B.load(); "
         "print(B.LIB_PATH); print(open('/proc/self/maps').read().count('libpkvt_san.so') > 0)"],
        cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120)
    assert probe.returncode == 0, probe.stdout
    assert probe.stdout.split()[-2:] == [lib, "True"], probe.stdout
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-n", "4",
                        "-p", "no:cacheprovider", *HOST_TESTS],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, timeout=900)
    tail = r.stdout[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stdout and "runtime error:" not in r.stdout, tail
    assert " passed" in tail
