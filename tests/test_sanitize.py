"""The host planner (span, ring and work-list tables, argument checks) under AddressSanitizer
and UndefinedBehaviorSanitizer, on the CPU.

Opt-in (MOA_SANITIZE=1; about a minute and a half): builds the instrumented copy of the package
(heterogeneous_sliding_windows_amd/build.py --sanitize, host code only), then runs the host and
rules-file tests against it in a subprocess with the ASan runtime preloaded, so every table the
planner builds for those tests (the full-size workloads' included) is checked for out-of-bounds
accesses, use after free and undefined behaviour.  A planted out-of-bounds read through the C
ABI must abort, which shows the checks are live.
"""

import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(os.environ.get("MOA_SANITIZE") != "1",
                                reason="set MOA_SANITIZE=1 to build and run the sanitizer pass")


def _build_module():
    spec = importlib.util.spec_from_file_location(
        "moa_build", os.path.join(ROOT, "heterogeneous_sliding_windows_amd", "build.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


@pytest.fixture(scope="module")
def sanitized():
    b = _build_module()
    try:
        b.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    b.build(sanitize=True)
    env = dict(os.environ)
    env["LD_PRELOAD"] = b.sanitizer_runtime()
    # Python itself is not instrumented: leaks at exit are its own
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["PYTHONPATH"] = os.pathsep.join([os.path.dirname(b.SANITIZE_PKG), ROOT])
    return b, env


def _run(env, code, timeout=900):
    return subprocess.run([sys.executable, "-c", code], env=env, cwd="/tmp", capture_output=True,
                          text=True, timeout=timeout)


def test_host_and_rules_tests_are_clean(sanitized):
    b, env = sanitized
    code = (
        "import sys, pytest\n"
        "import heterogeneous_sliding_windows_amd as m\n"
        f"assert m.LIB_PATH == {os.path.join(b.SANITIZE_PKG, 'libmoa.so')!r}, m.LIB_PATH\n"
        "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', "
        f"{os.path.join(ROOT, 'tests', 'test_host.py')!r}, "
        f"{os.path.join(ROOT, 'tests', 'test_rules.py')!r}]))\n")
    r = _run(env, code)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail


def test_planted_out_of_bounds_read_is_caught(sanitized):
    """n_kv_heads one past the end of the alpha/beta arrays: the planner reads past them."""
    _, env = sanitized
    code = (
        "import ctypes, numpy as np\n"
        "import heterogeneous_sliding_windows_amd as m\n"
        "a = np.zeros(1000, dtype=np.int64); b = np.full(1000, 0.5); s = np.zeros(1001, dtype=np.int32)\n"
        "m._lib.moa_spans(a.ctypes.data_as(m._I64P), b.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),"
        " 1001, 4096, s.ctypes.data_as(m._I32P))\n"
        "print('not caught')\n")
    r = _run(env, code, timeout=300)
    assert r.returncode != 0 and "not caught" not in r.stdout, (r.stdout + r.stderr)[-2000:]
    assert "AddressSanitizer" in r.stderr and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]
