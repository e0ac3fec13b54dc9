"""The CPU-side checks of the C ABI (tests/test_abi.py) once more, against a
build whose host layer carries AddressSanitizer and UndefinedBehaviorSanitizer
(device code is not instrumented).  The ASan runtime is preloaded into a child
Python process; any sanitizer report fails the run."""
import os
import subprocess
import sys

import pytest

from long_context_block_ssa_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _stale(lib):
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    srcs = _build.sources() + [os.path.join(ROOT, "include", "ssa.h")]
    return any(os.path.getmtime(s) > t for s in srcs)


@pytest.fixture(scope="module")
def san_env():
    if _stale(_build.SAN_LIB):
        _build.build(verbose=False, sanitize=True)
    rt = _build.asan_runtime()
    if not os.path.exists(rt):
        pytest.skip(f"ASan runtime not found ({rt!r})")
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, SSA_LIB_PATH=_build.SAN_LIB,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return env


def _run(cmd, env):
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


def test_sanitized_library_is_the_one_loaded(san_env):
    code = ("import ctypes, long_context_block_ssa_amd as s; s.load(); "
            "assert s.LIB_PATH.endswith('libssa_san.so'), s.LIB_PATH; "
            "ctypes.CDLL(None).__asan_init; print('ok')")
    assert "ok" in _run([sys.executable, "-c", code], san_env)


def test_abi_checks_under_asan_ubsan(san_env):
    out = _run([sys.executable, "-m", "pytest", "tests/test_abi.py", "-q", "-p", "no:cacheprovider"], san_env)
    assert " passed" in out
