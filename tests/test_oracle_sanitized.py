"""The oracle's own pins, rerun against a build of oracle.c instrumented
with AddressSanitizer and UndefinedBehaviorSanitizer (host code only), every
finding fatal: an out-of-bounds access, a signed overflow or an undefined
shift in the checker would end the child process with an error."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    try:
        path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                              text=True, check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_sanitizers(tmp_path):
    asan = _asan_runtime()
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    sys.path.insert(0, ROOT)
    from oracle import build
    lib = build.build(sanitize=True, out=str(tmp_path / "liboracle_san.so"))
    env = dict(os.environ)
    env.update(ORACLE_LIB=lib, LD_PRELOAD=asan, OMP_NUM_THREADS="4",
               # the interpreter's own allocations are not the oracle's to free
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    tests = sorted(f for f in os.listdir(os.path.join(ROOT, "tests"))
                   if f.startswith("test_oracle_") and f != os.path.basename(__file__))
    proc = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                           "-m", "not gpu", *[os.path.join("tests", f) for f in tests]],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (proc.stdout + proc.stderr)[-4000:]
    assert proc.returncode == 0, tail
    assert "passed" in proc.stdout, tail
    for word in ("AddressSanitizer", "runtime error:"):
        assert word not in proc.stdout + proc.stderr, tail
