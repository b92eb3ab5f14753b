"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

The oracle's C source is compiled with -fsanitize=address,undefined (every
report fatal) and the whole pin set runs against it in a child process that
preloads the ASan runtime: an out-of-bounds access, a use after free, a
signed overflow or a misaligned access anywhere on those paths aborts the
child and fails the test.  Leak checking is off (the Python interpreter
itself holds memory until exit).  CPU only.
"""
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _runtime(name):
    try:
        path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                              check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.timeout(900)
def test_pins_pass_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = oracle.build_sanitized(str(tmp_path / "liboracle_san.so"))
    env = dict(os.environ, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, os.path.join(HERE, "sanitized_pins_runner.py"), lib],
                       capture_output=True, text=True, env=env, timeout=880)
    tail = (r.stdout[-3000:] + "\n" + r.stderr[-3000:]).strip()
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
    assert "pins pass" in r.stdout, tail
