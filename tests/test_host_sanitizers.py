"""The CPU oracle and the input generator built with AddressSanitizer and
UndefinedBehaviorSanitizer, with the oracle's pins (and the generator's use in them) run
on that build in a child process: an out-of-bounds access, a use after free or undefined
behaviour in either C file ends the run with a sanitizer report."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    try:
        p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True, check=True)
    except (OSError, subprocess.CalledProcessError):
        return None
    path = p.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_and_generator_pins_under_asan_ubsan():
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("no ASan runtime for gcc on this host")
    env = dict(os.environ)
    env.update({
        "K3_HOST_SANITIZE": "1",
        "LD_PRELOAD": asan,
        # the interpreter itself is not instrumented: its own allocations are not leaks
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "OMP_NUM_THREADS": "4",
    })
    build = ("import sys; sys.path.insert(0, %r); import oracle, k3gen; "
             "assert oracle.SANITIZE and k3gen.SANITIZE; oracle.build(); k3gen.build()") % ROOT
    subprocess.run([sys.executable, "-c", build], env=env, check=True, cwd=ROOT)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=1200)
    tail = (r.stdout + r.stderr)[-4000:]
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail
    assert r.returncode == 0, tail
