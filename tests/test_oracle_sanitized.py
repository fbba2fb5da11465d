"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer.

ctc_oracle.c is compiled with -fsanitize=address,undefined (gcc, every finding
aborts), and the pins of tests/test_oracle_pins.py run against that copy in a
child process with the sanitizer runtime preloaded: an out-of-bounds access,
a use after free, a signed overflow or any other undefined behaviour on the
pins' inputs ends the run with a report.  Leak detection is off (the Python
interpreter keeps allocations until exit).
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _run_pins(lib):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    env = dict(os.environ)
    env.update(LD_PRELOAD=asan + ":" + ubsan, PCX_ORACLE_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
                        "-p", "no:xdist", os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=850)
    return r.returncode, r.stdout + r.stderr


@pytest.mark.timeout(900)
def test_pins_pass_under_sanitizers(tmp_path):
    rc, out = _run_pins(oracle.build_sanitized(str(tmp_path / "liboracle_san.so")))
    assert rc == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out


@pytest.mark.timeout(300)
def test_sanitizer_reports_a_planted_overflow(tmp_path):
    """The check can fail: a copy of the oracle whose occupancy row is one
    element short (a heap overflow on the last class) is stopped by
    AddressSanitizer on the first pin that asks for occupancies."""
    orig = "double* gam_row = (double*)malloc(sizeof(double) * (size_t)V);"
    src = oracle.source_text()
    assert src.count(orig) == 1
    lib = oracle.build_sanitized(str(tmp_path / "liboracle_bad.so"),
                                 src.replace(orig, orig.replace("(size_t)V", "(size_t)(V - 1)")))
    rc, out = _run_pins(lib)
    assert rc != 0
    assert "AddressSanitizer" in out and "heap-buffer-overflow" in out, out[-4000:]
