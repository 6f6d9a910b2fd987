"""The oracle's pins, run again against a build of conv_oracle.c with
AddressSanitizer and UndefinedBehaviorSanitizer (host code only, no GPU):
any out-of-bounds access, use of uninitialised memory through a bad index,
signed overflow or other undefined behaviour in the oracle fails the run.
The sanitizer runtimes are preloaded into a child Python process, which
runs tests/test_oracle_pins.py with the oracle routed to that build.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "conv_oracle.c")


def _runtime(name):
    try:
        p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                           check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.slow
def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not shutil.which("gcc") or not asan or not ubsan:
        pytest.skip("gcc with the AddressSanitizer and UBSan runtimes is not available")
    lib = str(tmp_path / "liboracle_san.so")
    # single-threaded (no OpenMP runtime inside the sanitizers)
    subprocess.run(["gcc", "-O1", "-g", "-std=c99", "-fPIC", "-shared",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-o", lib, SRC], check=True)
    env = dict(os.environ)
    env.update(GC_ORACLE_LIB=lib, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=99",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=98")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail
