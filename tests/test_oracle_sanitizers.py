"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer.

The oracle is built a second time with both sanitizers (every report fatal) and the pin
tests of every oracle function run against that build in a child process, with the
sanitizer runtimes preloaded.  Any out-of-bounds access, use after free, signed
overflow, misaligned access or other undefined behaviour in the oracle fails the run;
so would a pin that the instrumented build does not reproduce.  A second test plants a
one-past-the-end read in a copy of the source and checks that the same run reports it.
CPU only.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "qdelta_oracle.c")
PIN_FILES = ["tests/test_oracle_pins.py", "tests/test_oracle_bwd_pins.py", "tests/test_oracle_qed_pins.py",
             "tests/test_oracle_eda_pins.py"]


def _runtime(name):
    cc = os.environ.get("ORACLE_CC", "gcc")
    try:
        path = subprocess.run([cc, f"-print-file-name={name}"], capture_output=True, text=True,
                              check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _run_pins(tmp_path, src):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if shutil.which(os.environ.get("ORACLE_CC", "gcc")) is None or asan is None or ubsan is None:
        pytest.skip("no gcc with the sanitizer runtimes")
    sys.path.insert(0, ROOT)
    from oracle.build_oracle import build_sanitized
    lib = build_sanitized(str(tmp_path / "liboracle_qdelta_san.so"), src=src)
    env = dict(os.environ)
    env.update({
        "ORACLE_LIB": lib,
        "LD_PRELOAD": f"{asan} {ubsan}",
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "OMP_NUM_THREADS": "4",
    })
    # -s: no output capture, so a sanitizer report written to stderr as the process halts is kept
    cmd = [sys.executable, "-m", "pytest", "-q", "-s", "-x", "-p", "no:cacheprovider", "-m", "not gpu"] + PIN_FILES
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    return r.returncode, r.stdout + r.stderr


def test_oracle_pins_under_address_and_ub_sanitizers(tmp_path):
    rc, out = _run_pins(tmp_path, SRC)
    print(out[-2000:])
    assert "ERROR: AddressSanitizer" not in out
    assert "runtime error:" not in out
    assert rc == 0, out[-3000:]


def test_sanitized_run_reports_a_planted_overread(tmp_path):
    src = open(SRC).read()
    loop = "for (j = 0; j < n; ++j) acc += a[j] * b[j];"
    assert src.count(loop) == 1
    bad = tmp_path / "qdelta_oracle_overread.c"
    bad.write_text(src.replace(loop, "for (j = 0; j <= n; ++j) acc += a[j] * b[j];"))
    rc, out = _run_pins(tmp_path, str(bad))
    assert rc != 0
    assert "ERROR: AddressSanitizer" in out, out[-3000:]
