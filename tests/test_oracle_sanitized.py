"""The C oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(host code, gcc), with every pin run against it in a child process: an
out-of-bounds access, a use after free or undefined arithmetic aborts the
child.  CPU only."""
import json
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g"]


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_pins_under_address_and_ub_sanitizers(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc's sanitizer runtimes are not installed")
    lib = oracle.build(oracle.SRC, str(tmp_path / "libgs_oracle_san.so"), extra=SAN)
    env = dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([sys.executable, "-m", "tests.run_pins", lib], cwd=ROOT, env=env,
                         capture_output=True, text=True, timeout=900)
    assert run.returncode == 0, run.stderr[-4000:]
    assert "runtime error" not in run.stderr, run.stderr[-4000:]
    assert json.loads(run.stdout.strip().splitlines()[-1]) == []
