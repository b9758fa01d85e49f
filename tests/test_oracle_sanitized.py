"""The oracle's pins under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

tb_oracle.c is rebuilt with gcc's ASan + UBSan (host code; no GPU code is
involved) and every pin runs against that copy in a child Python process with
the ASan runtime preloaded, since the interpreter itself is not instrumented.
Any out-of-bounds access, use of freed memory, signed overflow, bad shift or
other undefined behaviour in the oracle aborts the child and fails the test.
"""

from __future__ import annotations

import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_FLAGS = ["-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-tree-vectorize", "-fPIC",
             "-shared", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all"]

CHILD = r"""
import sys
sys.path.insert(0, sys.argv[1])
import oracle
from tests import pins
o = oracle.Oracle(sys.argv[2])
for pin in pins.ALL_PINS:
    pin(o)
    print("pin ok:", pin.__name__, flush=True)
print("ALL PINS OK", flush=True)
"""


def _asan_runtime() -> str | None:
    try:
        path = subprocess.run(["gcc", "-print-file-name=libasan.so"], check=True,
                              capture_output=True, text=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_pins_under_asan_ubsan(tmp_path):
    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("gcc's ASan runtime is not installed")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", *SAN_FLAGS, oracle.SRC, "-o", lib, "-lm"], check=True)
    env = dict(os.environ)
    env["LD_PRELOAD"] = runtime
    # the interpreter's own allocations are not ours to judge; stop at the first report
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    proc = subprocess.run([sys.executable, "-c", CHILD, ROOT, lib], env=env,
                          capture_output=True, text=True, timeout=600)
    out = proc.stdout + proc.stderr
    assert proc.returncode == 0 and "ALL PINS OK" in proc.stdout, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
