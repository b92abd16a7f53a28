"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer: a copy of
the oracle built with both (host code, g++) must pass every pin suite without
a report -- an out-of-bounds index or a signed overflow in the oracle would
otherwise stay invisible to pins that happen to read the right memory.
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

from oracle import build as obuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = ["test_oracle_pins.py", "test_oracle_combine.py", "test_oracle_placement.py",
             "test_oracle_quality.py", "test_oracle_predict.py", "test_oracle_slots.py"]


def runtime(name: str) -> str | None:
    r = subprocess.run(["g++", "-print-file-name=" + name], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_pins_pass_on_a_sanitized_oracle(tmp_path):
    asan, ubsan = runtime("libasan.so"), runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("no g++ sanitizer runtimes")
    lib = obuild.build(sanitize=True, out=str(tmp_path / "libmoe_oracle_sanitized.so"))
    env = dict(os.environ)
    env["MOE_ORACLE_LIB"] = lib
    # the sanitizer runtimes go after whatever the environment already preloads
    env["LD_PRELOAD"] = " ".join(p for p in [env.get("LD_PRELOAD", ""), asan, ubsan] if p)
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0:abort_on_error=0:exitcode=86"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1:exitcode=87"
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider"]
    cmd += [os.path.join(ROOT, "tests", f) for f in PIN_FILES]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
