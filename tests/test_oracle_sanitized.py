"""The oracle is memory-clean: every pin runs against a copy of ep_oracle.c
built with AddressSanitizer and UndefinedBehaviorSanitizer (host code only),
in a child process with the ASan runtime preloaded; any out-of-bounds access,
use after free or undefined operation aborts the child."""
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

CHILD = r"""
import ctypes, sys
sys.path[:0] = [{root!r}, {here!r}]
import oracle, pins
orc = oracle.Oracle(oracle._bind(ctypes.CDLL({lib!r})))
for pin in pins.ALL_PINS:
    pin(orc)
print("all pins ran under the sanitizers:", len(pins.ALL_PINS))
"""


def _gcc_lib(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


@pytest.mark.skipif(_gcc_lib("libasan.so") is None, reason="gcc's AddressSanitizer runtime is not installed")
def test_oracle_pins_under_address_and_ub_sanitizers(tmp_path):
    lib = str(tmp_path / "libep_oracle_sanitized.so")
    src = os.path.join(ROOT, "oracle", "ep_oracle.c")
    subprocess.run(["gcc", "-std=c99", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                    "-I", os.path.dirname(src), "-o", lib, src, "-lm"], check=True)
    env = dict(os.environ)
    env["LD_PRELOAD"] = _gcc_lib("libasan.so")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    res = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, here=HERE, lib=lib)], env=env,
                         capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, f"sanitized oracle failed:\n{res.stdout[-2000:]}\n{res.stderr[-4000:]}"
    assert "all pins ran under the sanitizers" in res.stdout
