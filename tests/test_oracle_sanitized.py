"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

osdn_oracle.c does its own pointer and index arithmetic over caller-supplied
shapes, head lists and optional arrays, and runs its heads on several threads.
This test builds it with -fsanitize=address,undefined (gcc, CPU only) and runs
the oracle's pin tests against that build in a child process, with every
sanitizer report fatal, plus a few calls over the argument edge cases (empty
sequences, head subsets, every optional output, more threads than heads).
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "osdn_oracle.c")

PINS = ["tests/test_oracle_pins.py", "tests/test_oracle_golden.py", "tests/test_oracle_gated.py",
        "tests/test_oracle_kda.py", "tests/test_oracle_inputs.py"]

EDGE_CASES = r'''
import numpy as np
from oracle import oracle
g = np.random.default_rng(3)
for B, H, T, dk, dv in ((1, 1, 0, 4, 3), (2, 3, 1, 2, 5), (2, 2, 37, 8, 4)):
    k = g.standard_normal((B, H, T, dk))
    args = dict(q=g.standard_normal((B, H, T, dk)), k=k, v=g.standard_normal((B, H, T, dv)),
                beta=g.random((B, H, T)), r=g.random((B, H, T)),
                d0=g.random((B, H, dk)), S0=g.standard_normal((B, H, dv, dk)))
    want = ("o", "S", "d", "k_tilde", "d_all", "rho")
    for mode in ("osdn", "deltanet", "given"):
        kg = k[::-1].copy() if mode == "given" else None
        oracle.forward(**args, eta=0.3, mode=mode, k_given=kg, want=want, threads=7)
        oracle.forward(**args, eta=0.3, mode=mode, k_given=kg, want=want,
                       heads=[B * H - 1, 0], threads=3)
    oracle.forward(**args, eta=0.3, alpha=g.random((B, H, T)), want=want, threads=2)
    oracle.forward(**args, eta=0.3, alpha=g.random((B, H, T, dk)), want=want,
                   heads=[], threads=1)
    oracle.forward(**args, eta=0.3, alpha=g.random((B, H, T, dk)), want=want, threads=5)
print("edge cases done")
'''


def _runtime(name):
    p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("gcc") is None or _runtime("libasan.so") is None,
                    reason="gcc with the AddressSanitizer runtime is needed")
def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    lib = str(tmp_path / "liboracle_asan.so")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
           "-fno-fast-math", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", SRC, "-o", lib, "-lm"]
    subprocess.run(cmd, check=True)
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": _runtime("libasan.so"),
        "OSDN_ORACLE_LIB": lib,
        # the interpreter itself is not instrumented: its allocations are not
        # this test's concern
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "PYTHONPATH": ROOT,
    })
    pins = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                           "-m", "not gpu"] + PINS, cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=900)
    out = pins.stdout + pins.stderr
    assert pins.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    edge = subprocess.run([sys.executable, "-c", EDGE_CASES], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=300)
    out = edge.stdout + edge.stderr
    assert edge.returncode == 0 and "edge cases done" in edge.stdout, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
