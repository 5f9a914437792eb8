"""The three-instruction quotient the ordered softmax kernels write (e / s
from a correctly rounded reciprocal of the row sum and two fused
multiply-adds, P. Markstein 1990), checked on the host against IEEE division:
equal on every structured and random pair with e == 0 or e >= 2^-96 and
s >= 1, the guard that sends a wave to the division marks exactly
(0, 2^-96), and below that bound the short form does differ, so the guard
is needed (tests/c/rowsum_division.c)."""
import os
import shutil
import subprocess

import pytest

SRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "rowsum_division.c")


def test_rowsum_division_matches_ieee_division(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc missing")
    exe = os.path.join(str(tmp_path), "rowsum_division")
    r = subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Werror",
                        SRC, "-o", exe, "-lm"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe, "20000000", "7"], capture_output=True, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
    assert " 0 differ from the division" in r.stdout
