"""The per-wave element count of the LayerNorm kernels' one-exchange merge
(lr::wave_elems in row_reductions_amd/csrc/lr_map.hpp) against a brute-force
count built from the kernels' own chunk map, on the host
(tests/c/wave_elems.cpp): every team size, chunk count and phase, and row
lengths from 1 to the longest the team covers."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "c", "wave_elems.cpp")
CSRC = os.path.join(os.path.dirname(HERE), "row_reductions_amd", "csrc")


def test_wave_elems_matches_brute_force(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("g++ missing")
    exe = os.path.join(str(tmp_path), "wave_elems")
    r = subprocess.run(["g++", "-std=c++17", "-O2", "-Wall", "-Werror", "-I" + CSRC, SRC, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
    assert "wave counts checked" in r.stdout
