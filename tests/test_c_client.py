"""The C ABI from plain C: tests/c/abi_client.c includes only include/lr.h and
the HIP runtime header, is compiled by gcc as C11 and links liblr.so.  On the
CPU the client must compile and link; on the GPU it must run its checks
(softmax rows sum to one under every policy, RMSNorm of constant rows,
cross-entropy of uniform rows with an out-of-range label, a LayerNorm split
across workgroups through lr_run_f32 and a workspace, and argument errors
returned before any device work)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "row_reductions_amd")
SRC = os.path.join(ROOT, "tests", "c", "abi_client.c")


def build_client(tmp_path):
    if shutil.which("gcc") is None or not os.path.exists(os.path.join(LIB_DIR, "liblr.so")):
        pytest.skip("gcc or liblr.so missing")
    out = os.path.join(str(tmp_path), "abi_client")
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-O2", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROOT, "include"), "-I/opt/rocm/include", SRC, "-o", out,
           "-L" + LIB_DIR, "-llr", "-L/opt/rocm/lib", "-lamdhip64", "-lm",
           "-Wl,-rpath," + LIB_DIR, "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out


def test_c_client_compiles_and_links(tmp_path):
    exe = build_client(tmp_path)
    assert os.access(exe, os.X_OK)


@pytest.mark.gpu
def test_c_client_runs(tmp_path):
    exe = build_client(tmp_path)
    print("\n[gpu] C ABI client", flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi_client ok" in r.stdout
