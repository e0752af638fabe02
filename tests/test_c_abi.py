"""The C ABI from plain C: tests/c_abi/abi_check.c is compiled as C99 against
include/awq.h and linked with the library (CPU); on a GPU the program runs one small
layer through channel scale, pack, repack, both dequantizers, GEMV and GEMM and checks
the results in float64 on the host, with no Python in between (GPU)."""
import os
import shutil
import subprocess
import tempfile

import pytest

from bit_weight_only_w4a16_amd import build as B


def _need_tools():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    if not os.path.exists(B.LIB):
        pytest.skip("library not built")


def test_c_abi_check_compiles_and_links():
    _need_tools()
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "abi_check")
        r = subprocess.run(B.abi_check_command(out), capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        assert "warning" not in r.stderr, r.stderr
        assert os.path.exists(out)


@pytest.mark.gpu
def test_c_abi_check_runs_on_the_gpu():
    _need_tools()
    exe = B.ABI_CHECK_BIN
    if not os.path.exists(exe):
        exe = B.build_abi_check()
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi_check: ok" in r.stdout
