"""Register budget of every gfx950 kernel, read from the compiler's own report (no GPU).

Each HIP source is compiled to gfx950 assembly with the library's flags and the
per-kernel ScratchSize is checked: a kernel that runs out of VGPRs spills to scratch
memory, which is slow and has given wrong decode results for a variant that spilled
hundreds of bytes per lane. No kernel may spill, except the wide GEMM with its K split
inside the workgroup, whose epilogue keeps one 16-byte accumulator tile in scratch while
the two halves are added (after the main loop).
"""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess

import pytest

from bit_weight_only_w4a16_amd import build as B

SOURCES = sorted(f for f in os.listdir(B.CSRC) if f.endswith(".hip"))
ALLOWED = {re.compile(r"gemm_wide_kernelILi\dELi2E"): 32}   # bytes per lane

pytestmark = pytest.mark.skipif(
    not any(os.path.exists(c) for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc") or "")),
    reason="hipcc not available")


def kernel_scratch(src, out_dir):
    out = os.path.join(out_dir, src + ".s")
    cmd = [B.hipcc(), *B.HIPCC_FLAGS, *B.FILE_FLAGS.get(src, []), "--cuda-device-only", "-S",
           os.path.join(B.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    result, name = {}, None
    for line in open(out):
        m = re.match(r"\s+\.amdhsa_kernel\s+(\S+)", line)
        if m:
            name = m.group(1)
        m = re.match(r"; ScratchSize: (\d+)", line)
        if m and name:
            result[name] = int(m.group(1))
            name = None
    return result


@pytest.fixture(scope="module")
def scratch(tmp_path_factory):
    d = str(tmp_path_factory.mktemp("asm"))
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        parts = list(ex.map(lambda s: (s, kernel_scratch(s, d)), SOURCES))
    return dict(parts)


def test_every_source_has_kernels(scratch):
    assert sum(len(v) for v in scratch.values()) > 100
    assert len(scratch["gemv.hip"]) > 0 and len(scratch["gemm_wide.hip"]) > 0


def test_no_kernel_spills(scratch):
    bad = []
    for src, kernels in scratch.items():
        for name, size in kernels.items():
            limit = next((v for pat, v in ALLOWED.items() if pat.search(name)), 0)
            if size > limit:
                bad.append((src, name, size))
    assert not bad, bad
