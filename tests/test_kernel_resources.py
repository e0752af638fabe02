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


def compile_asm(src, out_dir):
    out = os.path.join(out_dir, src + ".s")
    cmd = [B.hipcc(), *B.HIPCC_FLAGS, *B.FILE_FLAGS.get(src, []), "--cuda-device-only", "-S",
           os.path.join(B.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out


def kernel_scratch(out):
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


def _vgprs(tok):
    tok = tok.strip().rstrip(",")
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def asm_to_mfma_hazards(out, need=2):
    """Matrix instructions that read a VGPR written by an inline-asm instruction fewer
    than `need` wait states earlier, in program order (s_nop k counts k + 1). The
    compiler inserts the wait states gfx950 requires between an ALU write and an MFMA
    read for the instructions it generates, but not after inline asm."""
    found, kernel, hist, in_asm = [], None, [], False
    for line in open(out):
        m = re.match(r"^(_Z\S*):", line)
        if m:
            kernel, hist = m.group(1), []
            continue
        s = line.strip()
        if kernel is None or not s:
            continue
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if s.startswith(";") or s.startswith(".") or s.endswith(":"):
            continue
        parts = s.split(None, 1)
        op, args = parts[0], (parts[1].split(",") if len(parts) > 1 else [])
        if op.startswith("v_mfma"):
            srcs = set().union(*[_vgprs(a) for a in args[1:]]) if len(args) > 1 else set()
            dist = 0
            for kind, regs, w in reversed(hist):
                if kind and regs & srcs:
                    if dist < need:
                        found.append((kernel, s, dist))
                    break
                dist += w
                if dist >= need:
                    break
        ws = int(parts[1]) + 1 if op == "s_nop" else 1
        hist = (hist + [(in_asm, _vgprs(args[0]) if (in_asm and args) else set(), ws)])[-16:]
    return found


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    d = str(tmp_path_factory.mktemp("asm"))
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        return dict(ex.map(lambda s: (s, compile_asm(s, d)), SOURCES))


@pytest.fixture(scope="module")
def scratch(asm):
    return {src: kernel_scratch(out) for src, out in asm.items()}


def test_no_mfma_reads_inline_asm_result_too_early(asm):
    """No matrix instruction reads an inline-asm result within two wait states (a decode
    variant that did returned wrong sums: the MFMA read the register's old contents)."""
    bad = [h for out in asm.values() for h in asm_to_mfma_hazards(out)]
    assert not bad, bad[:5]


def test_hazard_check_sees_an_unguarded_write(tmp_path):
    """The check itself: an asm write followed by an MFMA one instruction later is found,
    and the same with s_nop 1 in between is not."""
    body = ["_Zk:", ";;#ASMSTART", "v_and_or_b32 v5, v1, s2, v3", ";;#ASMEND",
            "v_lshrrev_b32_e32 v9, 8, v1", "v_mfma_f32_16x16x32_f16 v[10:13], v[20:23], v[4:7], 0"]
    p = tmp_path / "k.s"
    p.write_text("\n".join(body) + "\n")
    assert len(asm_to_mfma_hazards(str(p))) == 1
    body.insert(4, "s_nop 1")
    p.write_text("\n".join(body) + "\n")
    assert asm_to_mfma_hazards(str(p)) == []


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
