"""Build the gfx950 C-ABI library ``libawq_gfx950.so`` in-tree with hipcc.

    python -m bit_weight_only_w4a16_amd.build [--jobs N] [--verbose]

Every ``csrc/*.hip`` file is compiled for gfx950 only (no host fallback, no other GPU
target) and linked into one shared library next to this file.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libawq_gfx950.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # code object v5: loadable by the HIP runtime that PyTorch ships with
    "-mcode-object-version=5",
    # no packed-fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build the library")


# Matrix-core kernels keep their float32 accumulators in ordinary VGPRs: with AGPRs the
# register allocator copies accumulators between AGPRs inside the main loop. Kernels
# whose arguments are scalars (decode, narrow GEMM, split-K reduction, X' pre-scale)
# get them preloaded into SGPRs at wavefront launch (up to 16 user SGPRs: the kernarg
# pointer and 14 argument dwords).
FILE_FLAGS = {
    "gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-amdgpu-kernarg-preload-count=16"],
    "gemv.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-amdgpu-kernarg-preload-count=16"],
    "gemm_wide.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-amdgpu-kernarg-preload-count=16"],
    "chain.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "ceilings.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str, verbose: bool, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), *extra, "-c", src,
           "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def build(jobs: int = 8, verbose: bool = False, tuning_out: str | None = None) -> str:
    """Compile and link the library. With `tuning_out`, a separate copy is built at that
    path with -DAWQ_TUNING, which reads configuration overrides from the environment
    (for sweeps); the product library next to this file never does."""
    build_dir = BUILD if tuning_out is None else os.path.join(BUILD, "tuning")
    extra = () if tuning_out is None else ("-DAWQ_TUNING",)
    out = LIB if tuning_out is None else os.path.abspath(tuning_out)
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources found")
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, extra), srcs))
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if tuning_out is None:
        build_probe(verbose)
        build_abi_check(verbose)
    return out


PROBE_SRC = os.path.join(PKG, "probe", "ceilings.hip")
PROBE_LIB = os.path.join(PKG, "libawq_probe_gfx950.so")


def build_probe(verbose: bool = False) -> str:
    """The benchmark's ceiling probes (streaming read, empty launch) as their own library."""
    obj = _compile(PROBE_SRC, verbose)
    tmp = PROBE_LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", obj, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"probe link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


ABI_CHECK_SRC = os.path.join(ROOT, "tests", "c_abi", "abi_check.c")
ABI_CHECK_BIN = os.path.join(ROOT, "tests", "c_abi", "abi_check")


def abi_check_command(out: str) -> list:
    """gcc line for the plain-C user of the library (C99 against include/awq.h, linked
    with the built library and the HIP runtime)."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"),
            ABI_CHECK_SRC, "-o", out, "-L", PKG, "-lawq_gfx950",
            "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm",
            f"-Wl,-rpath,{PKG}", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}"]


def build_abi_check(verbose: bool = False) -> str:
    """Compile the C ABI check program (run by the GPU tests) next to its source."""
    cmd = abi_check_command(ABI_CHECK_BIN)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"C ABI check failed to build:\n{r.stdout}\n{r.stderr}")
    return ABI_CHECK_BIN


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=8)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--tuning", metavar="PATH",
                    help="build a copy that reads tuning overrides from the environment, at PATH")
    args = ap.parse_args()
    print(build(args.jobs, args.verbose, args.tuning))


if __name__ == "__main__":
    main()
