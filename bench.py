#!/usr/bin/env python3
"""W4A16 decode / prefill benchmark on one MI355X.

Workload (one "step"): the seven linear layers of one Llama-7B decoder block at batch 1
-- q, k, v, o (4096 -> 4096), gate, up (4096 -> 11008), down (11008 -> 4096) -- each an
AWQ 4-bit asymmetric layer with group 128, fp16 activations ~N(0,1) with 1% outlier
channels x20, weights ~N(0, 0.02^2), channel scale from 32 calibration rows applied
online (inv_s_c). The seven GEMVs of a step are one HIP graph; steps rotate through
enough copies of the weights (> 1 GB) that every step reads its weights from HBM, not
from the 256 MB last-level cache.

value = algorithmic bytes of a step (codes + scales + zeros + x + y + inv_s_c) / time.
The same run times the prefill GEMM at M = 2048 on the Llama-3-8B shapes (4096 -> 6144,
4096 -> 28672, 14336 -> 4096) and reports it under "gemm", and times the CPU oracle on a
bounded sample of the decode workload under "cpu_baseline".
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

GROUP = 128
DECODE_LAYERS = [  # (name, N, K)
    ("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
    ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008),
]
PREFILL_LAYERS = [("qkv", 6144, 4096), ("gate_up", 28672, 4096), ("down", 4096, 14336)]
PREFILL_M = 2048
DOMINANT = "gate"  # 4096 -> 11008: the largest share of the step's kernel time


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotate-bytes", type=float, default=1.2e9,
                    help="total bytes of distinct weight copies the steps cycle through")
    ap.add_argument("--no-gemm", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--gemm-iters", type=int, default=20)
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the W4A16 layer runs on a single MI355X here; "
              "multi-GPU runs are not part of this benchmark", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from bit_weight_only_w4a16_amd import awq, synth
    from bit_weight_only_w4a16_amd import roofline as rl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ------------------------------------------------------------ decode layers
    log("quantizing the seven decode layers on the GPU")
    layers = []
    for j, (name, n, k) in enumerate(DECODE_LAYERS):
        d = synth.layer_inputs(1, 1, n, k, layer=j)
        w = torch.from_numpy(d["w"]).to(dev)
        s_c, inv = awq.awq_channel_scale(torch.from_numpy(d["x_cal"]).to(dev), 0.5)
        qw, sc, qz = awq.awq_pack(w, s_c)
        packed = awq.awq_repack(qw, sc, qz, n, k)
        del w, qw, sc, qz
        layers.append({"name": name, "n": n, "k": k, "x": torch.from_numpy(d["x"]).to(dev),
                       "inv": inv, "packed": packed,
                       "y": torch.empty((1, n), dtype=torch.float16, device=dev),
                       "bytes": rl.algorithmic_bytes(1, n, k, GROUP, rl.FMT_ASYM, with_inv=True)})
    step_bytes = sum(L["bytes"] for L in layers)
    step_weight_bytes = sum(L["packed"].numel() for L in layers)
    rot = max(2, math.ceil(args.rotate_bytes / step_weight_bytes))
    copies = [[L["packed"]] + [L["packed"].clone() for _ in range(rot - 1)] for L in layers]
    ws = awq.workspace(1, 11008, 11008, dev)
    for L in layers:  # grow once to the largest need, before any capture
        ws = awq.workspace(1, L["n"], L["k"], dev)

    def run_step(r, events=None):
        for j, L in enumerate(layers):
            if events is not None:
                events[j][0].record()
            awq.awq_gemv(L["x"], L["inv"], copies[j][r], L["n"], L["k"], GROUP, awq.FMT_ASYM,
                         y=L["y"], ws=ws)
            if events is not None:
                events[j][1].record()

    # warmup (eager) and graph capture: one graph per rotation copy, one for all copies
    for i in range(max(1, args.warmup)):
        run_step(i % rot)
    torch.cuda.synchronize()
    g_all = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_all):
        for r in range(rot):
            run_step(r)
    g_one = []
    for r in range(rot):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run_step(r)
        g_one.append(g)
    for _ in range(2):
        g_all.replay()
    torch.cuda.synchronize()

    # ------------------------------------------------------------ timed region
    log(f"timing {args.steps} steps ({rot} weight copies)")
    K = args.steps
    q, rem = divmod(K, rot)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(q):
        g_all.replay()
    for r in range(rem):
        g_one[r].replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    sec = t1 - t0
    value_gbs = step_bytes * K / sec / 1e9

    # ------------------------------------------- per-kernel durations (HIP events)
    # One graph per layer shape holding that layer's GEMV over all its weight copies,
    # replayed between two events on the capture stream: launches run back to back, and
    # the average per launch is the kernel time (checked against rocprofv3's trace).
    per_layer = {}
    for shape_layer in ("q", "gate", "down"):
        j = next(i for i, L in enumerate(layers) if L["name"] == shape_layer)
        L = layers[j]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for r in range(rot):
                awq.awq_gemv(L["x"], L["inv"], copies[j][r], L["n"], L["k"], GROUP,
                             awq.FMT_ASYM, y=L["y"], ws=ws)
        g.replay()
        torch.cuda.synchronize()
        reps = max(2, (8 * K) // (7 * rot))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * rot)
        per_layer[shape_layer] = {"shape": f"{L['k']}->{L['n']}", "us": round(us, 3),
                                  "GB/s": round(L["bytes"] / us / 1e3, 1), "launches": reps * rot}
        del g
    dom = next(L for L in layers if L["name"] == DOMINANT)
    dom_us = per_layer[DOMINANT]["us"]
    achieved = dom["bytes"] / dom_us / 1e3  # GB/s
    sum_kernel_us = 4 * per_layer["q"]["us"] + 2 * per_layer["gate"]["us"] + per_layer["down"]["us"]
    traffic = measured_traffic(dom["bytes"])

    # ------------------------------------------------------------ prefill GEMM
    gemm = None
    if not args.no_gemm:
        log("prefill GEMM M=2048")
        del copies, g_all, g_one
        torch.cuda.empty_cache()
        gl = []
        tot_flop = tot_us = 0.0
        for j, (name, n, k) in enumerate(PREFILL_LAYERS):
            d = synth.layer_inputs(3, PREFILL_M, n, k, layer=j)
            w = torch.from_numpy(d["w"]).to(dev)
            s_c, inv = awq.awq_channel_scale(torch.from_numpy(d["x_cal"]).to(dev), 0.5)
            qw, sc, qz = awq.awq_pack(w, s_c)
            packed = awq.awq_repack(qw, sc, qz, n, k)
            del w, qw, sc, qz
            x = torch.from_numpy(d["x"]).to(dev)
            y = torch.empty((PREFILL_M, n), dtype=torch.float16, device=dev)
            for _ in range(3):
                awq.awq_gemm(x, inv, packed, n, k, y=y)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(args.gemm_iters):
                awq.awq_gemm(x, inv, packed, n, k, y=y)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / args.gemm_iters
            fl = rl.flops(PREFILL_M, n, k)
            tot_flop += fl
            tot_us += us
            gl.append({"shape": f"{k}->{n}", "M": PREFILL_M, "us": round(us, 2),
                       "TFLOP/s": round(fl / us / 1e6, 1),
                       "frac": round(fl / us / 1e6 / rl.MFMA_F16_PEAK_TFLOPS, 4)})
            del packed, x, y
        agg = tot_flop / tot_us / 1e6
        gemm = {"workload": "llama3_8b_prefill_m2048", "metric": "TFLOP/s", "value": round(agg, 1),
                "roofline": {"bound": "mfma", "achieved": round(agg, 1),
                             "peak": round(rl.MFMA_F16_PEAK_TFLOPS, 1), "unit": "TFLOP/s",
                             "frac": round(agg / rl.MFMA_F16_PEAK_TFLOPS, 4)},
                "layers": gl}

    if args.copy_probe:
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    # ------------------------------------------------------------ CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        log("CPU oracle baseline")
        cpu = cpu_baseline(args.cpu_seconds)

    out = {
        "metric": "W4A16 GEMV HBM GB/s at M=1 (7B decoder layer, 7 GEMVs)",
        "value": round(value_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(sec / K * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 weights x fp16 activations, fp32 accumulate",
        "data": "synthetic (seeded N(0,1) activations with 1% x20 outlier channels, "
                "N(0,0.02^2) weights, AWQ RTN asym int4 g128)",
        "config": {"workload": "llama7b_decode_gemv_m1", "layers": "4x4096->4096, "
                   "2x4096->11008, 1x11008->4096", "M": 1, "group": GROUP, "format": "asym",
                   "step_bytes": step_bytes, "weight_rotation_copies": rot,
                   "submission": "one HIP graph per step"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1),
                     "peak": rl.HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / rl.HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": f"awq_gemv 4096->11008 M=1 ({dom_us:.3f} us/launch)"},
        "per_layer_kernel": per_layer,
        "kernel_sum_us_per_step": round(sum_kernel_us, 3),
        "kernel_only_GB/s": round(step_bytes / sum_kernel_us / 1e3, 1),
        "gemm": gemm,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_4096x11008_m1_traffic.txt")
GEMV_SOURCES = ("bit_weight_only_w4a16_amd/csrc/gemv.hip",
                "bit_weight_only_w4a16_amd/csrc/awq_internal.hpp")


def gemv_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in GEMV_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(algorithmic_bytes: int):
    """HBM bytes per launch of the dominant GEMV, as measured by rocprofv3 counters
    (FETCH_SIZE + WRITE_SIZE, each scaled by what it reads for a plain copy of known
    size) and recorded with the hash of the kernel source; None if the kernel source
    changed since, or if no measurement is recorded."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256_16") != gemv_source_hash():
        return None
    return int(float(kv["traffic_bytes_per_launch"]))


def cpu_baseline(seconds: float):
    """The CPU oracle (as it stands) on the dominant decode layer: dequantize + product."""
    import numpy as np

    import oracle
    from bit_weight_only_w4a16_amd import synth
    from bit_weight_only_w4a16_amd import roofline as rl

    from threadpoolctl import threadpool_limits

    n, k = 11008, 4096
    d = synth.layer_inputs(1, 1, n, k, layer=4)
    s, inv = oracle.channel_scale(d["x_cal"], 0.5)
    layer = oracle.quantize_layer(d["w"], s, GROUP, oracle.FMT_ASYM)
    reps, t = 0, 0.0
    with threadpool_limits(1):
        while t < seconds or reps < 1:
            t0 = time.perf_counter()
            w_d = oracle.dequant_packed(layer["qweight"], layer["scales"], layer["qzeros"],
                                        GROUP, oracle.FMT_ASYM)
            oracle.matmul_ref(d["x"], w_d, inv)
            t += time.perf_counter() - t0
            reps += 1
    byts = rl.algorithmic_bytes(1, n, k, GROUP, rl.FMT_ASYM, with_inv=True)
    return {"value": round(byts * reps / t / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"oracle dequant + float64 product of the 4096->11008 decode layer "
                      f"(M=1), {reps} repetitions in {t:.1f} s, BLAS limited to 1 thread",
            "ms_per_layer": round(t / reps * 1e3, 1)}


if __name__ == "__main__":
    main()
