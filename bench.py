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

Also reported (same JSON line):
  per_layer_kernel  each decode shape alone, back-to-back launches in a graph;
  fused_step        the same seven products as four launches (q|k|v as one 4096 -> 12288
                    layer, gate|up as one 4096 -> 22016 layer), and the linear-layer
                    token-rate bound of a 32-block 7B model at both step times;
  batched           M = 8, 16, 32, 64 rows at 4096 -> 11008 (the GEMV -> matrix-core
                    crossover);
  llama70b_m1       8192 -> 28672 and 28672 -> 8192 at M = 1, asymmetric and symmetric;
  group_sizes       the 4096 -> 11008 decode layer with groups of 32, 64, 128 and 4096;
  scale_search      the AWQ exponent grid search (21 candidates) on one 4096 -> 11008 layer;
  gemm              the prefill GEMM at M = 2048 on the Llama-3-8B shapes (4096 -> 6144,
                    4096 -> 28672, 14336 -> 4096);
  unfused           awq_dequant to binary16 + the library fp16 GEMM (hipBLASLt through
                    torch.matmul) at the same shapes: the unfused baseline;
  ceilings          a read-only kernel streaming each decode shape's weight bytes with the
                    decode kernel's access pattern, and the cost of an empty launch;
  cpu_baseline      the CPU oracle on bounded samples of the decode and batched workloads.
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
# the block's dependencies, in DECODE_LAYERS order (q, k, v, o, gate, up, down)
CHAIN_SRCS = [-1, -1, -1, 2, 3, 3, 5]
FUSED_LAYERS = [("qkv", 12288, 4096), ("o", 4096, 4096), ("gate_up", 22016, 4096),
                ("down", 4096, 11008)]
PREFILL_LAYERS = [("qkv", 6144, 4096), ("gate_up", 28672, 4096), ("down", 4096, 14336)]
PREFILL_M = 2048
BATCHED_M = (8, 16, 32, 64)
LAYERS_70B = [("up", 28672, 8192), ("down", 8192, 28672)]
M_70B = (16, 256, 4096)
N_BLOCKS_7B = 32
GEMV_MAX_M = 4  # above this the split-K matrix-core GEMM is faster (batched rows)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotate-bytes", type=float, default=1.2e9,
                    help="total bytes of distinct weight copies the launches cycle through")
    ap.add_argument("--no-gemm", action="store_true", help="skip prefill GEMM and unfused")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip fused step, batched decode and 70B layers")
    ap.add_argument("--only-extra", default="",
                    help="comma-separated extra sections to run (fused_step, batched, llama70b, "
                         "group_sizes, scale_search); default all")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=16.0)
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

    import torch

    from bit_weight_only_w4a16_amd import awq, synth
    from bit_weight_only_w4a16_amd import roofline as rl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def make_layer(config, n, k, m=1, layer=0, fmt=awq.FMT_ASYM):
        """Quantize a synthetic layer on the GPU (channel scale, pack, repack)."""
        d = synth.layer_inputs(config, m, n, k, layer=layer)
        w = torch.from_numpy(d["w"]).to(dev)
        s_c, inv = awq.awq_channel_scale(torch.from_numpy(d["x_cal"]).to(dev), 0.5)
        qw, sc, qz = awq.awq_pack(w, s_c, GROUP, fmt)
        packed = awq.awq_repack(qw, sc, qz, n, k, GROUP, fmt)
        del w, qw, sc, qz
        return {"n": n, "k": k, "m": m, "fmt": fmt, "inv": inv, "packed": packed,
                "x": torch.from_numpy(d["x"]).to(dev),
                "y": torch.empty((m, n), dtype=torch.float16, device=dev)}

    def rotation(weight_bytes):
        return max(2, math.ceil(args.rotate_bytes / weight_bytes))

    def graph_us(launches, reps, trials=3, warm_ms=20.0):
        """Per-launch microseconds of a graph of back-to-back launches, replayed `reps`
        times between two events on the capture stream; median of `trials`. The graph
        first runs for about `warm_ms` of GPU time, so that the clocks have settled at
        their loaded level (the first milliseconds after an idle host phase run slower)."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for f in launches:
                f()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        for _ in range(min(2000, int(warm_ms * 1e-3 / max(e0.elapsed_time(e1) * 1e-3, 1e-6)))):
            g.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(trials):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3 / (reps * len(launches)))
        del g
        return sorted(ts)[len(ts) // 2]

    def product(fn, L, packed, ws):
        return lambda: fn(L["x"], L["inv"], packed, L["n"], L["k"], GROUP, L["fmt"],
                          y=L["y"], ws=ws)

    # ------------------------------------------------------------ decode layers
    log("quantizing the seven decode layers on the GPU")
    layers = []
    for j, (name, n, k) in enumerate(DECODE_LAYERS):
        L = make_layer(1, n, k, layer=j)
        L["name"] = name
        L["bytes"] = rl.algorithmic_bytes(1, n, k, GROUP, rl.FMT_ASYM, with_inv=True)
        layers.append(L)
    step_bytes = sum(L["bytes"] for L in layers)
    step_weight_bytes = sum(L["packed"].numel() for L in layers)
    rot = rotation(step_weight_bytes)
    copies = [[L["packed"]] + [L["packed"].clone() for _ in range(rot - 1)] for L in layers]
    ws = None
    for L in layers:  # grow once to the largest need, before any capture
        ws = awq.workspace(1, L["n"], L["k"], dev)

    def run_step(r):
        for j, L in enumerate(layers):
            awq.awq_gemv(L["x"], L["inv"], copies[j][r], L["n"], L["k"], GROUP, awq.FMT_ASYM,
                         y=L["y"], ws=ws)

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
    # per-step spread (outside the timed region), in the headline's submission mode: the
    # graph of `rot` steps replayed between two events, the time divided by `rot`
    n_spread = max(10, min(50, K // rot))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_spread)]
    for ea, eb in evs:
        ea.record()
        g_all.replay()
        eb.record()
    torch.cuda.synchronize()
    per_step = sorted(ea.elapsed_time(eb) * 1e3 / rot for ea, eb in evs)
    step_spread = {"median": round(per_step[n_spread // 2], 3),
                   "p10": round(per_step[n_spread // 10], 3),
                   "p90": round(per_step[(9 * n_spread) // 10], 3),
                   "samples": n_spread, "steps_per_sample": rot,
                   "submission": "one graph of the rotation's steps, as the headline"}
    del g_all, g_one, evs

    # ------------------------------------------- per-kernel durations (HIP events)
    # One graph per layer shape holding that layer's GEMV over its own set of weight
    # copies (more than `rotate_bytes` of them, like the step, so that no launch finds its
    # weights in the 256 MB Infinity Cache), replayed between two events on the capture
    # stream: launches run back to back, and the average per launch is the kernel time
    # (checked against rocprofv3's trace).
    del copies
    torch.cuda.empty_cache()
    per_layer = {}
    for shape_layer in ("q", "gate", "down"):
        j = next(i for i, L in enumerate(layers) if L["name"] == shape_layer)
        L = layers[j]
        lrot = rotation(L["packed"].numel())
        lcp = [L["packed"]] + [L["packed"].clone() for _ in range(lrot - 1)]
        reps = max(2, (8 * K) // (7 * lrot))
        us = graph_us([product(awq.awq_gemv, L, lcp[r], ws) for r in range(lrot)], reps)
        per_layer[shape_layer] = {"shape": f"{L['k']}->{L['n']}", "us": round(us, 3),
                                  "GB/s": round(L["bytes"] / us / 1e3, 1),
                                  "launches": 3 * reps * lrot, "weight_copies": lrot}
        del lcp
        torch.cuda.empty_cache()
    # measured ceilings: a read-only kernel streaming each decode shape's packed weight
    # bytes with the decode kernel's access pattern, and one empty launch
    ceil = None
    if not args.no_ceilings:
        log("ceilings: streaming read and empty launch")
        sizes = {name: layers[next(i for i, L in enumerate(layers) if L["name"] == name)]["packed"].numel()
                 for name in ("q", "gate", "down")}
        ceil = ceilings(dev, sizes, graph_us, rotation)
        for name in ("q", "gate", "down"):
            c = ceil["stream_read"][name]
            c["decode_over_stream"] = round(c["best_us"] / per_layer[name]["us"], 3)

    # The dominant kernel is the decode kernel itself: its 7 launches are the whole step
    # (the 4096 -> 4096 launches alone are 45 % of it). Roofline over one step: the
    # algorithmic bytes of the 7 launches / their summed kernel time, i.e. bytes per
    # launch / average launch duration.
    sum_kernel_us = 4 * per_layer["q"]["us"] + 2 * per_layer["gate"]["us"] + per_layer["down"]["us"]
    achieved = step_bytes / sum_kernel_us / 1e3  # GB/s
    traffic = measured_traffic()
    del layers
    torch.cuda.empty_cache()

    extra = {}
    only = {t for t in args.only_extra.split(",") if t}

    def want(section):
        return not args.no_extra and (not only or section in only)

    if want("fused_step"):
        # -------------------------------------- fused q|k|v and gate|up: four launches
        log("fused decode step (4 launches)")
        fl = [make_layer(1, n, k, layer=20 + j) for j, (_, n, k) in enumerate(FUSED_LAYERS)]
        f_bytes = sum(rl.algorithmic_bytes(1, L["n"], L["k"], GROUP, rl.FMT_ASYM, True)
                      for L in fl)
        f_rot = rotation(sum(L["packed"].numel() for L in fl))
        f_cp = [[L["packed"]] + [L["packed"].clone() for _ in range(f_rot - 1)] for L in fl]
        for L in fl:
            ws = awq.workspace(1, L["n"], L["k"], dev)
        launches = [product(awq.awq_gemv, L, f_cp[j][r], ws)
                    for r in range(f_rot) for j, L in enumerate(fl)]
        f_us = graph_us(launches, max(2, K // f_rot)) * len(fl)  # per step
        step_us = sec / K * 1e6
        extra["fused_step"] = {
            "launches": [f"{L['k']}->{L['n']}" for L in fl], "us_per_step": round(f_us, 3),
            "GB/s": round(f_bytes / f_us / 1e3, 1),
            "linear_tok_per_s_7b": {"7_launches": round(1e6 / (N_BLOCKS_7B * step_us), 1),
                                    "4_launches": round(1e6 / (N_BLOCKS_7B * f_us), 1),
                                    "bound_at_8TB/s": round(rl.max_tokens_per_s(
                                        rl.HBM_PEAK_GBS, N_BLOCKS_7B * step_bytes / 1e9), 1)}}
        del f_cp, fl, launches
        torch.cuda.empty_cache()

    if want("chain_step"):
        # ------------------------- the decoder block as one awq_gemv_chain launch (NEXT-2)
        # the seven products with the block's dependencies (q, k, v read x; o reads v;
        # gate and up read o; down reads up), one launch per step over rotating weights;
        # beside it the same launch with every layer reading x (no waits inside)
        log("decoder block as one launch (awq_gemv_chain)")
        cl = [make_layer(1, n, k, layer=30 + j) for j, (_, n, k) in enumerate(DECODE_LAYERS)]
        c_bytes = sum(rl.algorithmic_bytes(1, L["n"], L["k"], GROUP, rl.FMT_ASYM, True) for L in cl)
        c_rot = rotation(sum(L["packed"].numel() for L in cl))
        c_cp = [[L["packed"]] + [L["packed"].clone() for _ in range(c_rot - 1)] for L in cl]
        state = awq.chain_state(dev)

        def chain_specs(r, srcs):
            return [{"packed": c_cp[j][r], "n": L["n"], "k": L["k"], "inv_s_c": L["inv"],
                     "y": L["y"], "src": srcs[j], **({"x": L["x"]} if srcs[j] < 0 else {})}
                    for j, L in enumerate(cl)]

        res = {}
        for tag, srcs in (("block", CHAIN_SRCS), ("independent", [-1] * len(cl))):
            specs = [chain_specs(r, srcs) for r in range(c_rot)]
            us = graph_us([(lambda sp=sp: awq.awq_gemv_chain(sp, state)) for sp in specs],
                          max(2, K // c_rot))
            res[tag] = {"us_per_step": round(us, 3), "GB/s": round(c_bytes / us / 1e3, 1)}
        torch.cuda.synchronize()
        errors = awq.chain_errors(state)
        extra["chain_step"] = {
            "entry": "awq_gemv_chain", "launches_per_step": 1,
            "dependencies": "q, k, v <- x; o <- v; gate, up <- o; down <- up",
            **res, "waits_timed_out": errors,
            "linear_tok_per_s_7b": round(1e6 / (N_BLOCKS_7B * res["block"]["us_per_step"]), 1)}
        del c_cp, cl, state
        torch.cuda.empty_cache()

    if want("batched"):
        # -------------------------------------- batched decode M = 8 .. 64, 4096 -> 11008
        log("batched decode")
        bl = make_layer(2, 11008, 4096, m=max(BATCHED_M))
        b_rot = rotation(bl["packed"].numel())
        b_cp = [bl["packed"]] + [bl["packed"].clone() for _ in range(b_rot - 1)]
        xall = bl["x"]
        batched = []
        for m in BATCHED_M:
            L = dict(bl, m=m, x=xall[:m].contiguous(),
                     y=torch.empty((m, bl["n"]), dtype=torch.float16, device=dev))
            ws = awq.workspace(m, L["n"], L["k"], dev)
            fn, name = (awq.awq_gemv, "awq_gemv") if m <= GEMV_MAX_M else (awq.awq_gemm, "awq_gemm")
            us = graph_us([product(fn, L, b_cp[r], ws) for r in range(b_rot)], 10)
            byts = rl.algorithmic_bytes(m, L["n"], L["k"], GROUP, rl.FMT_ASYM, True)
            batched.append({"M": m, "entry": name, "us": round(us, 3),
                            "GB/s": round(byts / us / 1e3, 1),
                            "TFLOP/s": round(rl.flops(m, L["n"], L["k"]) / us / 1e6, 2)})
        extra["batched"] = {"shape": "4096->11008", "rows": batched}
        del b_cp, bl, xall
        torch.cuda.empty_cache()

    if want("llama70b"):
        # -------------------------------------- 70B layers, M = 1, 16, 256, 4096
        log("70B layers")
        rows70, rows70b = [], []
        for fmt, fname in ((awq.FMT_ASYM, "asym"), (awq.FMT_SYM8, "sym")):
            for j, (name, n, k) in enumerate(LAYERS_70B):
                L = make_layer(4, n, k, m=max(M_70B), layer=j, fmt=fmt)
                r70 = rotation(L["packed"].numel())
                cp = [L["packed"]] + [L["packed"].clone() for _ in range(r70 - 1)]
                wbytes = rl.weight_bytes(n, k, GROUP, fmt)
                for m in (1,) + M_70B:
                    Lm = dict(L, m=m, x=L["x"][:m].contiguous(),
                              y=torch.empty((m, n), dtype=torch.float16, device=dev))
                    ws = awq.workspace(m, n, k, dev)
                    fn = awq.awq_gemv if m <= GEMV_MAX_M else awq.awq_gemm
                    nrot = r70 if m <= 64 else 2  # weights from HBM where bandwidth-bound
                    us = graph_us([product(fn, Lm, cp[r % nrot], ws) for r in range(max(nrot, 2))],
                                  5 if m < 4096 else 2, warm_ms=100.0 if m >= 256 else 20.0)
                    byts = rl.algorithmic_bytes(m, n, k, GROUP, fmt, True)
                    row = {"layer": name, "shape": f"{k}->{n}", "format": fname, "M": m,
                           "us": round(us, 3), "GB/s": round(byts / us / 1e3, 1),
                           "TFLOP/s": round(rl.flops(m, n, k) / us / 1e6, 2),
                           "weight_bytes_per_row": round(wbytes / m)}
                    if m <= 64:
                        row["bound"], row["frac"] = "hbm", round(byts / us / 1e3 / rl.HBM_PEAK_GBS, 4)
                    else:
                        row["bound"] = "mfma"
                        row["frac"] = round(rl.flops(m, n, k) / us / 1e6 / rl.MFMA_F16_PEAK_TFLOPS, 4)
                    (rows70 if m == 1 else rows70b).append(row)
                    del Lm
                del cp, L
                torch.cuda.empty_cache()
        extra["llama70b_m1"] = rows70
        extra["llama70b_batched"] = rows70b

    if want("group_sizes"):
        # -------------------------------------- group sizes (NEXT-4): 4096 -> 11008, M = 1
        log("group sizes")
        gs_rows = []
        for gsz in (32, 64, 128, 4096):
            d = synth.layer_inputs(1, 1, 11008, 4096, layer=4)
            w = torch.from_numpy(d["w"]).to(dev)
            s_c, inv = awq.awq_channel_scale(torch.from_numpy(d["x_cal"]).to(dev), 0.5)
            qw, sc, qz = awq.awq_pack(w, s_c, gsz, awq.FMT_ASYM)
            pk = awq.awq_repack(qw, sc, qz, 11008, 4096, gsz, awq.FMT_ASYM)
            del w, qw, sc, qz
            L = {"n": 11008, "k": 4096, "fmt": awq.FMT_ASYM, "inv": inv,
                 "x": torch.from_numpy(d["x"]).to(dev),
                 "y": torch.empty((1, 11008), dtype=torch.float16, device=dev)}
            rg = rotation(pk.numel())
            cp = [pk] + [pk.clone() for _ in range(rg - 1)]
            fn = lambda r, cp=cp, L=L, gsz=gsz: awq.awq_gemv(L["x"], L["inv"], cp[r], 11008, 4096,
                                                          gsz, awq.FMT_ASYM, y=L["y"])
            us = graph_us([lambda r=r: fn(r) for r in range(rg)], 10)
            byts = rl.algorithmic_bytes(1, 11008, 4096, gsz, rl.FMT_ASYM, True)
            gs_rows.append({"group": gsz, "us": round(us, 3), "GB/s": round(byts / us / 1e3, 1),
                            "algorithmic_bytes": byts})
            del cp, pk
            torch.cuda.empty_cache()
        extra["group_sizes"] = {"shape": "4096->11008", "M": 1, "rows": gs_rows}

    if want("scale_search"):
        # -------------------------------------- AWQ exponent search (NEXT-1), one 7B layer
        log("AWQ scale search")
        d = synth.layer_inputs(1, 1, 11008, 4096, layer=4)
        w = torch.from_numpy(d["w"]).to(dev)
        xc = torch.from_numpy(d["x_cal"]).to(dev)
        sws = torch.empty(awq.awq_scale_search_workspace_bytes(xc.shape[0], 11008, 4096),
                          dtype=torch.uint8, device=dev)
        awq.awq_scale_search(w, xc, GROUP, awq.FMT_ASYM, 20, ws=sws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        best, losses = awq.awq_scale_search(w, xc, GROUP, awq.FMT_ASYM, 20, ws=sws)
        e1.record()
        torch.cuda.synchronize()
        lo = losses.cpu().tolist()
        extra["scale_search"] = {"layer": "4096->11008", "calibration_rows": int(xc.shape[0]),
                                 "grid": 20, "ms": round(e0.elapsed_time(e1), 3),
                                 "best_alpha": best.item(),
                                 "loss_alpha0": round(lo[0], 4), "loss_best": round(min(lo), 4)}
        del w, xc, sws
        torch.cuda.empty_cache()

    # ------------------------------------------------------------ prefill GEMM
    gemm = unfused = None
    if not args.no_gemm:
        log("prefill GEMM M=2048")
        gl = []
        ul = []
        tot_flop = tot_us = 0.0
        for j, (name, n, k) in enumerate(PREFILL_LAYERS):
            L = make_layer(3, n, k, m=PREFILL_M, layer=j)
            cp = [L["packed"], L["packed"].clone()]
            ws = awq.workspace(PREFILL_M, n, k, dev)
            us = graph_us([product(awq.awq_gemm, L, cp[r % 2], ws) for r in range(6)], 3,
                          warm_ms=150.0)
            fl = rl.flops(PREFILL_M, n, k)
            tot_flop += fl
            tot_us += us
            gl.append({"shape": f"{k}->{n}", "M": PREFILL_M, "us": round(us, 2),
                       "TFLOP/s": round(fl / us / 1e6, 1),
                       "frac": round(fl / us / 1e6 / rl.MFMA_F16_PEAK_TFLOPS, 4)})
            # unfused baseline: dequantize to binary16, then the library fp16 GEMM
            xs = (L["x"].float() * L["inv"].float()).half()  # X' as the fused path forms it
            wd = torch.empty((n, k), dtype=torch.float16, device=dev)

            def unfused_call(pk):
                awq.awq_dequant(pk, None, None, awq.LAYOUT_GFX950, n, k, GROUP, awq.FMT_ASYM,
                                out=wd)
                torch.matmul(xs, wd.t(), out=L["y"])

            # timed eagerly (the library GEMM cannot be captured into a graph here) over
            # the same two weight copies as the fused GEMM, after about 150 ms of the
            # same work so that the clocks have settled
            for r in range(max(2, int(150e3 / us))):
                unfused_call(cp[r % 2])
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for r in range(20):
                unfused_call(cp[r % 2])
            e1.record()
            torch.cuda.synchronize()
            u_us = e0.elapsed_time(e1) * 1e3 / 20
            ul.append({"shape": f"{k}->{n}", "M": PREFILL_M, "us": round(u_us, 2),
                       "TFLOP/s": round(fl / u_us / 1e6, 1),
                       "fused_speedup": round(u_us / us, 3)})
            del L, cp, xs, wd
            torch.cuda.empty_cache()
        agg = tot_flop / tot_us / 1e6
        gemm = {"workload": "llama3_8b_prefill_m2048", "metric": "TFLOP/s", "value": round(agg, 1),
                "roofline": {"bound": "mfma", "achieved": round(agg, 1),
                             "peak": round(rl.MFMA_F16_PEAK_TFLOPS, 1), "unit": "TFLOP/s",
                             "frac": round(agg / rl.MFMA_F16_PEAK_TFLOPS, 4)},
                "layers": gl}
        unfused = {"what": "awq_dequant to binary16 W_d, then torch.matmul (hipBLASLt fp16)",
                   "prefill": ul}

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
        "step_us_spread": step_spread,
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
                     "kernel": f"awq_gemv M=1, the 7 launches of a step ({sum_kernel_us / 7:.3f} "
                               f"us/launch average, {step_bytes / 7:.0f} B/launch average)"},
        "per_layer_kernel": per_layer,
        "ceilings": ceil,
        "kernel_sum_us_per_step": round(sum_kernel_us, 3),
        "kernel_only_GB/s": round(step_bytes / sum_kernel_us / 1e3, 1),
        **extra,
        "gemm": gemm,
        "unfused": unfused,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_decode_step_m1_traffic.txt")
GEMV_SOURCES = ("bit_weight_only_w4a16_amd/csrc/gemv.hip",
                "bit_weight_only_w4a16_amd/csrc/awq_internal.hpp")


def gemv_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in GEMV_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch (average over the 7 launches of a decode step) of the decode
    kernel, as measured by rocprofv3 counters (FETCH_SIZE + WRITE_SIZE, each scaled by
    what it reads for a plain copy of known size) and recorded with the hash of the
    kernel source; None if the kernel source changed since, or if none is recorded."""
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


def ceilings(dev, sizes, graph_us, rotation):
    """Streaming-read ceiling per decode shape (best of the probe's launch shapes, each
    over its own >1.2 GB of buffers so that no launch reads from the Infinity Cache) and
    the per-launch cost of an empty kernel, both as back-to-back launches in a graph."""
    import ctypes

    import torch

    from bit_weight_only_w4a16_amd import build as B

    probe = ctypes.CDLL(B.PROBE_LIB)
    probe.awq_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                            ctypes.c_void_p, ctypes.c_void_p]
    probe.awq_probe_empty.argtypes = [ctypes.c_void_p]
    sink = torch.zeros(4, dtype=torch.int32, device=dev)

    def stream():
        return torch.cuda.current_stream().cuda_stream

    out = {"stream_read": {}}
    for name, nbytes in sizes.items():
        stride = (nbytes + 255) // 256 * 256
        rot = rotation(stride)
        buf = torch.empty(rot * stride, dtype=torch.uint8, device=dev)
        base = buf.data_ptr()
        per_shape = []
        for shape in range(probe.awq_probe_shapes()):
            launches = [lambda r=r, shape=shape: probe.awq_probe_stream_read(
                base + r * stride, nbytes, shape, sink.data_ptr(), stream()) for r in range(rot)]
            per_shape.append(round(graph_us(launches, max(2, 1000 // rot)), 3))
        best = min(per_shape)
        out["stream_read"][name] = {"bytes": nbytes, "us_per_shape": per_shape, "best_us": best,
                                    "best_GB/s": round(nbytes / best / 1e3, 1),
                                    "copies": rot}
        del buf
        torch.cuda.empty_cache()
    out["empty_launch_us"] = round(graph_us([lambda: probe.awq_probe_empty(stream())] * 100, 20), 3)
    # matrix-core / ALU co-issue: 8 matrix instructions per iteration, each followed by
    # 0 .. 4 packed binary16 multiplies, one or two wavefronts per SIMD on every CU
    probe.awq_probe_mfma_alu.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_void_p]
    iters = 4000
    co = torch.empty(512 * 256, dtype=torch.float32, device=dev)
    coissue = {}
    for blocks, label in ((256, "one_wave_per_simd"), (512, "two_waves_per_simd")):
        row = {}
        for alu in range(5):
            for _ in range(3):
                probe.awq_probe_mfma_alu(co.data_ptr(), alu, blocks, iters, stream())
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(5):
                probe.awq_probe_mfma_alu(co.data_ptr(), alu, blocks, iters, stream())
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / 5
            mfma = blocks * 4 * iters * 8
            row[f"alu_{alu}"] = {"us": round(us, 1),
                                 "TFLOP/s": round(mfma * 16384 / us / 1e6, 1)}
        base = row["alu_0"]["us"]
        for alu in range(5):
            row[f"alu_{alu}"]["slowdown"] = round(row[f"alu_{alu}"]["us"] / base, 3)
        coissue[label] = row
    out["mfma_alu_coissue"] = coissue
    del co
    out["what"] = ("read-only kernel over the packed weight bytes of each decode shape, "
                   "16-byte non-temporal loads, 1 KiB per wavefront load, all loads of a "
                   "wavefront in flight; empty kernel back to back; graph-timed like the decode "
                   "kernel; mfma_alu_coissue: 8 independent 16x16x32 f16 matrix instructions per "
                   "iteration, each followed by alu_N packed f16 multiplies, on 256 or 512 "
                   "workgroups of 256 threads")
    return out


def cpu_baseline(seconds: float):
    """The CPU oracle (as it stands) on the benchmark's workloads: dequantization and the
    float64 product timed separately, with BLAS on every CPU thread this process is given
    (at most 16: the share of host CPUs that comes with one GPU), and on one thread."""
    import numpy as np

    import oracle
    from bit_weight_only_w4a16_amd import synth
    from bit_weight_only_w4a16_amd import roofline as rl

    from threadpoolctl import threadpool_info, threadpool_limits

    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    blas = [{"api": i.get("internal_api"), "version": i.get("version"),
             "threads": i.get("num_threads")} for i in threadpool_info()
            if i.get("user_api") == "blas"]

    def timed(fn, threads, budget):
        reps, t = 0, 0.0
        with threadpool_limits(threads):
            while t < budget or reps < 1:
                t0 = time.perf_counter()
                fn()
                t += time.perf_counter() - t0
                reps += 1
        return t / reps

    work = [  # (workload, config index, M, N, K)
        ("tiny_512x512_m1", 0, 1, 512, 512),
        ("llama7b_gate_4096x11008_m1", 1, 1, 11008, 4096),
        ("llama7b_gate_4096x11008_m16", 2, 16, 11008, 4096),
    ]
    rows = {}
    head = None
    for name, cfg, m, n, k in work:
        d = synth.layer_inputs(cfg, m, n, k, layer=4 if cfg == 1 else 0)
        s, inv = oracle.channel_scale(d["x_cal"], 0.5)
        layer = oracle.quantize_layer(d["w"], s, GROUP, oracle.FMT_ASYM)
        w_d = oracle.dequant_packed(layer["qweight"], layer["scales"], layer["qzeros"], GROUP,
                                    oracle.FMT_ASYM)
        byts = rl.algorithmic_bytes(m, n, k, GROUP, rl.FMT_ASYM, with_inv=True)
        budget = seconds / (len(work) * 4)
        deq = lambda: oracle.dequant_packed(layer["qweight"], layer["scales"], layer["qzeros"],
                                            GROUP, oracle.FMT_ASYM)
        prod = lambda: oracle.matmul_ref(d["x"], w_d, inv)
        r = {}
        for tag, threads in (("all", cores), ("one", 1)):
            td, tp = timed(deq, threads, budget), timed(prod, threads, budget)
            r[tag] = {"dequant_ms": round(td * 1e3, 2), "product_ms": round(tp * 1e3, 2),
                      "GB/s": round(byts / (td + tp) / 1e9, 4),
                      "GFLOP/s": round(rl.flops(m, n, k) / (td + tp) / 1e9, 3)}
        rows[name] = r
        if cfg == 1:
            head = r["all"]["GB/s"]
        del d, layer, w_d
    return {"value": head, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": "the oracle's dequantization and float64 product of one 4096->11008 "
                      "layer at M=1 (the decode layer the headline step is dominated by); "
                      f"about {seconds:.0f} s of CPU time over the rows below",
            "blas": blas, "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "workloads": rows}


if __name__ == "__main__":
    main()
