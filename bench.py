#!/usr/bin/env python3
"""Benchmark of the SmoothQuant W8A8 linear-layer path on one MI355X.

Default workload: the seven linear projections of one Llama-2-13B decoder
layer at 2048 prefill tokens (q, k, v, o 5120x5120; gate, up 13824x5120;
down 5120x13824), bf16 activations with 0.3% outlier channels x U(20,100),
N(0, 0.02) bf16 weights, alpha = 0.5, bf16 output. One step is one pass of the
whole path over one batch:
    per input (4 distinct: q/k/v share one, gate/up share one)
        calibration max|x| per input channel           sq_calib_absmax
    per projection (7)
        max|W| per input channel                       sq_calib_absmax
        smoothing factors + closed-form act scale      sq_smooth_factors
        W diag(s) -> per-row int8                      sq_quant_weight
        x * (1/s) -> per-tensor int8                   sq_smooth_quant_act
        int8 GEMM + fused dequant -> bf16              sq_w8a8_gemm
The batch is its own calibration batch (one batch of synthetic input per
step). Inputs are resident in HBM before timing starts.

value = int8 GEMM operations of the step (2*M*N*K summed over the seven
projections) / step time, in TOPS. The JSON line also carries the roofline of
the dominant kernel (the GEMM, timed with HIP events on the stream it runs on,
inside the timed steps) and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W8A8 smooth+quant+INT8 GEMM TOPS at 13B shapes; % of int8 MFMA peak"
PEAK_INT8_TOPS = 5000.0   # MI355X dense int8 MFMA, 5.0 POP/s
PEAK_HBM_GBS = 8000.0     # MI355X HBM3E, 8 TB/s


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--cpu-rows", type=int, default=512,
                    help="output rows of each GEMM the oracle computes in the CPU sample")
    ap.add_argument("--traffic", type=str, default=None,
                    help="JSON file with HBM traffic per GEMM launch (bytes) from rocprofv3 counters")
    return ap.parse_args()


class Group:
    def __init__(self, name, x_host, device):
        import torch
        from w8a8_post_quantization_channel_amd import synth
        self.name = name
        self.x_host = x_host
        self.x = synth.to_torch(x_host, device)
        self.act_max = torch.zeros(x_host.shape[1], dtype=torch.float32, device=device)


def setup(device):
    """Draw the layer's inputs on the host, move them to HBM, build layers."""
    import torch
    from w8a8_post_quantization_channel_amd import synth
    from w8a8_post_quantization_channel_amd.layer import W8A8Linear
    groups = {g: Group(g, synth.c2_group_x(g), device) for g in synth.C2_GROUPS}
    projs = []
    for name, g, n, k, _ in synth.C2_PROJECTIONS:
        w_host = synth.c2_projection_w(name)
        layer = W8A8Linear(synth.to_torch(w_host, device), alpha=0.5, max_tokens=synth.C2_TOKENS,
                           out_dtype=torch.bfloat16)
        layer.act_max = groups[g].act_max  # projections that share an input share its statistic
        projs.append((name, groups[g], layer, w_host))
    torch.cuda.synchronize()
    return groups, projs


def run_step(groups, projs, gemm_events=None):
    """One pass of the whole path. gemm_events: list to append (start, end)
    event pairs bracketing each GEMM launch."""
    import torch
    from w8a8_post_quantization_channel_amd import capi
    for g in groups.values():
        capi.sq_calib_absmax(g.x, g.act_max, False)
    for name, g, layer, _ in projs:
        layer.prepare()
        xq = layer.quantize_input(g.x)
        if gemm_events is not None:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            layer.matmul(xq)
            e1.record()
            gemm_events.append((name, e0, e1))
        else:
            layer.matmul(xq)


def gemm_ops(projs, m):
    return sum(2.0 * m * layer.n * layer.k for _, _, layer, _ in projs)


def cpu_baseline(groups, projs, rows):
    """The CPU oracle on a bounded sample of one step: every statistic and
    quantization pass in full, each GEMM on `rows` of the 2048 output rows;
    the full-step time is extrapolated linearly in GEMM rows."""
    import numpy as np
    from oracle.oracle import Oracle
    o = Oracle()
    m = next(iter(groups.values())).x_host.shape[0]
    t_total = 0.0
    wall0 = time.perf_counter()
    act_max = {}
    for g in groups.values():
        t0 = time.perf_counter()
        act_max[g.name] = o.calib_absmax(g.x_host)
        t_total += time.perf_counter() - t0
    for name, g, layer, w_host in projs:
        t0 = time.perf_counter()
        w_max = o.calib_absmax(w_host)
        s, inv_s, a = o.smooth_factors(act_max[g.name], w_max, 0.5)
        wq, ws = o.quant_weight(w_host, s)
        xq = o.quant_act(g.x_host, inv_s, a)
        t1 = time.perf_counter()
        acc = o.gemm_i32(np.ascontiguousarray(xq[:rows]), wq)
        o.dequant(acc, a, ws, bf16=True)
        t2 = time.perf_counter()
        t_total += (t1 - t0) + (t2 - t1) * (m / rows)
    wall = time.perf_counter() - wall0
    value = gemm_ops(projs, m) / t_total / 1e12
    return {"value": value, "unit": "TOPS", "cores": o.num_threads(), "kind": "oracle",
            "sample": (f"one 13B-layer step: all statistics and quantization passes in full, each of the 7 GEMMs "
                       f"on {rows} of {m} rows, extrapolated linearly in rows to the full step "
                       f"({t_total:.1f} s estimated; {wall:.1f} s of CPU work measured)")}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print("bench.py: this build runs on one GPU only; --gpus above 1 is not supported "
              "(the multi-GPU design is described in DESIGN.md)", file=sys.stderr)
        sys.exit(2)
    import torch
    from w8a8_post_quantization_channel_amd import capi
    capi.load()  # fails loudly when libsq.so is missing
    device = torch.device("cuda", 0)
    groups, projs = setup(device)
    m = next(iter(groups.values())).x.shape[0]

    for _ in range(args.warmup):
        run_step(groups, projs)
    torch.cuda.synchronize()

    events = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_step(groups, projs, events)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    ms_per_step = elapsed * 1e3 / args.steps
    ops = gemm_ops(projs, m)
    value = ops / (elapsed / args.steps) / 1e12

    # dominant kernel: the GEMM, averaged over every launch in the timed steps
    gemm_ms = [e0.elapsed_time(e1) for _, e0, e1 in events]
    by_name = {}
    for (name, _, _), t in zip(events, gemm_ms):
        by_name.setdefault(name, []).append(t)
    ops_by_name = {name: 2.0 * m * layer.n * layer.k for name, _, layer, _ in projs}
    avg_launch_ms = sum(gemm_ms) / len(gemm_ms)
    avg_launch_ops = sum(ops_by_name[n] for n, _, _ in events) / len(events)
    achieved = avg_launch_ops / (avg_launch_ms * 1e-3) / 1e12
    traffic = None
    if args.traffic:
        traffic = json.load(open(args.traffic)).get("bytes_per_launch")
    roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_INT8_TOPS, "unit": "TOPS",
                "frac": achieved / PEAK_INT8_TOPS, "traffic": traffic,
                "kernel": "gemm_kernel<OpI8, BMxBN, EpiDequant<bf16>>",
                "tiling": {n: list(capi.sq_gemm_tiling(m, layer.n)) for n, _, layer, _ in projs},
                "avg_launch_us": avg_launch_ms * 1e3,
                "per_projection_tops": {n: ops_by_name[n] / (sum(v) / len(v) * 1e-3) / 1e12
                                        for n, v in by_name.items()}}
    gemm_share = sum(gemm_ms) / (elapsed * 1e3)

    out = {
        "metric": METRIC, "value": value, "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8",
        "data": "synthetic (seeded numpy draws: N(0,1) activations, 0.3% outlier channels x U(20,100); "
                "N(0,0.02) weights; bf16)",
        "config": {"workload": "llama2-13b decoder layer, 7 linear projections, 2048 prefill tokens",
                   "tokens": m, "alpha": 0.5, "in_dtype": "bf16", "out_dtype": "bf16",
                   "projections": {n: [layer.n, layer.k] for n, _, layer, _ in projs},
                   "step": "calib absmax + weight absmax + smoothing + weight quant + act quant + int8 GEMM"},
        "roofline": roofline,
        "gemm_share_of_step": gemm_share,
        "gpu": torch.cuda.get_device_name(0),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(groups, projs, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
