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
step). Inputs are resident in HBM before timing starts. Everything runs on
one stream (--overlap: the preparation chain on a second stream, so
projection p + 1 is prepared while projection p multiplies).

value = int8 GEMM operations of the step (2*M*N*K summed over the seven
projections) / step time, in TOPS. The JSON line also carries the roofline of
the dominant kernel (the GEMM, timed with HIP events on the stream it runs on,
inside the timed steps) and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import itertools
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
    ap.add_argument("--overlap", action="store_true",
                    help="two phases (attention, MLP projections) on two streams: each phase's preparation on a "
                         "second stream, its grouped GEMM on the main stream, so preparation runs beside the "
                         "other phase's GEMM")
    ap.add_argument("--ramp-seconds", type=float, default=0.5,
                    help="untimed steps for at least this long before the warm-up steps: after the host-side "
                         "setup the GPU needs a few hundred ms of sustained load before its step time settles")
    ap.add_argument("--event-every", type=int, default=4,
                    help="bracket the GEMM launches with HIP events on every n-th timed step (each event pair "
                         "costs a few microseconds of step time)")
    ap.add_argument("--per-projection", action="store_true",
                    help="prepare the projections one by one with the single-form entry points (default: the "
                         "batched entry points, one launch per kind of pass for the whole block)")
    ap.add_argument("--cpu-rows", type=int, default=512,
                    help="output rows of each GEMM the oracle computes in the CPU sample")
    ap.add_argument("--traffic", type=str, default=None,
                    help="counter summary with the HBM bytes per GEMM launch (default: the committed "
                         "profiles/gemm_traffic__llama13b_prefill2048.md, used only if it matches gemm.hip)")
    ap.add_argument("--scales", default="f32", choices=["f32", "f16"],
                    help="scale storage of the layer13b step: fp32 (default), or every scale stored in fp16 "
                         "(smoothing factors, activation scale, per-row weight scales; the _f16 entry points)")
    ap.add_argument("--workload", default="layer13b",
                    choices=["layer13b", "decode7b", "alpha_search", "prefill70b", "hbm_passes", "copy_probe",
                             "variants", "fp8", "ceilings", "c1"],
                    help="layer13b (default, the headline line); the others measure the remaining "
                         "workloads, one JSON line each")
    return ap.parse_args()


class Group:
    def __init__(self, name, x_host, device):
        import torch
        from w8a8_post_quantization_channel_amd import synth
        self.name = name
        self.x_host = x_host
        self.x = synth.to_torch(x_host, device)
        self.act_max = torch.zeros(x_host.shape[1], dtype=torch.float32, device=device)


def setup(device, scales="f32"):
    """Draw the layer's inputs on the host, move them to HBM, build layers
    (scale storage `scales`: "f32" or "f16")."""
    import torch
    from w8a8_post_quantization_channel_amd import synth
    from w8a8_post_quantization_channel_amd.layer import W8A8Linear
    groups = {g: Group(g, synth.c2_group_x(g), device) for g in synth.C2_GROUPS}
    projs = []
    for name, g, n, k, _ in synth.C2_PROJECTIONS:
        w_host = synth.c2_projection_w(name)
        layer = W8A8Linear(synth.to_torch(w_host, device), alpha=0.5, max_tokens=synth.C2_TOKENS,
                           out_dtype=torch.bfloat16, scales=scales)
        layer.act_max = groups[g].act_max  # projections that share an input share its statistic
        projs.append((name, groups[g], layer, w_host))
    torch.cuda.synchronize()
    return groups, projs


PHASES = (("q", "k", "v", "o"), ("gate", "up", "down"))  # attention, then MLP: no input in common


def phased_block(groups, projs):
    """The 13B block as two phases (attention projections, MLP projections)."""
    from w8a8_post_quantization_channel_amd.layer import PhasedBlock
    by_name = {name: (g, layer) for name, g, layer, _ in projs}
    phases = []
    for names in PHASES:
        used = []
        for n in names:
            if by_name[n][0] not in used:
                used.append(by_name[n][0])
        phases.append(([by_name[n][1] for n in names], [(g.x, g.act_max) for g in used],
                       [by_name[n][0].x for n in names]))
    return PhasedBlock(phases)


def run_phased(block, side, gemm_events=None):
    """One pass of the whole path on two streams (preparation on `side`, the
    two grouped GEMM launches on the current stream); gemm_events as in
    run_step, one pair per phase ("attn", "mlp")."""
    import torch
    main = torch.cuda.current_stream()
    marks = {}

    def on_gemm(i, before):
        if gemm_events is None:
            return
        e = torch.cuda.Event(enable_timing=True)
        e.record(main)
        if before:
            marks[i] = e
        else:
            gemm_events.append((("attn", "mlp")[i], marks[i], e))

    block.step(side, main, on_gemm)


def block_tiling(m, projs, phases=False):
    """The tile of each projection in the block's grouped GEMM launch (one
    launch, or one per phase), as the library chooses it for the group; the
    launch lists the products newest-first."""
    from w8a8_post_quantization_channel_amd import capi
    names = [n for n, _, _, _ in projs]
    shape = {n: (m, layer.n, layer.k) for n, _, layer, _ in projs}
    out = {}
    for part in (PHASES if phases else [names]):
        part = [n for n in names if n in part][::-1]
        out.update(zip(part, map(list, capi.sq_gemm_batched_tiling([shape[n] for n in part]))))
    return {n: out[n] for n in names}


def run_step(groups, projs, gemm_events=None, side=None, batched=True):
    """One pass of the whole path. gemm_events: list to append (name, start,
    end) event pairs bracketing each GEMM launch, recorded on the stream the
    GEMM runs on. side: a second stream for the preparation chain (statistics,
    smoothing, weight and activation quantization), so that projection p + 1
    is prepared while the GEMM of projection p runs; each GEMM waits for its
    own preparation, and the step starts after the previous step's GEMMs.
    batched: the statistics (4 inputs + 7 weights), smoothing factors and
    weight codes of all projections come from the batched entry points before
    the first GEMM; otherwise they are made projection by projection."""
    import torch
    from w8a8_post_quantization_channel_amd import capi
    from w8a8_post_quantization_channel_amd.layer import forward_block, prepare_block
    main = torch.cuda.current_stream()
    prep = side if side is not None else main
    if side is not None:
        side.wait_stream(main)
    if batched:
        layers = [layer for _, _, layer, _ in projs]
        e0 = e1 = None
        if gemm_events is not None:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)

        def between():
            if side is not None:
                main.wait_stream(prep)
            if e0 is not None:
                e0.record(main)

        with torch.cuda.stream(prep):
            prepare_block(layers, [(g.x, g.act_max) for g in groups.values()], prep)
            forward_block(layers, [g.x for _, g, _, _ in projs], prep, main, between)
        if e1 is not None:
            e1.record(main)
            gemm_events.append(("block", e0, e1))
        return
    with torch.cuda.stream(prep):
        for g in groups.values():
            capi.sq_calib_absmax(g.x, g.act_max, False, stream=prep)
    for name, g, layer, _ in projs:
        with torch.cuda.stream(prep):
            if not batched:
                layer.prepare(stream=prep)
            xq = layer.quantize_input(g.x, stream=prep)
        if side is not None:
            main.wait_stream(prep)
        if gemm_events is not None:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(main)
            layer.matmul(xq, stream=main)
            e1.record(main)
            gemm_events.append((name, e0, e1))
        else:
            layer.matmul(xq, stream=main)


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gemm_traffic__llama13b_prefill2048.md")


def gemm_source_hash() -> str:
    import hashlib
    path = os.path.join(ROOT, "w8a8_post_quantization_channel_amd", "csrc", "gemm.hip")
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def gemm_traffic(path=None):
    """HBM bytes per GEMM launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE
    (scaled by a plain copy), read from the committed summary; None when the
    summary is missing or was taken on a different gemm.hip."""
    import re
    path = path or TRAFFIC_SUMMARY
    if not os.path.exists(path):
        return None
    text = open(path).read()
    h = re.search(r"^gemm\.hip sha256\[:16\]: ([0-9a-f]{16})$", text, re.M)
    b = re.search(r"^bytes_per_launch: ([0-9.eE+]+)$", text, re.M)
    if not h or not b or h.group(1) != gemm_source_hash():
        return None
    return float(b.group(1))


def gemm_ops(projs, m):
    return sum(2.0 * m * layer.n * layer.k for _, _, layer, _ in projs)


def cpu_baseline(groups, projs, rows, one_thread_rows=32, scales="f32"):
    """The CPU oracle on a bounded sample of one step: every statistic and
    quantization pass in full, each GEMM on `rows` of the 2048 output rows;
    the full-step time is extrapolated linearly in GEMM rows. Run on all the
    threads the oracle starts with, then again on one thread (GEMMs on
    one_thread_rows rows)."""
    from oracle.oracle import Oracle
    o = Oracle()
    out = oracle_step(o, groups, projs, rows, scales)
    threads = o.num_threads()
    o.set_num_threads(1)
    one = oracle_step(o, groups, projs, one_thread_rows, scales)
    o.set_num_threads(threads)
    out["cpu_model"] = cpu_model()
    out["one_thread"] = {"value": one["value"], "unit": "TOPS", "cores": 1, "sample": one["sample"]}
    return out


def oracle_step(o, groups, projs, rows, scales="f32"):
    import numpy as np
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
        if scales == "f16":
            s16, a16 = o.smooth_factors_h(act_max[g.name], w_max, 0.5)
            wq, ws16 = o.quant_weight_h(w_host, s16)
            xq = o.quant_act_h(g.x_host, s16, a16)
        else:
            s, inv_s, a = o.smooth_factors(act_max[g.name], w_max, 0.5)
            wq, ws = o.quant_weight(w_host, s)
            xq = o.quant_act(g.x_host, inv_s, a)
        t1 = time.perf_counter()
        acc = o.gemm_i32(np.ascontiguousarray(xq[:rows]), wq)
        if scales == "f16":
            o.dequant_h(acc, a16, ws16, bf16=True)
        else:
            o.dequant(acc, a, ws, bf16=True)
        t2 = time.perf_counter()
        t_total += (t1 - t0) + (t2 - t1) * (m / rows)
    wall = time.perf_counter() - wall0
    value = gemm_ops(projs, m) / t_total / 1e12
    return {"value": value, "unit": "TOPS", "cores": o.num_threads(), "kind": "oracle",
            "sample": (f"one 13B-layer step: all statistics and quantization passes in full, each of the 7 GEMMs "
                       f"on {rows} of {m} rows, extrapolated linearly in rows to the full step "
                       f"({t_total:.1f} s estimated; {wall:.1f} s of CPU work measured)")}


def timed(fn, reps, warmup=3, warm_ms=30.0):
    """Average milliseconds of fn() on the current stream (HIP events), after
    `warmup` untimed calls and at least warm_ms of untimed calls (the first
    calls after other work touched other buffers run slow)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < warm_ms:
        fn()
        torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def workload_decode7b(device):
    """Llama-2-7B decode: x * (1/s) -> int8 and the int8 GEMM with fused
    dequant, M in {1, 8, 16, 64}, weights cold (32 layers' weights rotate, more
    than the 256 MB Infinity Cache). The 32 layers are captured once in a HIP
    graph (act quant + GEMM per layer; and the GEMMs alone) and replayed, so
    the figure is GPU time without host launch gaps; the replay's last output
    is checked against an eager call. Algorithmic bytes: int8 weight + bf16 x
    + int8 x + bf16 y + scales (GEMM alone: int8 weight + int8 x + bf16 y +
    scales)."""
    import torch
    from w8a8_post_quantization_channel_amd import capi, synth
    layers = 32
    out = {}
    stream = torch.cuda.Stream()

    def replay_ms(graph, reps=10):
        graph.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    for sid, (name, n, k) in enumerate(synth.SHAPES_7B):
        wq = [torch.randint(-127, 128, (n, k), dtype=torch.int8, device=device) for _ in range(layers)]
        ws = torch.rand(n, device=device) * 1e-3 + 1e-4
        inv_s = torch.rand(k, device=device) + 0.5
        a = torch.full((4,), 0.05, device=device)
        for m in synth.DECODE_M:
            x = torch.randn((m, k), device=device).to(torch.bfloat16)
            xq = torch.empty((m, k), dtype=torch.int8, device=device)
            y = torch.empty((m, n), dtype=torch.bfloat16, device=device)
            capi.sq_smooth_quant_act(x, inv_s, a, xq)  # eager reference of the last layer
            capi.sq_w8a8_gemm(xq, wq[-1], a, ws, y)
            torch.cuda.synchronize()
            y_ref = y.clone()
            y.zero_()
            g_full, g_gemm = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_full, stream=stream):
                for l in range(layers):
                    capi.sq_smooth_quant_act(x, inv_s, a, xq)
                    capi.sq_w8a8_gemm(xq, wq[l], a, ws, y)
            with torch.cuda.graph(g_gemm, stream=stream):
                for l in range(layers):
                    capi.sq_w8a8_gemm(xq, wq[l], a, ws, y)
            us_full = replay_ms(g_full) * 1e3 / layers
            ok_full = torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
            us_gemm = replay_ms(g_gemm) * 1e3 / layers
            ok_gemm = torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
            if not (ok_full and ok_gemm):
                raise RuntimeError(f"graph replay differs from the eager result ({name}, m={m})")
            byts = n * k + m * k * 3 + m * n * 2 + n * 4 + k * 4
            gbytes = n * k + m * k + m * n * 2 + n * 4
            out[f"{name}_{n}x{k}_m{m}"] = {
                "us": us_full, "GB/s": byts / (us_full * 1e-6) / 1e9,
                "hbm_frac": byts / (us_full * 1e-6) / 1e9 / PEAK_HBM_GBS,
                "gemm_us": us_gemm, "gemm_GB/s": gbytes / (us_gemm * 1e-6) / 1e9,
                "gemm_hbm_frac": gbytes / (us_gemm * 1e-6) / 1e9 / PEAK_HBM_GBS}
            del g_full, g_gemm
        del wq
        torch.cuda.empty_cache()
    tot_b = sum(v["GB/s"] * v["us"] for v in out.values()) / sum(v["us"] for v in out.values())
    # the projections that read one input, as one batched GEMM call per layer
    # (one vector-ALU or skinny launch for all of them) against a call each
    grouped = {}
    for gname, n, k, cnt in (("qkv", 4096, 4096, 3), ("gate_up", 11008, 4096, 2)):
        wq = [[torch.randint(-127, 128, (n, k), dtype=torch.int8, device=device) for _ in range(cnt)]
              for _ in range(layers)]
        ws = [torch.rand(n, device=device) * 1e-3 + 1e-4 for _ in range(cnt)]
        a = [torch.full((4,), 0.05, device=device) for _ in range(cnt)]
        for m in (1, 2, 4, 8, 16, 64):
            xq = torch.randint(-127, 128, (m, k), dtype=torch.int8, device=device)
            ys = [torch.empty((m, n), dtype=torch.bfloat16, device=device) for _ in range(cnt)]
            g_b, g_s = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_b, stream=stream):
                for l in range(layers):
                    capi.sq_w8a8_gemm_batched([xq] * cnt, wq[l], a, ws, ys)
            with torch.cuda.graph(g_s, stream=stream):
                for l in range(layers):
                    for j in range(cnt):
                        capi.sq_w8a8_gemm(xq, wq[l][j], a[j], ws[j], ys[j])
            us_b = replay_ms(g_b) * 1e3 / layers
            y_b = [y.clone() for y in ys]
            us_s = replay_ms(g_s) * 1e3 / layers
            if not all(torch.equal(p.view(torch.int16), q.view(torch.int16)) for p, q in zip(y_b, ys)):
                raise RuntimeError(f"batched decode GEMM differs from the single calls ({gname}, m={m})")
            gbytes = cnt * (n * k + m * k + m * n * 2 + n * 4)
            grouped[f"{gname}_{cnt}x{n}x{k}_m{m}"] = {
                "batched_us": us_b, "batched_GB/s": gbytes / (us_b * 1e-6) / 1e9,
                "batched_hbm_frac": gbytes / (us_b * 1e-6) / 1e9 / PEAK_HBM_GBS,
                "single_calls_us": us_s, "single_calls_hbm_frac": gbytes / (us_s * 1e-6) / 1e9 / PEAK_HBM_GBS}
            del g_b, g_s
        del wq
        torch.cuda.empty_cache()
    return {"metric": "W8A8 decode (act quant + int8 GEMM) HBM GB/s, Llama-2-7B shapes, cold weights",
            "value": tot_b, "unit": "GB/s", "n_gpus": 1, "higher_is_better": True, "dtype": "int8",
            "data": "synthetic",
            "config": {"workload": "llama2-7b decode, M in {1,8,16,64}, 32 rotating layers, HIP-graph replay"},
            "per_case": out, "grouped_gemm": grouped, "cpu_oracle": decode_oracle_times()}


def decode_oracle_times(ms=(1, 64)):
    """The oracle's act quant + int8 GEMM + bf16 dequant for one decode call
    of each 7B shape, on all of its threads and on one (median of 3)."""
    import os as _os
    import statistics
    import numpy as np
    from oracle.oracle import Oracle
    from w8a8_post_quantization_channel_amd import synth
    o = Oracle()
    threads = min(len(_os.sched_getaffinity(0)), 16)
    g = np.random.default_rng(3100)
    res = {"cpu_model": cpu_model(), "threads": threads}
    for name, n, k in synth.SHAPES_7B:
        wq = g.integers(-127, 128, (n, k), dtype=np.int8)
        ws = g.uniform(1e-4, 1e-3, n).astype(np.float32)
        inv_s = g.uniform(0.5, 1.5, k).astype(np.float32)
        for m in ms:
            x = g.standard_normal((m, k), dtype=np.float32)

            def call():
                xq = o.quant_act(x, inv_s, np.float32(0.05))
                o.dequant(o.gemm_i32(xq, wq), np.float32(0.05), ws, bf16=True)

            row = {}
            for label, t in (("all_threads_us", threads), ("one_thread_us", 1)):
                o.set_num_threads(t)
                call()
                times = []
                for _ in range(3):
                    t0 = time.perf_counter()
                    call()
                    times.append((time.perf_counter() - t0) * 1e6)
                row[label] = statistics.median(times)
            res[f"{name}_{n}x{k}_m{m}"] = row
    o.set_num_threads(threads)
    return res


def workload_alpha_search(device):
    """Alpha grid search on a 4096 -> 11008 layer: 8 kept batches of 2048
    tokens (Student-t, 12 channels x50), grid {0.25, 0.5, 0.75, 1}."""
    import torch
    from w8a8_post_quantization_channel_amd import capi, synth
    xs = [synth.to_torch(x, device) for x in synth.c4_batches(8)]
    w = synth.to_torch(synth.c4_weight(), device)
    nbytes = capi.sq_alpha_search_workspace(8, 2048, 11008, 4096, 4)
    wsp = torch.empty(nbytes, dtype=torch.uint8, device=device)
    capi.sq_alpha_search(xs, w, wsp)
    reps = 5
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        mse, best = capi.sq_alpha_search(xs, w, wsp)
    ms = (time.perf_counter() - t0) * 1e3 / reps
    ops_i8 = 4 * 2.0 * 8 * 2048 * 11008 * 4096
    ops_ref = 2.0 * 8 * 2048 * 11008 * 4096
    return {"metric": "alpha grid search time, 4096->11008 layer, 8x2048 tokens", "value": ms, "unit": "ms",
            "n_gpus": 1, "higher_is_better": False, "dtype": "int8+bf16", "data": "synthetic",
            "config": {"workload": "alpha search 8x2048 tokens, K=4096, N=11008, grid 0.25/0.5/0.75/1.0"},
            "mse": mse, "best_alpha": synth.ALPHA_GRID[best],
            "effective_TOPS": (ops_i8 + ops_ref) / (ms * 1e-3) / 1e12}


def workload_copy_probe(device):
    """A plain copy of known size (torch's copy kernel, 1 GiB read + 1 GiB
    written per launch, 5 launches): the reference that scales the FETCH_SIZE
    and WRITE_SIZE counters to bytes."""
    import torch
    n = 1 << 29  # bf16 elements: 1 GiB
    x = torch.ones(n, dtype=torch.bfloat16, device=device)
    y = torch.empty_like(x)
    ms = timed(lambda: y.copy_(x), 5, warmup=0)
    return {"metric": "plain copy, bytes per launch", "value": n * 2, "unit": "bytes read (and written) per launch",
            "n_gpus": 1, "higher_is_better": True, "launches": 5, "us_per_launch": ms * 1e3,
            "config": {"workload": "copy 1 GiB bf16 -> bf16"}}


def workload_prefill70b(device):
    """Llama-2-70B prefill, 4096 tokens, int8 weights of all 80 layers
    resident in HBM (68.4 GB): per layer, the runtime path (act quant + int8
    GEMM) of the 7 projections, as one batched activation quantizer (q/k/v read
    the attention input once, gate/up the MLP input) and one grouped GEMM;
    the per-projection schedule (14 launches per layer) is timed beside it.
    Weights are random int8 (the values do not change the timing)."""
    import torch
    from w8a8_post_quantization_channel_amd import capi
    layers, m = 80, 4096
    projs = [("q", 8192, 8192, "attn"), ("k", 1024, 8192, "attn"), ("v", 1024, 8192, "attn"),
             ("o", 8192, 8192, "attn_out"), ("gate", 28672, 8192, "mlp"), ("up", 28672, 8192, "mlp"),
             ("down", 8192, 28672, "mlp_mid")]
    g = torch.Generator(device=device)
    g.manual_seed(70)
    weights = []
    for _ in range(layers):
        weights.append([torch.randint(-127, 128, (n, k), dtype=torch.int8, device=device, generator=g)
                        for _, n, k, _ in projs])
    resident = sum(w.numel() for lw in weights for w in lw)
    ks = {"attn": 8192, "attn_out": 8192, "mlp": 8192, "mlp_mid": 28672}
    xs = {name: torch.randn((m, k), device=device, generator=g).to(torch.bfloat16) for name, k in ks.items()}
    inv_s = [torch.rand(k, device=device, generator=g) + 0.5 for _, _, k, _ in projs]
    ws = [torch.rand(n, device=device, generator=g) * 1e-3 for _, n, _, _ in projs]
    a = [torch.full((4,), 0.05, device=device) for _ in projs]
    xq = [torch.empty((m, k), dtype=torch.int8, device=device) for _, _, k, _ in projs]
    y = [torch.empty((m, n), dtype=torch.bfloat16, device=device) for _, n, _, _ in projs]
    x_of = [xs[src] for _, _, _, src in projs]

    def layer_batched(i):
        capi.sq_smooth_quant_act_batched(x_of, inv_s, a, xq)
        capi.sq_w8a8_gemm_batched(xq, weights[i], a, ws, y)

    def layer_single(i):
        for j in range(len(projs)):
            capi.sq_smooth_quant_act(x_of[j], inv_s[j], a[j], xq[j])
            capi.sq_w8a8_gemm(xq[j], weights[i][j], a[j], ws[j], y[j])

    def run(layer):
        for i in range(2):
            layer(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(layers):
            layer(i)
        torch.cuda.synchronize()
        return time.perf_counter() - t0
    run(layer_batched)
    dt_single = run(layer_single)
    dt = run(layer_batched)
    ops = layers * sum(2.0 * m * n * k for _, n, k, _ in projs)
    return {"metric": "W8A8 act quant + int8 GEMM TOPS, Llama-2-70B shapes, 80 layers resident",
            "value": ops / dt / 1e12, "unit": "TOPS", "n_gpus": 1, "higher_is_better": True, "dtype": "int8",
            "data": "synthetic", "config": {"workload": "llama2-70b prefill 4096 tokens x 80 layers",
                                            "resident_int8_weight_GB": resident / 1e9,
                                            "tiling": dict(zip([p for p, _, _, _ in projs], map(list, capi.sq_gemm_batched_tiling(
                                                [(m, n, k) for _, n, k, _ in projs])))),
                                            "schedule": "per layer: one batched act quant + one grouped GEMM"},
            "ms_per_layer": dt * 1e3 / layers, "frac_of_int8_peak": ops / dt / 1e12 / PEAK_INT8_TOPS,
            "per_projection_ms_per_layer": dt_single * 1e3 / layers,
            "per_projection_tops": ops / dt_single / 1e12}


def workload_hbm_passes(device):
    """The HBM-bound passes at the workloads' largest sizes: calibration
    absmax over 512 x 512 tokens (K = 5120 and 13824), activation quant at
    4096 x 28672 and over the 262144 x 5120 calibration-size tensor, weight
    absmax + quant of a 28672 x 8192 weight and weight quant of each 13B
    shape and of the 13B block (batched). Passes that move less than 1.1 GB
    per call cycle through enough buffer sets to exceed it, so repeated calls
    do not run from the 256 MB Infinity Cache."""
    import torch
    from w8a8_post_quantization_channel_amd import capi, synth
    out = {}
    for k in (5120, 13824):
        x = synth.device_activations(2100 + k, 512 * 512, k, synth.outlier_channels(2000 + k, k), device)
        am = torch.empty(k, dtype=torch.float32, device=device)
        ms = timed(lambda: capi.sq_calib_absmax(x, am, False), 5)
        byts = x.numel() * 2 + k * 4
        out[f"calib_absmax_262144x{k}"] = {"us": ms * 1e3, "GB/s": byts / (ms * 1e-3) / 1e9,
                                           "hbm_frac": byts / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
        del x
        torch.cuda.empty_cache()
    # every pass below runs over enough buffer sets (each call the next set)
    # that one cycle moves more than 1.1 GB, past the 256 MB Infinity Cache
    def sets_for(nbytes):
        return max(1, -(-int(1.1e9) // int(nbytes)))

    def cycle(calls):
        it = itertools.cycle(calls)
        return lambda: next(it)()

    def record(key, ms, byts, nsets):
        out[key] = {"us": ms * 1e3, "GB/s": byts / (ms * 1e-3) / 1e9,
                    "hbm_frac": byts / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "buffer_sets": nsets}

    # activation quant: the 70B MLP input (4096 x 28672) and the 13B
    # calibration-size tensor (262144 x 5120, 4.0 GB of traffic)
    for m, k in ((4096, 28672), (262144, 5120)):
        byts = m * k * 3 + k * 4
        nsets = sets_for(byts)
        inv_s = torch.rand(k, device=device) + 0.5
        a = torch.full((4,), 0.05, device=device)
        bufs = [((torch.randn((m, k), device=device) * 0.5).to(torch.bfloat16),
                 torch.empty((m, k), dtype=torch.int8, device=device)) for _ in range(nsets)]
        ms = timed(cycle([lambda x=x, xq=xq: capi.sq_smooth_quant_act(x, inv_s, a, xq) for x, xq in bufs]),
                   max(10, 2 * nsets))
        record(f"act_quant_{m}x{k}", ms, byts, nsets)
        if nsets > 1:  # the same call on one buffer set, for comparison
            x, xq = bufs[0]
            ms = timed(lambda: capi.sq_smooth_quant_act(x, inv_s, a, xq), 10)
            record(f"act_quant_{m}x{k}_same_buffers", ms, byts, 1)
        del bufs
        torch.cuda.empty_cache()
    # weight statistics and codes of a 70B MLP weight and of each 13B shape
    for n, k in ((28672, 8192), (5120, 5120), (13824, 5120), (5120, 13824)):
        qbytes = n * k * 3 + k * 4 + n * 4
        nsets = sets_for(qbytes)
        bufs = [((torch.randn((n, k), device=device) * 0.02).to(torch.bfloat16),
                 torch.rand(k, device=device) + 0.5, torch.empty(k, dtype=torch.float32, device=device),
                 torch.empty((n, k), dtype=torch.int8, device=device),
                 torch.empty(n, dtype=torch.float32, device=device)) for _ in range(nsets)]
        if n == 28672:
            ms = timed(cycle([lambda w=w, wm=wm: capi.sq_calib_absmax(w, wm, False) for w, _, wm, _, _ in bufs]),
                       max(10, 2 * nsets))
            record(f"weight_absmax_{n}x{k}", ms, n * k * 2 + k * 4, nsets)
        ms = timed(cycle([lambda w=w, s_=s_, wq=wq, wsc=wsc: capi.sq_quant_weight(w, s_, wq, wsc)
                          for w, s_, _, wq, wsc in bufs]), max(10, 2 * nsets))
        record(f"weight_quant_{n}x{k}", ms, qbytes, nsets)
        del bufs
        torch.cuda.empty_cache()
    # the 13B block's seven weights as the step prepares them: statistics and
    # codes from the batched entry points
    blk = [(5120, 5120)] * 4 + [(13824, 5120)] * 2 + [(5120, 13824)]
    qbytes = sum(n * k * 3 + k * 4 + n * 4 for n, k in blk)
    nsets = sets_for(qbytes)
    sets = []
    for _ in range(nsets):
        sets.append(([(torch.randn(sh, device=device) * 0.02).to(torch.bfloat16) for sh in blk],
                     [torch.rand(k, device=device) + 0.5 for _, k in blk],
                     [torch.empty(sh, dtype=torch.int8, device=device) for sh in blk],
                     [torch.empty(n, dtype=torch.float32, device=device) for n, _ in blk],
                     [torch.empty(k, dtype=torch.float32, device=device) for _, k in blk]))
    ms = timed(cycle([lambda W=W, WM=WM: capi.sq_calib_absmax_batched(W, WM, False) for W, _, _, _, WM in sets]),
               max(10, 2 * nsets))
    record("weight_absmax_13b_block_batched", ms, sum(n * k * 2 + k * 4 for n, k in blk), nsets)
    ms = timed(cycle([lambda W=W, S=S, WQ=WQ, WS=WS: capi.sq_quant_weight_batched(W, S, WQ, WS)
                      for W, S, WQ, WS, _ in sets]), max(10, 2 * nsets))
    record("weight_quant_13b_block_batched", ms, qbytes, nsets)
    # the same with binary16 scale storage: s and w_scale in fp16 (half the
    # s bytes every block reads from L2)
    h16 = [([s.half() for s in S], [torch.empty(n, dtype=torch.float16, device=device) for n, _ in blk])
           for _, S, _, _, _ in sets]
    ms = timed(cycle([lambda W=W, S16=S16, WQ=WQ, WS16=WS16: capi.sq_quant_weight_f16_batched(W, S16, WQ, WS16)
                      for (W, _, WQ, _, _), (S16, WS16) in zip(sets, h16)]), max(10, 2 * nsets))
    record("weight_quant_13b_block_batched_f16_scales", ms, sum(n * k * 3 + k * 2 + n * 2 for n, k in blk), nsets)
    del sets, h16
    torch.cuda.empty_cache()
    # practical ceilings on the same tensor sizes: a plain copy (read = write)
    # and a plain bf16 -> int8 conversion (2 bytes read per byte written, the
    # traffic mix of the quantization passes), both torch kernels
    x = torch.randn((4096, 28672), device=device).to(torch.bfloat16)
    y = torch.empty_like(x)
    ms = timed(lambda: y.copy_(x), 10)
    byts = x.numel() * 4
    out["ceiling_copy_bf16_4096x28672"] = {"us": ms * 1e3, "GB/s": byts / (ms * 1e-3) / 1e9,
                                           "hbm_frac": byts / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    yq = torch.empty(x.shape, dtype=torch.int8, device=device)
    ms = timed(lambda: yq.copy_(x), 10)
    byts = x.numel() * 3
    out["ceiling_bf16_to_int8_4096x28672"] = {"us": ms * 1e3, "GB/s": byts / (ms * 1e-3) / 1e9,
                                              "hbm_frac": byts / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    calib = [v for kk, v in out.items() if kk.startswith("calib")]
    return {"metric": "HBM GB/s of the calibration absmax (512x512 tokens) and activation quant passes",
            "value": min(v["GB/s"] for v in calib + [out["act_quant_4096x28672"], out["act_quant_262144x5120"]]),
            "unit": "GB/s",
            "n_gpus": 1, "higher_is_better": True, "dtype": "bf16->fp32/int8", "data": "synthetic",
            "config": {"workload": "largest HBM passes of the 13B calibration and 70B prefill workloads"},
            "per_pass": out}


def ceiling_operand_sets(device):
    """Register operands for the MFMA-only loop (16 operands x 64 lanes x 16
    bytes): all-ones bytes; uniform random bytes (seeded); and 32x32 fragments
    of the 13B step's own codes, chain c's A operand from the weight codes of
    q_proj (rows 1024 + 32c .., the first operand of the GEMM's MFMAs) and its
    B operand from the activation codes of the same projection, 32 K bytes at
    K = 2048 as the GEMM's fragments hold them."""
    import numpy as np
    import torch
    sets = {"ones": np.ones((16, 64, 16), np.int8),
            "random": np.random.default_rng(20240531).integers(-128, 128, (16, 64, 16)).astype(np.int8)}
    groups, projs = setup(device)
    _, g, layer, _ = projs[0]
    layer.calibrate(g.x)
    layer.prepare()
    xq = layer.quantize_input(g.x).cpu().numpy()
    wq = layer.wq.cpu().numpy()
    codes = np.empty((16, 64, 16), np.int8)
    k0 = 2048
    for c in range(8):
        for lane in range(64):
            r, kk = lane % 32, k0 + (lane // 32) * 16
            codes[2 * c, lane] = wq[1024 + 32 * c + r, kk:kk + 16]
            codes[2 * c + 1, lane] = xq[1024 + 32 * c + r, kk:kk + 16]
    sets["codes"] = codes
    del groups, projs, layer, xq, wq
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return sets


def workload_ceilings(device):
    """Measured ceilings written for this path: an MFMA-only loop (int8
    v_mfma_i32_32x32x32_i8 on register operands: all-ones bytes, random bytes,
    or fragments of the step's own codes; 8 independent chains per wave, 1 and
    2 blocks of 4 waves per compute unit), a 16-byte-vector copy, a narrowing
    copy (2 bytes read per byte written, the quantizers' mix) and a
    16-byte-vector read of 1 GiB each (well past the 256 MB Infinity Cache).
    Each MFMA run is checked against its closed-form sum, the copy byte for
    byte, the read against the XOR of its words."""
    import numpy as np
    import torch
    from w8a8_post_quantization_channel_amd import capi, ceiling
    out = {}
    sink = torch.zeros(4, dtype=torch.int32, device=device)
    iters = 20000
    for name, ops_host in ceiling_operand_sets(device).items():
        dots = ceiling.ceiling_chain_dots(ops_host)
        if max(abs(d) for d in dots) * iters >= 1 << 31:
            raise RuntimeError(f"{name}: accumulators would leave int32 ({dots})")
        operands = torch.from_numpy(ops_host.reshape(-1).copy()).to(device)
        for per_cu in (1, 2):
            sink.zero_()
            ops = ceiling.sq_ceiling_mfma(iters, per_cu, operands, sink)
            torch.cuda.synchronize()
            waves = ops // (8 * iters * 2 * 32 * 32 * 32)
            expect = ceiling.ceiling_expected_sink(ops_host, iters, waves)
            got = int(sink[0].item()) % (1 << 32)
            if got != expect:
                raise RuntimeError(f"MFMA loop check failed ({name}): {got} != {expect}")
            # steady state: half a second of untimed calls, then ~0.2-0.5 s timed (a few
            # ms of MFMA load is too short for the power manager to settle)
            ms = timed(lambda: ceiling.sq_ceiling_mfma(iters, per_cu, operands, sink), 100, warmup=2, warm_ms=500)
            tops = ops / (ms * 1e-3) / 1e12
            out[f"mfma_loop_{name}_{per_cu}_blocks_per_cu"] = {
                "TOPS": tops, "frac_of_int8_peak": tops / PEAK_INT8_TOPS,
                # the clock at which a matrix pipe issuing every cycle gives this rate
                "issue_clock_GHz": 2.4 * tops / PEAK_INT8_TOPS}
    n = 1 << 30
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, device=device)
    dst = torch.empty_like(src)
    ceiling.sq_ceiling_copy(src, dst)
    torch.cuda.synchronize()
    if not torch.equal(src, dst):
        raise RuntimeError("copy check failed")
    ms = timed(lambda: ceiling.sq_ceiling_copy(src, dst), 10)
    out["copy_1GiB"] = {"GB/s": 2 * n / (ms * 1e-3) / 1e9, "hbm_frac": 2 * n / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    del dst
    half = torch.empty(n // 2, dtype=torch.uint8, device=device)
    ceiling.sq_ceiling_narrow(src, half)
    torch.cuda.synchronize()
    if not torch.equal(half, src.view(-1, 16)[:, :8].reshape(-1)):
        raise RuntimeError("narrowing copy check failed")
    ms = timed(lambda: ceiling.sq_ceiling_narrow(src, half), 10)
    out["narrow_1GiB_to_512MiB"] = {"GB/s": 1.5 * n / (ms * 1e-3) / 1e9,
                                    "hbm_frac": 1.5 * n / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    del half
    xor = np.bitwise_xor.reduce(src.cpu().numpy().view(np.uint32))
    sink.zero_()
    ceiling.sq_ceiling_read(src, sink)
    torch.cuda.synchronize()
    if int(sink[0].item()) % (1 << 32) != int(xor):
        raise RuntimeError("read check failed")
    ms = timed(lambda: ceiling.sq_ceiling_read(src, sink), 10)
    out["read_1GiB"] = {"GB/s": n / (ms * 1e-3) / 1e9, "hbm_frac": n / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    return {"metric": "measured ceilings: int8 MFMA-only loop TOPS (step's own codes), 16-byte copy and read GB/s",
            "value": out["mfma_loop_codes_1_blocks_per_cu"]["TOPS"], "unit": "TOPS",
            "n_gpus": 1, "higher_is_better": True, "dtype": "int8 / bytes", "data": "synthetic",
            "config": {"workload": "MFMA-only loop on every compute unit; 1 GiB copy and read"}, "per_case": out}


def workload_c1(device):
    """The pages' small fp32 example (X 16x1024 with input channel 50 at 100,
    W 2048x1024, alpha 0.5, calibrated on X itself): latency of the whole path
    (calibration absmax of X, weight absmax, smoothing factors, weight codes,
    activation codes, int8 GEMM with fp32 output; six launches), eager and
    replayed from a HIP graph, each checked bit for bit against the oracle;
    beside it the oracle's time for the same pass on all host cores and on
    one. Medians over repeated passes."""
    import os as _os
    import statistics
    import numpy as np
    import torch
    from oracle.oracle import Oracle
    from w8a8_post_quantization_channel_amd import capi, synth
    xh, wh = synth.c1()
    n, k = wh.shape
    m = xh.shape[0]
    x, w = torch.from_numpy(xh).to(device), torch.from_numpy(wh).to(device)
    f32 = dict(dtype=torch.float32, device=device)
    act_max, w_max = torch.empty(k, **f32), torch.empty(k, **f32)
    s, inv_s, a = torch.empty(k, **f32), torch.empty(k, **f32), torch.empty(4, **f32)
    wq, ws = torch.empty((n, k), dtype=torch.int8, device=device), torch.empty(n, **f32)
    xq, y = torch.empty((m, k), dtype=torch.int8, device=device), torch.empty((m, n), **f32)

    def path():
        capi.sq_calib_absmax(x, act_max, False)
        capi.sq_calib_absmax(w, w_max, False)
        capi.sq_smooth_factors(act_max, w_max, 0.5, s, inv_s, a)
        capi.sq_quant_weight(w, s, wq, ws)
        capi.sq_smooth_quant_act(x, inv_s, a, xq)
        capi.sq_w8a8_gemm(xq, wq, a, ws, y)

    o = Oracle()
    ref = o.layer_forward([xh], wh, xh, 0.5, bf16_out=False)["y"]

    def check(what):
        torch.cuda.synchronize()
        if not np.array_equal(y.cpu().numpy(), ref):
            raise RuntimeError(f"C1 output differs from the oracle ({what})")

    path()
    check("eager")

    def per_pass(fn, reps=300):
        wall, gpu = [], []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            wall.append((time.perf_counter() - t0) * 1e6)
            gpu.append(e0.elapsed_time(e1) * 1e3)
        return statistics.median(wall), statistics.median(gpu)

    for _ in range(50):
        path()
    eager_wall, eager_gpu = per_pass(path)
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        path()
    for rep in range(3):  # every replay checked, eager work between replays
        y.zero_()
        graph.replay()
        check(f"graph replay {rep}")
        path()
        check(f"eager after replay {rep}")
    graph_wall, graph_gpu = per_pass(graph.replay)
    check("after timed replays")

    def oracle_us(threads, reps=7):
        o.set_num_threads(threads)
        t = []
        for _ in range(reps):
            t0 = time.perf_counter()
            o.layer_forward([xh], wh, xh, 0.5, bf16_out=False)
            t.append((time.perf_counter() - t0) * 1e6)
        return statistics.median(t)

    cores = len(_os.sched_getaffinity(0))
    cpu_all = oracle_us(min(cores, 16))
    cpu_one = oracle_us(1)
    o.set_num_threads(min(cores, 16))
    return {"metric": "C1 (16x1024 -> 2048, fp32) whole-path latency, HIP-graph replay", "value": graph_wall,
            "unit": "us", "n_gpus": 1, "higher_is_better": False, "dtype": "fp32 in/out, int8 codes",
            "data": "synthetic (the pages' example shapes: N(0,1)*5, channel 50 = 100; W N(0,1); seed 101)",
            "config": {"workload": "C1 single fp32 layer, 6 launches per pass", "m": m, "n": n, "k": k},
            "graph_replay_us": {"host_wall": graph_wall, "gpu_events": graph_gpu},
            "eager_us": {"host_wall": eager_wall, "gpu_events": eager_gpu},
            "oracle_us": {"threads": min(cores, 16), "all_threads": cpu_all, "one_thread": cpu_one,
                          "cpu_model": cpu_model()},
            "check": "output bit-identical to the oracle (eager, each graph replay)"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def workload_variants(device):
    """The widened rows, each beside the form it replaces:
    - dynamic vs static activation scale: the runtime forward (activation
      quantization + GEMM) of the seven 13B projections at 2048 tokens;
    - 1/s folded into the RMSNorm weight: one fused norm + quantizer pass
      against RMSNorm (bf16 out) followed by the activation quantizer, at the
      13B (2048 x 5120) and 70B (4096 x 8192) norm shapes;
    - averaged per-sample maxima and the 99.9% nearest-rank percentile
      against the plain running maximum over the 13B calibration set
      (512 samples x 512 tokens x 5120)."""
    import torch
    from w8a8_post_quantization_channel_amd import capi, synth
    from w8a8_post_quantization_channel_amd.layer import forward_block, forward_block_dynamic
    out = {}
    groups, projs = setup(device)
    for _ in range(2):
        run_step(groups, projs)  # calibrate + prepare every projection
    torch.cuda.synchronize()
    static_ms = timed(lambda: [layer.forward(g.x) for _, g, layer, _ in projs], 20)
    dynamic_ms = timed(lambda: [layer.forward_dynamic(g.x) for _, g, layer, _ in projs], 20)
    layers = [layer for _, _, layer, _ in projs]
    xs = [g.x for _, g, _, _ in projs]
    static_b_ms = timed(lambda: forward_block(layers, xs), 50, warmup=10)
    dynamic_b_ms = timed(lambda: forward_block_dynamic(layers, xs), 50, warmup=10)
    step_ms = timed(lambda: run_step(groups, projs), 20)
    out["dynamic_scale_13b"] = {
        "static_forward_us": static_ms * 1e3, "dynamic_forward_us": dynamic_ms * 1e3,
        "overhead_vs_static_forward": dynamic_ms / static_ms - 1.0,
        "overhead_vs_whole_step": (dynamic_ms - static_ms) / step_ms,
        "forward": "7 projections: activation quantization + int8 GEMM, 2048 tokens, one projection at a time",
        "batched": {"static_forward_us": static_b_ms * 1e3, "dynamic_forward_us": dynamic_b_ms * 1e3,
                    "overhead_vs_static_forward": dynamic_b_ms / static_b_ms - 1.0,
                    "overhead_vs_whole_step": (dynamic_b_ms - static_b_ms) / step_ms,
                    "forward": "the block in few launches: static = batched codes + grouped GEMM; dynamic = "
                               "batched live statistics of the 4 inputs + batched act scales + the same"}}
    del groups, projs
    torch.cuda.empty_cache()

    for name, m, k in (("13b", 2048, 5120), ("70b", 4096, 8192)):
        h = synth.device_activations(4100 + k, m, k, synth.outlier_channels(4000 + k, k), device)
        g = torch.rand(k, device=device) + 0.5
        inv_s = torch.rand(k, device=device) + 0.25
        gf = torch.empty(k, dtype=torch.float32, device=device)
        capi.sq_fold_norm_weight(g, inv_s, gf)
        a = torch.full((4,), 0.05, device=device)
        y = torch.empty((m, k), dtype=torch.bfloat16, device=device)
        xq = torch.empty((m, k), dtype=torch.int8, device=device)
        fused_ms = timed(lambda: capi.sq_rmsnorm_quant_act(h, gf, 1e-5, a, xq), 50)
        norm_ms = timed(lambda: capi.sq_rmsnorm(h, g, 1e-5, y), 50)
        quant_ms = timed(lambda: capi.sq_smooth_quant_act(y, inv_s, a, xq), 50)
        byts = m * k * 3 + k * 4
        out[f"norm_fold_{name}_{m}x{k}"] = {
            "fused_us": fused_ms * 1e3, "unfused_norm_us": norm_ms * 1e3, "unfused_quant_us": quant_ms * 1e3,
            "speedup": (norm_ms + quant_ms) / fused_ms, "fused_GB/s": byts / (fused_ms * 1e-3) / 1e9,
            "fused_hbm_frac": byts / (fused_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "bytes_per_element": {"fused": 3, "unfused": 7}}
        # the norm's consumers as in a block (13B attention norm: q, k, v; 70B
        # MLP norm: gate, up), each with its own folded weight and act scale:
        # one fused pass per consumer against one pass writing every
        # consumer's codes, and against RMSNorm then the batched quantizer
        n = 3 if name == "13b" else 2
        gfs = [gf] + [torch.empty(k, dtype=torch.float32, device=device) for _ in range(n - 1)]
        invs = [inv_s] + [torch.rand(k, device=device) + 0.25 for _ in range(n - 1)]
        for i in range(1, n):
            capi.sq_fold_norm_weight(g, invs[i], gfs[i])
        acs = [torch.full((4,), 0.05 + 0.01 * i, device=device) for i in range(n)]
        xqs = [torch.empty((m, k), dtype=torch.int8, device=device) for _ in range(n)]
        per_ms = timed(lambda: [capi.sq_rmsnorm_quant_act(h, gfs[i], 1e-5, acs[i], xqs[i]) for i in range(n)], 50)
        multi_ms = timed(lambda: capi.sq_rmsnorm_quant_act_multi(h, gfs, 1e-5, acs, xqs), 50)
        unf_ms = timed(lambda: (capi.sq_rmsnorm(h, g, 1e-5, y),
                                capi.sq_smooth_quant_act_batched([y] * n, invs, acs, xqs)), 50)
        mbytes = m * k * (2 + n) + n * k * 4
        out[f"norm_fold_{name}_{m}x{k}"]["consumers"] = {
            "n": n, "one_pass_us": multi_ms * 1e3, "pass_per_consumer_us": per_ms * 1e3,
            "norm_then_batched_quant_us": unf_ms * 1e3, "one_pass_GB/s": mbytes / (multi_ms * 1e-3) / 1e9,
            "one_pass_hbm_frac": mbytes / (multi_ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
        del h, y, xq, xqs
        torch.cuda.empty_cache()

    samples, rows, k = 512, 512, 5120
    x = synth.device_activations(4200, samples * rows, k, synth.outlier_channels(4201, k), device)
    smax = torch.empty((samples, k), dtype=torch.float32, device=device)
    total = torch.zeros(k, dtype=torch.float64, device=device)
    am = torch.empty(k, dtype=torch.float32, device=device)
    mean_ms = timed(lambda: capi.sq_calib_sample_max_sum(x, samples, smax, total), 5)
    max_ms = timed(lambda: capi.sq_calib_absmax(x, am, False), 5)
    byts = x.numel() * 2 + samples * k * 4
    out["calib_mean_of_max_262144x5120"] = {
        "us": mean_ms * 1e3, "GB/s": byts / (mean_ms * 1e-3) / 1e9,
        "hbm_frac": byts / (mean_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "plain_max_us": max_ms * 1e3}
    ws = torch.empty(capi.sq_calib_percentile_workspace(k, capi.SQ_BF16), dtype=torch.uint8, device=device)
    pct_ms = timed(lambda: capi.sq_calib_percentile(x, 0.999, ws, am), 3)
    byts = x.numel() * 2
    out["calib_percentile_99.9_262144x5120"] = {
        "us": pct_ms * 1e3, "passes_over_x": 2, "GB/s_per_pass": 2 * byts / (pct_ms * 1e-3) / 1e9,
        "hbm_frac_per_pass": 2 * byts / (pct_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "plain_max_us": max_ms * 1e3}
    return {"metric": "widened rows beside the forms they replace (time, GB/s)",
            "value": out["norm_fold_70b_4096x8192"]["fused_GB/s"], "unit": "GB/s (fused norm + quantizer, 70B shape)",
            "n_gpus": 1, "higher_is_better": True, "dtype": "bf16->int8", "data": "synthetic",
            "config": {"workload": "dynamic scale (13B forward), RMSNorm fold (13B/70B norm shapes), "
                                   "mean of per-sample maxima and 99.9% percentile (13B calibration set)"},
            "per_row": out}


def workload_fp8(device):
    """The FP8 (OCP E4M3) variant on the 13B layer (2048 tokens, 7 projections):
    the whole step with e4m3 codes (statistics, smoothing, FP8 weight and
    activation quantization, FP8 GEMM) and each projection's FP8 GEMM beside
    the int8 GEMM on the same shape (both dense 5.0 P/s peaks on MI355X)."""
    import torch
    from w8a8_post_quantization_channel_amd import capi
    groups, projs = setup(device)
    for _ in range(2):
        run_step(groups, projs)
    torch.cuda.synchronize()
    m = next(iter(groups.values())).x.shape[0]
    f8 = []
    for name, g, layer, _ in projs:
        a8 = torch.empty(4, dtype=torch.float32, device=device)
        wq8 = torch.empty((layer.n, layer.k), dtype=torch.uint8, device=device)
        ws8 = torch.empty(layer.n, dtype=torch.float32, device=device)
        xq8 = torch.empty((m, layer.k), dtype=torch.uint8, device=device)
        f8.append((name, g, layer, a8, wq8, ws8, xq8))

    def fp8_step():
        for g in groups.values():
            capi.sq_calib_absmax(g.x, g.act_max, False)
        for name, g, layer, a8, wq8, ws8, xq8 in f8:
            capi.sq_calib_absmax(layer.w, layer.w_max, False)
            capi.sq_smooth_factors(layer.act_max, layer.w_max, layer.alpha, layer.s, layer.inv_s, layer.act_scale)
            capi.sq_act_scale_fp8(layer.act_max, layer.inv_s, a8)
            capi.sq_quant_weight_fp8(layer.w, layer.s, wq8, ws8)
            capi.sq_smooth_quant_act_fp8(g.x, layer.inv_s, a8, xq8)
            capi.sq_fp8_gemm(xq8, wq8, a8, ws8, layer.y[:m])

    ys8 = [torch.empty((m, layer.n), dtype=torch.bfloat16, device=device) for _, _, layer, *_ in f8]

    def fp8_step_batched():
        """The same step through the batched FP8 entry points, on the int8
        step's schedule: one statistics launch, batched smoothing and codes,
        one grouped FP8 GEMM with the products issued newest-first."""
        layers = [layer for _, _, layer, *_ in f8]
        stats = [(g.x, g.act_max) for g in groups.values()] + [(l.w, l.w_max) for l in layers]
        capi.sq_calib_absmax_batched([x for x, _ in stats], [a for _, a in stats], False)
        capi.sq_smooth_factors_fp8_batched([l.act_max for l in layers], [l.w_max for l in layers],
                                           [l.alpha for l in layers], [l.s for l in layers],
                                           [l.inv_s for l in layers], [e[3] for e in f8])
        capi.sq_quant_weight_fp8_batched([l.w for l in layers], [l.s for l in layers], [e[4] for e in f8],
                                         [e[5] for e in f8])
        capi.sq_smooth_quant_act_fp8_batched([e[1].x for e in f8], [l.inv_s for l in layers], [e[3] for e in f8],
                                             [e[6] for e in f8])
        r = list(range(len(f8)))[::-1]
        capi.sq_fp8_gemm_batched([f8[i][6] for i in r], [f8[i][4] for i in r], [f8[i][3] for i in r],
                                 [f8[i][5] for i in r], [ys8[i] for i in r])

    fp8_step()
    fp8_step_batched()
    torch.cuda.synchronize()
    for (name, _, layer, *_), y in zip(f8, ys8):  # the two schedules compute the same outputs
        if not torch.equal(y.view(torch.int16), layer.y[:m].view(torch.int16)):
            raise RuntimeError(f"batched FP8 step differs from the per-projection one ({name})")
    # each step kind gets 30 untimed steps first: the first steps after the
    # other kind touched its own gigabyte of buffers run well above steady state
    step8_ms = timed(fp8_step, 50, warmup=30)
    step8_batched_ms = timed(fp8_step_batched, 50, warmup=30)
    step_i8_ms = timed(lambda: run_step(groups, projs, batched=False), 50, warmup=30)
    step_i8_batched_ms = timed(lambda: run_step(groups, projs), 50, warmup=30)
    per = {}
    ops_total = 0.0
    for name, g, layer, a8, wq8, ws8, xq8 in f8:
        ops = 2.0 * m * layer.n * layer.k
        ops_total += ops
        xq = layer.quantize_input(g.x)
        t8 = timed(lambda: capi.sq_fp8_gemm(xq8, wq8, a8, ws8, layer.y[:m]), 50)
        ti8 = timed(lambda: layer.matmul(xq), 50)
        per[name] = {"fp8_gemm_tops": ops / (t8 * 1e-3) / 1e12, "int8_gemm_tops": ops / (ti8 * 1e-3) / 1e12,
                     "shape": [m, layer.n, layer.k]}
    gemm8 = sum(2.0 * m * l.n * l.k / (per[n]["fp8_gemm_tops"] * 1e12) for n, _, l, *_ in f8)
    return {"metric": "W8A8 FP8 (E4M3) step TOPS at 13B shapes", "value": ops_total / (step8_batched_ms * 1e-3) / 1e12,
            "unit": "TOPS", "n_gpus": 1, "higher_is_better": True, "dtype": "fp8_e4m3", "data": "synthetic",
            "config": {"workload": "llama2-13b decoder layer, 7 projections, 2048 prefill tokens, FP8 E4M3 codes"},
            "step_batched_ms": step8_batched_ms, "step_per_projection_ms": step8_ms,
            "int8_step_ms": step_i8_ms, "int8_step_batched_ms": step_i8_batched_ms,
            "note": "value: the FP8 step through the batched entry points (the int8 default line's schedule); "
                    "step_per_projection_ms the FP8 step projection by projection, int8_step_ms the int8 step on "
                    "that schedule, int8_step_batched_ms the int8 step with the batched entry points",
            "fp8_gemm_tops_all": ops_total / gemm8 / 1e12,
            "fp8_gemm_frac_of_peak": ops_total / gemm8 / 1e12 / PEAK_INT8_TOPS,
            "per_projection": per}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print("bench.py: runs on one GPU only; --gpus above 1 is not supported (the kernels run one GPU's "
              "share of the work; sharding across GPUs is not implemented)", file=sys.stderr)
        sys.exit(2)
    import torch
    from w8a8_post_quantization_channel_amd import capi
    capi.load()  # fails loudly when libsq.so is missing
    device = torch.device("cuda", 0)
    other = {"decode7b": workload_decode7b, "alpha_search": workload_alpha_search, "copy_probe": workload_copy_probe,
             "prefill70b": workload_prefill70b, "hbm_passes": workload_hbm_passes, "variants": workload_variants,
             "ceilings": workload_ceilings, "c1": workload_c1,
             "fp8": workload_fp8}
    if args.workload in other:
        out = other[args.workload](device)
        out["gpu"] = torch.cuda.get_device_name(0)
        print(json.dumps(out), flush=True)
        return
    groups, projs = setup(device, args.scales)
    m = next(iter(groups.values())).x.shape[0]
    side = torch.cuda.Stream() if args.overlap else None  # default priority, like the main stream

    batched = not args.per_projection
    if args.overlap:
        if not batched:
            raise SystemExit("--overlap runs the batched entry points; drop --per-projection")
        block = phased_block(groups, projs)

        def one_step(ev=None):
            run_phased(block, side, ev)
    else:
        def one_step(ev=None):
            run_step(groups, projs, ev, batched=batched)
    ramp_steps = 0
    t_ramp = time.perf_counter()
    while time.perf_counter() - t_ramp < args.ramp_seconds:
        for _ in range(10):
            one_step()
        torch.cuda.synchronize()
        ramp_steps += 10
    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()

    events = []
    every = max(1, args.event_every)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        one_step(events if i % every == 0 else None)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    ms_per_step = elapsed * 1e3 / args.steps
    ops = gemm_ops(projs, m)
    value = ops / (elapsed / args.steps) / 1e12

    # dominant kernel: the GEMM, averaged over every bracketed launch in the
    # timed steps (batched: one grouped launch per step for all projections)
    gemm_ms = [e0.elapsed_time(e1) for _, e0, e1 in events]
    by_name = {}
    for (name, _, _), t in zip(events, gemm_ms):
        by_name.setdefault(name, []).append(t)
    ops_by_name = {name: 2.0 * m * layer.n * layer.k for name, _, layer, _ in projs}
    ops_by_name["block"] = ops
    for tag, names in zip(("attn", "mlp"), PHASES):
        ops_by_name[tag] = sum(ops_by_name[n] for n in names)
    avg_launch_ms = sum(gemm_ms) / len(gemm_ms)
    avg_launch_ops = sum(ops_by_name[n] for n, _, _ in events) / len(events)
    achieved = avg_launch_ops / (avg_launch_ms * 1e-3) / 1e12
    traffic = gemm_traffic(args.traffic)
    roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_INT8_TOPS, "unit": "TOPS",
                "frac": achieved / PEAK_INT8_TOPS, "traffic": traffic,
                "kernel": "gemm_dma_kernel<OpI8, TN, EpiDequant<bf16>> (256 x 32*TN tiles), one launch per "
                          "projection" if args.per_projection else
                          "gemm_dma_grouped_kernel<OpI8, TN, bf16> (256 x 32*TN tiles), one launch per phase "
                          "(q, k, v, o; gate, up, down), beside the other phase's preparation" if args.overlap else
                          "gemm_dma_grouped_kernel<OpI8, TN, bf16> (256 x 32*TN tiles), one launch for the 7 "
                          "projections",
                "scale_storage": args.scales,
                "tiling": ({n: list(capi.sq_gemm_tiling(m, layer.n)) for n, _, layer, _ in projs}
                           if args.per_projection else block_tiling(m, projs, args.overlap)),
                "avg_launch_us": avg_launch_ms * 1e3,
                "per_projection_tops": {n: ops_by_name[n] / (sum(v) / len(v) * 1e-3) / 1e12
                                        for n, v in by_name.items()}}
    sampled_steps = (args.steps + every - 1) // every
    gemm_share = sum(gemm_ms) / sampled_steps / ms_per_step

    out = {
        "metric": METRIC, "value": value, "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8",
        "data": "synthetic (seeded numpy draws: N(0,1) activations, 0.3% outlier channels x U(20,100); "
                "N(0,0.02) weights; bf16)",
        "config": {"workload": "llama2-13b decoder layer, 7 linear projections, 2048 prefill tokens",
                   "tokens": m, "alpha": 0.5, "in_dtype": "bf16", "out_dtype": "bf16",
                   "scale_storage": "fp16 (every scale)" if args.scales == "f16" else "fp32",
                   "projections": {n: [layer.n, layer.k] for n, _, layer, _ in projs},
                   "step": "calib absmax + weight absmax + smoothing + weight quant + act quant + int8 GEMM",
                   "preparation": "per projection" if args.per_projection else
                   "batched over the 7 projections (statistics, smoothing, weight codes)",
                   "schedule": "two streams, two phases (q, k, v, o; gate, up, down): a phase's grouped GEMM "
                   "runs beside the other phase's preparation" if args.overlap else "one stream"},
        "roofline": roofline,
        "ramp_steps": ramp_steps,
        "gemm_events": f"every {every}th timed step ({len(events)} GEMM launches bracketed)",
        "gemm_share_of_step": gemm_share,
        "gpu": torch.cuda.get_device_name(0),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(groups, projs, args.cpu_rows, scales=args.scales)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
