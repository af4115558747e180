"""GPU parity of the batched entry points (several projections per call)
against the CPU oracle item by item, and against the single-call path on the
seven projections of a Llama-2-13B block. Bar: bit-exact (statistics, smoothing
factors, scales and int8 codes are all exact or single-rounded values)."""
from __future__ import annotations

import numpy as np
import pytest

from oracle.oracle import Oracle
from tests.gpu_pipeline import assert_bitexact, dev
from w8a8_post_quantization_channel_amd import capi, synth

pytestmark = pytest.mark.gpu
ORACLE = Oracle()


@pytest.fixture(scope="module", autouse=True)
def _lib():
    capi.load()


def _t(a):
    return synth.to_torch(a, dev())


def _h(t):
    return synth.from_torch(t)


# (rows, k, bf16): mixed element types, a zero-row item, ragged rows, K from 64 to 13824
ABS_ITEMS = [(300, 1088, True), (0, 256, True), (2048, 5120, True), (7, 64, False), (513, 13824, True),
             (96, 320, False), (1, 4096, True)]


@pytest.mark.parametrize("accumulate", [False, True])
def test_absmax_batched(accumulate):
    import torch
    xs = [synth.activations(4000 + i, r, k, synth.outlier_channels(4100 + i, k), bf16=b)
          for i, (r, k, b) in enumerate(ABS_ITEMS)]
    g = synth.rng(4200)
    prev = [g.uniform(0.0, 3.0, k).astype(np.float32) for _, k, _ in ABS_ITEMS]
    outs = [_t(p) if accumulate else torch.full((k,), 9.0, dtype=torch.float32, device=dev())
            for p, (_, k, _) in zip(prev, ABS_ITEMS)]
    capi.sq_calib_absmax_batched([_t(x) for x in xs], outs, accumulate)
    torch.cuda.synchronize()
    for i, (x, o) in enumerate(zip(xs, outs)):
        ref = ORACLE.calib_absmax(x, prev[i].copy() if accumulate else None)
        assert_bitexact(f"absmax item {i}", _h(o), ref)


# (k, alpha): q, k and v share one statistic; a K of 64 and one of 13824
SMOOTH_ITEMS = [(5120, 0.5, 0), (5120, 0.75, 0), (5120, 0.25, 0), (64, 1.0, 1), (13824, 0.5, 2), (1088, 0.0, 3)]


def test_smooth_factors_batched():
    import torch
    g = synth.rng(4300)
    stats = {}
    for k, _, grp in SMOOTH_ITEMS:
        if grp not in stats:
            am = g.uniform(0.01, 60.0, k).astype(np.float32)
            am[g.integers(0, k, 3)] = 0.0  # floored channels
            stats[grp] = am
    act_max = {grp: _t(v) for grp, v in stats.items()}
    w_max = [g.uniform(0.001, 2.0, k).astype(np.float32) for k, _, _ in SMOOTH_ITEMS]
    f32 = dict(dtype=torch.float32, device=dev())
    ss = [torch.empty(k, **f32) for k, _, _ in SMOOTH_ITEMS]
    inv = [torch.empty(k, **f32) for k, _, _ in SMOOTH_ITEMS]
    sc = [torch.empty(4, **f32) for _ in SMOOTH_ITEMS]
    capi.sq_smooth_factors_batched([act_max[grp] for _, _, grp in SMOOTH_ITEMS], [_t(w) for w in w_max],
                                   [a for _, a, _ in SMOOTH_ITEMS], ss, inv, sc)
    torch.cuda.synchronize()
    for i, (k, alpha, grp) in enumerate(SMOOTH_ITEMS):
        rs, ri, ra = ORACLE.smooth_factors(stats[grp], w_max[i], alpha)
        assert_bitexact(f"s item {i}", _h(ss[i]), rs)
        assert_bitexact(f"inv_s item {i}", _h(inv[i]), ri)
        assert_bitexact(f"act_scale item {i}", _h(sc[i])[:1], np.array([ra], np.float32))


# (n, k, bf16): every row-length class of the stream kernel (rows of 64 .. 65536 bf16
# values), the long-row kernel, several items per class in one launch, ragged row counts
QW_ITEMS = [(37, 1024, True), (300, 5120, True), (5, 5120, True), (129, 13824, True), (8, 2048, False),
            (33, 4096, True), (3, 10240, False), (2, 16384, True), (17, 32768, True), (3, 70016, True),
            (1, 64, True), (64, 1088, True), (9, 640, False), (11, 8192, True), (7, 11008, True),
            (5, 12288, True)]


def test_quant_weight_batched():
    import torch
    ws, ss = [], []
    for i, (n, k, b) in enumerate(QW_ITEMS):
        w = synth.weights(4400 + i, n, k, std=1.0, bf16=False)
        w[0, min(7, k - 1)] = 300.0  # a large element in the first row
        if n > 2:
            w[n - 1] = 0.0  # a zero row (scale at the floor)
        ws.append(synth.to_bf16_bits(w) if b else w)
        ss.append(synth.rng(4500 + i).uniform(0.1, 10.0, k).astype(np.float32))
    wqs = [torch.empty((n, k), dtype=torch.int8, device=dev()) for n, k, _ in QW_ITEMS]
    wsc = [torch.empty(n, dtype=torch.float32, device=dev()) for n, _, _ in QW_ITEMS]
    capi.sq_quant_weight_batched([_t(w) for w in ws], [_t(s) for s in ss], wqs, wsc)
    torch.cuda.synchronize()
    for i in range(len(QW_ITEMS)):
        rq, rs = ORACLE.quant_weight(ws[i], ss[i])
        assert_bitexact(f"wq item {i}", _h(wqs[i]), rq)
        assert_bitexact(f"w_scale item {i}", _h(wsc[i]), rs)


def test_block_prepare_batched_equals_single_calls():
    """The 13B block's statistics, smoothing factors and weight codes from the
    batched calls equal those of one single-form call per projection."""
    import torch
    f32 = dict(dtype=torch.float32, device=dev())
    groups = {g: _t(synth.c2_group_x(g, rows=512)) for g in synth.C2_GROUPS}
    projs = [(p, g, _t(synth.c2_projection_w(p))) for p, g, *_ in synth.C2_PROJECTIONS]

    def buffers():
        am = {g: torch.empty(x.shape[1], **f32) for g, x in groups.items()}
        per = []
        for _, g, w in projs:
            n, k = w.shape
            per.append(dict(w_max=torch.empty(k, **f32), s=torch.empty(k, **f32), inv_s=torch.empty(k, **f32),
                            a=torch.empty(4, **f32), wq=torch.empty((n, k), dtype=torch.int8, device=dev()),
                            ws=torch.empty(n, **f32)))
        return am, per

    am1, per1 = buffers()
    for g, x in groups.items():
        capi.sq_calib_absmax(x, am1[g])
    for (_, g, w), b in zip(projs, per1):
        capi.sq_calib_absmax(w, b["w_max"])
        capi.sq_smooth_factors(am1[g], b["w_max"], 0.5, b["s"], b["inv_s"], b["a"])
        capi.sq_quant_weight(w, b["s"], b["wq"], b["ws"])

    am2, per2 = buffers()
    gl = list(groups)
    capi.sq_calib_absmax_batched([groups[g] for g in gl] + [w for _, _, w in projs],
                                 [am2[g] for g in gl] + [b["w_max"] for b in per2])
    capi.sq_smooth_factors_batched([am2[g] for _, g, _ in projs], [b["w_max"] for b in per2], [0.5] * len(projs),
                                   [b["s"] for b in per2], [b["inv_s"] for b in per2], [b["a"] for b in per2])
    capi.sq_quant_weight_batched([w for _, _, w in projs], [b["s"] for b in per2], [b["wq"] for b in per2],
                                 [b["ws"] for b in per2])
    torch.cuda.synchronize()
    for g in gl:
        assert torch.equal(am1[g], am2[g]), g
    for (p, _, _), b1, b2 in zip(projs, per1, per2):
        for key in ("w_max", "s", "inv_s", "wq", "ws"):
            assert torch.equal(b1[key], b2[key]), (p, key)
        assert torch.equal(b1["a"][:1], b2["a"][:1]), (p, "act_scale")


def test_quant_act_batched():
    """Inputs shared by up to five consumers (five split over two passes), mixed
    element types, an empty batch; every consumer's codes bit-exact."""
    import torch
    g = synth.rng(4600)
    xa = synth.activations(4601, 300, 1088, synth.outlier_channels(4602, 1088), bf16=True)
    xb = synth.activations(4603, 2048, 5120, synth.outlier_channels(4604, 5120), bf16=True)
    xc = synth.activations(4605, 37, 320, None, bf16=False)
    xd = synth.activations(4606, 513, 13824, synth.outlier_channels(4607, 13824), bf16=True)
    xe = np.zeros((0, 256), np.uint16)
    inputs = {"a": xa, "b": xb, "c": xc, "d": xd, "e": xe}
    dev_in = {n: (_t(v) if v.size else torch.empty((0, 256), dtype=torch.bfloat16, device=dev()))
              for n, v in inputs.items()}
    plan = ["a", "a", "a", "a", "a", "b", "b", "c", "d", "e", "b"]  # five consumers of a, three of b
    inv_s, scales, outs = [], [], []
    for i, name in enumerate(plan):
        x = inputs[name]
        k = x.shape[1]
        inv = g.uniform(0.02, 3.0, k).astype(np.float32)
        xf = synth.bf16_bits_to_f32(x) if x.dtype == np.uint16 else x
        a = np.float32(0.7 * np.abs(xf * inv).max() / 127.0) if x.size else np.float32(0.01)  # some saturation
        inv_s.append(inv)
        scales.append(np.array([a, 0, 0, 0], np.float32))
        outs.append(torch.full(x.shape, 3, dtype=torch.int8, device=dev()))
    capi.sq_smooth_quant_act_batched([dev_in[n] for n in plan], [_t(v) for v in inv_s], [_t(v) for v in scales],
                                     outs)
    torch.cuda.synchronize()
    for i, name in enumerate(plan):
        x = inputs[name]
        if not x.size:
            assert outs[i].numel() == 0
            continue
        assert_bitexact(f"xq item {i} ({name})", _h(outs[i]), ORACLE.quant_act(x, inv_s[i], scales[i][0]))


def test_gemm_batched():
    """Products that take the pipelined tiles (with single-call widths of 128
    and 160; each output type's group runs at one width chosen for the group),
    a skinny (m <= 64), a vector-ALU (m <= 4) and a register-staged one, mixed
    output types, some with the int32 accumulator: every output bit-exact
    against the oracle."""
    import torch
    cases = [(512, 5120, 192, True, True), (300, 5120, 320, False, False), (1024, 8192, 128, True, False),
             (40, 1000, 704, True, True), (200, 600, 256, False, True), (256, 4112, 64, True, False),
             (0, 512, 64, True, False), (2048, 5120, 64, True, True), (3, 1003, 4160, False, True)]
    tilings = {capi.sq_gemm_tiling(m, n) for m, n, *_ in cases if m}
    assert {(256, 128), (256, 160), (64, 16), (4, 4)} <= tilings, tilings
    g = synth.rng(4700)
    xqs, wqs, scs, wss, ys, accs, host = [], [], [], [], [], [], []
    for m, n, k, bf16, with_acc in cases:
        xq = g.integers(-127, 128, (m, k), dtype=np.int8)
        wq = g.integers(-127, 128, (n, k), dtype=np.int8)
        ws = g.uniform(1e-4, 1e-2, n).astype(np.float32)
        a = np.array([g.uniform(0.005, 0.05), 0, 0, 0], np.float32)
        host.append((xq, wq, ws, a))
        xqs.append(_t(xq) if m else torch.empty((0, k), dtype=torch.int8, device=dev()))
        wqs.append(_t(wq))
        scs.append(_t(a))
        wss.append(_t(ws))
        ys.append(torch.empty((m, n), dtype=torch.bfloat16 if bf16 else torch.float32, device=dev()))
        accs.append(torch.empty((m, n), dtype=torch.int32, device=dev()) if with_acc else None)
    capi.sq_w8a8_gemm_batched(xqs, wqs, scs, wss, ys, accs)
    torch.cuda.synchronize()
    for i, ((m, n, k, bf16, with_acc), (xq, wq, ws, a)) in enumerate(zip(cases, host)):
        if not m:
            continue
        racc = ORACLE.gemm_i32(xq, wq)
        if with_acc:
            assert_bitexact(f"acc item {i}", _h(accs[i]), racc)
        assert_bitexact(f"y item {i}", _h(ys[i]), ORACLE.dequant(racc, a[0], ws, bf16=bf16))


def test_gemm_grouped_split_rings():
    """One grouped launch whose first products run on 256 x 256 tiles (split
    LDS rings: the weight panel three stages deep, the activation panel two)
    and whose last products on 256 x 128 (the kernel's second width, which
    evens out the last round), as the library chooses for this group: ragged
    m and n in every product, K of 1.5 to 5.5 steps of 128 bytes (a half last
    step in each), some items with the int32 accumulator; every output
    bit-exact against the oracle."""
    import torch
    cases = [(1900, 5000, 320, True), (1900, 13800, 192, False), (1900, 13800, 448, True), (700, 5000, 704, False)]
    tiles = capi.sq_gemm_batched_tiling([(m, n, k) for m, n, k, _ in cases])
    assert tiles[0] == (256, 256) and (256, 128) in tiles, tiles
    g = synth.rng(4810)
    xqs, wqs, scs, wss, ys, accs, host = [], [], [], [], [], [], []
    for m, n, k, with_acc in cases:
        xq = g.integers(-127, 128, (m, k), dtype=np.int8)
        wq = g.integers(-127, 128, (n, k), dtype=np.int8)
        ws = g.uniform(1e-4, 1e-2, n).astype(np.float32)
        a = np.array([g.uniform(0.005, 0.05), 0, 0, 0], np.float32)
        host.append((xq, wq, ws, a))
        xqs.append(_t(xq))
        wqs.append(_t(wq))
        scs.append(_t(a))
        wss.append(_t(ws))
        ys.append(torch.empty((m, n), dtype=torch.bfloat16, device=dev()))
        accs.append(torch.empty((m, n), dtype=torch.int32, device=dev()) if with_acc else None)
    capi.sq_w8a8_gemm_batched(xqs, wqs, scs, wss, ys, accs)
    torch.cuda.synchronize()
    for i, ((m, n, k, with_acc), (xq, wq, ws, a)) in enumerate(zip(cases, host)):
        racc = ORACLE.gemm_i32(xq, wq)
        if with_acc:
            assert_bitexact(f"acc item {i}", _h(accs[i]), racc)
        assert_bitexact(f"y item {i}", _h(ys[i]), ORACLE.dequant(racc, a[0], ws, bf16=True))


@pytest.mark.parametrize("f16", [False, True])
def test_gemm_batched_decode_grouped(f16):
    """Decode-sized products in one batched call: those with m <= 4 and the
    same activation-row class, chunks in flight, output type and scale storage
    share a vector-ALU launch (q, k, v of a decode step; ragged n; K from 64 to
    20480, which spans the chunk classes); those with 4 < m <= 64 and the same
    skinny configuration share a skinny launch. Every output and accumulator
    bit-exact against the oracle and against the single calls."""
    import torch
    cases = [(1, 4096, 4096, True, False), (1, 4096, 4096, True, True), (1, 4096, 4096, True, False),
             (1, 1003, 4096, True, True), (2, 512, 4160, False, True), (3, 600, 11008, True, False),
             (4, 260, 11008, True, True), (1, 256, 64, False, False), (4, 130, 20480, True, True),
             (2, 77, 192, True, False),
             # 4 < m <= 64: the skinny kernel, grouped by configuration (ragged n and m)
             (8, 4096, 4096, True, False), (8, 4096, 4096, True, True), (5, 1003, 4096, True, False),
             (16, 600, 4160, False, True), (13, 8200, 1088, True, False), (40, 1000, 704, True, True),
             (64, 9000, 448, True, True), (33, 8200, 320, True, False), (24, 200, 11008, False, False)]
    g = synth.rng(4750 + int(f16))
    xqs, wqs, scs, wss, ys, accs, host = [], [], [], [], [], [], []
    for m, n, k, bf16, with_acc in cases:
        xq = g.integers(-127, 128, (m, k), dtype=np.int8)
        wq = g.integers(-127, 128, (n, k), dtype=np.int8)
        ws = g.uniform(1e-4, 1e-2, n).astype(np.float32)
        a = np.float32(g.uniform(0.005, 0.05))
        if f16:
            ws16 = ORACLE.f16_encode(ws)
            a16 = np.array([ORACLE.scale_f16(a), 0, 0, 0, 0, 0, 0, 0], np.uint16)
            host.append((xq, wq, ws16, a16))
            scs.append(_t(a16.view(np.float16)))
            wss.append(_t(ws16.view(np.float16)))
        else:
            host.append((xq, wq, ws, np.array([a, 0, 0, 0], np.float32)))
            scs.append(_t(host[-1][3]))
            wss.append(_t(ws))
        xqs.append(_t(xq))
        wqs.append(_t(wq))
        ys.append(torch.empty((m, n), dtype=torch.bfloat16 if bf16 else torch.float32, device=dev()))
        accs.append(torch.empty((m, n), dtype=torch.int32, device=dev()) if with_acc else None)
    batched = capi.sq_w8a8_gemm_f16_batched if f16 else capi.sq_w8a8_gemm_batched
    single = capi.sq_w8a8_gemm_f16 if f16 else capi.sq_w8a8_gemm
    for lo, hi in ((0, 10), (10, len(cases))):  # the m <= 4 items, then the skinny ones (at most 16 per call)
        batched(xqs[lo:hi], wqs[lo:hi], scs[lo:hi], wss[lo:hi], ys[lo:hi], accs[lo:hi])
    torch.cuda.synchronize()
    for i, ((m, n, k, bf16, with_acc), (xq, wq, ws, a)) in enumerate(zip(cases, host)):
        racc = ORACLE.gemm_i32(xq, wq)
        if with_acc:
            assert_bitexact(f"acc item {i}", _h(accs[i]), racc)
        ref = ORACLE.dequant_h(racc, a[0], ws, bf16=bf16) if f16 else ORACLE.dequant(racc, a[0], ws, bf16=bf16)
        assert_bitexact(f"y item {i}", _h(ys[i]), ref)
        y1 = torch.empty_like(ys[i])
        single(xqs[i], wqs[i], scs[i], wss[i], y1)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int8), ys[i].view(torch.int8)), f"item {i}: batched differs from single"


def test_block_forward_batched_equals_single_calls():
    """Activation codes and outputs of the 13B block's seven projections from
    the batched quantizer and the grouped GEMM equal the single calls'."""
    import torch
    f32 = dict(dtype=torch.float32, device=dev())
    rows = 1024
    groups = {g: _t(synth.c2_group_x(g, rows=rows)) for g in synth.C2_GROUPS}
    g = synth.rng(4800)
    projs = []
    for p, grp, n, k, _ in synth.C2_PROJECTIONS:
        inv = _t(g.uniform(0.05, 2.0, k).astype(np.float32))
        a = torch.tensor([g.uniform(0.01, 0.1), 0, 0, 0], **f32)
        wq = _t(g.integers(-127, 128, (n, k), dtype=np.int8))
        ws = _t(g.uniform(1e-4, 1e-2, n).astype(np.float32))
        projs.append((p, groups[grp], inv, a, wq, ws))

    def outputs():
        return ([torch.empty((rows, x.shape[1]), dtype=torch.int8, device=dev()) for _, x, *_ in projs],
                [torch.empty((rows, wq.shape[0]), dtype=torch.bfloat16, device=dev()) for *_, wq, _ in projs])

    xq1, y1 = outputs()
    for (p, x, inv, a, wq, ws), xq, y in zip(projs, xq1, y1):
        capi.sq_smooth_quant_act(x, inv, a, xq)
        capi.sq_w8a8_gemm(xq, wq, a, ws, y)
    xq2, y2 = outputs()
    capi.sq_smooth_quant_act_batched([x for _, x, *_ in projs], [pr[2] for pr in projs], [pr[3] for pr in projs], xq2)
    capi.sq_w8a8_gemm_batched(xq2, [pr[4] for pr in projs], [pr[3] for pr in projs], [pr[5] for pr in projs], y2)
    torch.cuda.synchronize()
    for (p, *_), a1, a2, b1, b2 in zip(projs, xq1, xq2, y1, y2):
        assert torch.equal(a1, a2), (p, "xq")
        assert torch.equal(b1.view(torch.int16), b2.view(torch.int16)), (p, "y")


def test_phased_block_equals_one_stream():
    """The 13B block run as two phases on two streams (preparation of one
    phase beside the other's products, passes back to back) gives the same
    codes and outputs, bit for bit, as the one-stream block on every pass."""
    import torch
    from w8a8_post_quantization_channel_amd.layer import PhasedBlock, W8A8Linear, forward_block, prepare_block
    rows = 512
    groups = {g: _t(synth.c2_group_x(g, rows=rows)) for g in synth.C2_GROUPS}

    def make():
        layers, acts = {}, {}
        for g, x in groups.items():
            acts[g] = torch.empty(x.shape[1], dtype=torch.float32, device=dev())
        for p, g, *_ in synth.C2_PROJECTIONS:
            layer = W8A8Linear(_t(synth.c2_projection_w(p)), alpha=0.5, max_tokens=rows, out_dtype=torch.bfloat16)
            layer.act_max = acts[g]
            layers[p] = layer
        return layers, acts

    names = [p for p, *_ in synth.C2_PROJECTIONS]
    grp = {p: g for p, g, *_ in synth.C2_PROJECTIONS}
    ref_layers, ref_acts = make()
    prepare_block([ref_layers[p] for p in names], [(groups[g], ref_acts[g]) for g in groups])
    ref_y = forward_block([ref_layers[p] for p in names], [groups[grp[p]] for p in names])
    torch.cuda.synchronize()

    layers, acts = make()
    phases = []
    for part in (("q", "k", "v", "o"), ("gate", "up", "down")):
        used = sorted({grp[p] for p in part})
        phases.append(([layers[p] for p in part], [(groups[g], acts[g]) for g in used],
                       [groups[grp[p]] for p in part]))
    block = PhasedBlock(phases)
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    for rep in range(3):
        ys = block.step(side, main)
        torch.cuda.synchronize()
        for p, y, r in zip(names, ys, ref_y):
            assert torch.equal(y.view(torch.int16), r.view(torch.int16)), (rep, p)
            assert torch.equal(layers[p].wq, ref_layers[p].wq), (rep, p)
            assert torch.equal(layers[p].xq, ref_layers[p].xq), (rep, p)
    # passes enqueued back to back, synchronised only at the end
    for p in names:
        layers[p].y.zero_()
    for _ in range(4):
        ys = block.step(side, main)
    torch.cuda.synchronize()
    for p, y, r in zip(names, ys, ref_y):
        assert torch.equal(y.view(torch.int16), r.view(torch.int16)), ("back to back", p)


def test_act_scale_batched_equals_single_calls():
    import torch
    g = synth.rng(4900)
    ks = [64, 5120, 13824, 1088]
    am = [_t(g.uniform(0.0, 50.0, k).astype(np.float32)) for k in ks]
    am[0].zero_()  # an all-zero statistic takes the floor
    inv = [_t(g.uniform(0.05, 2.0, k).astype(np.float32)) for k in ks]
    one = [torch.empty(4, dtype=torch.float32, device=dev()) for _ in ks]
    two = [torch.empty(4, dtype=torch.float32, device=dev()) for _ in ks]
    for a, i, o in zip(am, inv, one):
        capi.sq_act_scale(a, i, o)
    capi.sq_act_scale_batched(am, inv, two)
    torch.cuda.synchronize()
    for k, o1, o2 in zip(ks, one, two):
        assert torch.equal(o1[:1], o2[:1]), k


def test_dynamic_block_forward_equals_per_layer():
    """The 13B block's dynamic forward in four launches gives the per-layer
    dynamic forward's scales and outputs, bit for bit."""
    import torch
    from w8a8_post_quantization_channel_amd.layer import W8A8Linear, forward_block_dynamic, prepare_block
    rows = 512
    groups = {gname: _t(synth.c2_group_x(gname, rows=rows)) for gname in synth.C2_GROUPS}
    acts = {gname: torch.empty(x.shape[1], dtype=torch.float32, device=dev()) for gname, x in groups.items()}
    layers, xs = [], []
    for p, gname, *_ in synth.C2_PROJECTIONS:
        layer = W8A8Linear(_t(synth.c2_projection_w(p)), alpha=0.5, max_tokens=rows, out_dtype=torch.bfloat16)
        layer.act_max = acts[gname]
        layers.append(layer)
        xs.append(groups[gname])
    prepare_block(layers, [(groups[gname], acts[gname]) for gname in groups])
    # runtime inputs beyond the calibrated range: the dynamic scale differs from the static one
    live = {gname: (x.float() * 1.7).to(torch.bfloat16) for gname, x in groups.items()}
    xs = [live[gname] for _, gname, *_ in synth.C2_PROJECTIONS]
    ref = [l.forward_dynamic(x).clone() for l, x in zip(layers, xs)]
    ref_scale = [l.dyn_scale[:1].clone() for l in layers]
    torch.cuda.synchronize()
    for l in layers:
        l.dyn_scale.zero_()
        l.y.zero_()
    ys = forward_block_dynamic(layers, xs)
    torch.cuda.synchronize()
    for (p, *_), l, y, r, rs in zip(synth.C2_PROJECTIONS, layers, ys, ref, ref_scale):
        assert torch.equal(l.dyn_scale[:1], rs), p
        assert torch.equal(y.view(torch.int16), r.view(torch.int16)), p


@pytest.mark.gpu
def test_side_stream_without_preallocated_buffers():
    """A layer with no preallocated buffers run on a non-current stream: the
    codes and the output it allocates are recorded on that stream, so work
    queued afterwards on the current stream cannot take their memory while
    the layer's kernels still run. Checked against the oracle."""
    import numpy as np
    import torch

    from oracle.oracle import Oracle
    from w8a8_post_quantization_channel_amd import synth
    from w8a8_post_quantization_channel_amd.layer import W8A8Linear

    d = torch.device("cuda", 0)
    m, n, k = 1024, 2048, 1024
    out = synth.outlier_channels(71, k)
    x = synth.activations(72, m, k, out)
    w = synth.weights(73, n, k)
    xt, wt = synth.to_torch(x, d), synth.to_torch(w, d)
    layer = W8A8Linear(wt, alpha=0.5, max_tokens=0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    layer.calibrate(xt, stream=side)
    layer.prepare(stream=side)
    ys = []
    for _ in range(3):
        ys.append(layer.forward(xt, stream=side))
        # churn the allocator on the current stream while the side stream works
        junk = [torch.full((m, k), 7, dtype=torch.int8, device=d) for _ in range(4)]
        del junk
    side.synchronize()
    torch.cuda.synchronize()
    ref = Oracle().layer_forward([x], w, x, 0.5, bf16_out=True)
    for y in ys:
        assert np.array_equal(synth.from_torch(y), ref["y"])
