"""GPU parity: the HIP path through the C ABI against the CPU oracle, on the
same seeded inputs.

Bar: int8 codes and int32 accumulators bit-exact; statistics exact; smoothing
factors, scales and dequantized outputs within 1e-5 relative (fp32) or 1e-2
(after a bf16 store) -- in practice they are bit-exact too, which the
`exact` checks assert wherever the fixed fp32 op order makes the result
unique.
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle.oracle import Oracle
from tests.gpu_pipeline import assert_bitexact, assert_rel, dev, gpu_layer
from w8a8_post_quantization_channel_amd import capi, synth

pytestmark = pytest.mark.gpu
ORACLE = Oracle()
TOL_F32, TOL_BF16 = 1e-5, 1e-2


@pytest.fixture(scope="module", autouse=True)
def _lib():
    capi.load()


def check_layer(g, r, out_bf16, rows=None):
    """g: GPU arrays; r: oracle arrays. rows: sampled output rows of acc/y."""
    assert_bitexact("act_max", g["act_max"], r["act_max"])
    assert_bitexact("w_max", g["w_max"], r["w_max"])
    assert_rel("s", g["s"], r["s"], TOL_F32)
    assert_rel("inv_s", g["inv_s"], r["inv_s"], TOL_F32)
    assert_rel("act_scale", g["act_scale"], np.array([r["act_scale"]], np.float32), TOL_F32)
    assert_rel("w_scale", g["w_scale"], r["w_scale"], TOL_F32)
    assert_bitexact("s (exact)", g["s"], r["s"])
    assert_bitexact("wq", g["wq"], r["wq"])
    assert_bitexact("xq", g["xq"], r["xq"])
    gy, gacc = g["y"], g.get("acc")
    if rows is not None:
        gy = gy[rows]
        gacc = gacc[rows] if gacc is not None else None
    if gacc is not None:
        assert_bitexact("acc", gacc, r["acc"])
    assert_rel("y", gy, r["y"], TOL_BF16 if out_bf16 else TOL_F32)
    assert_bitexact("y (exact)", gy, r["y"])


def oracle_layer_rows(xs_calib, w, x, alpha, out_bf16, rows):
    """Oracle chain with the product evaluated on sampled rows of x only."""
    o = ORACLE
    k = w.shape[1]
    act_max = np.zeros(k, np.float32)
    for xc in xs_calib:
        o.calib_absmax(xc, act_max)
    w_max = o.calib_absmax(w)
    s, inv_s, a = o.smooth_factors(act_max, w_max, alpha)
    wq, ws = o.quant_weight(w, s)
    xq = o.quant_act(x, inv_s, a)
    acc = o.gemm_i32(np.ascontiguousarray(xq[rows]), wq)
    y = o.dequant(acc, a, ws, bf16=out_bf16)
    return dict(act_max=act_max, w_max=w_max, s=s, inv_s=inv_s, act_scale=a, wq=wq, w_scale=ws, xq=xq, acc=acc, y=y)


# ---- whole layer, small and ragged ----------------------------------------------

def test_c1_single_fp32_layer():
    x, w = synth.c1()
    g = gpu_layer([x], w, x, 0.5, out_bf16=False)
    r = ORACLE.layer_forward([x], w, x, 0.5, bf16_out=False)
    check_layer(g, r, False)


@pytest.mark.parametrize("m,n,k,bf16_in,bf16_out", [
    (300, 520, 1088, True, True),     # ragged M, N tail, K % 128 == 64
    (1, 16, 64, False, False),        # smallest legal shape
    (257, 272, 192, True, False),
    (2100, 4112, 256, True, True),    # large-tile path with ragged M and N
    (64, 4096, 11008, True, True),    # K = 11008 (not a multiple of 512 bf16 columns)
])
def test_layer_shapes(m, n, k, bf16_in, bf16_out):
    out = synth.outlier_channels(700 + m, k)
    xc = [synth.activations(710 + m + b, 96, k, out, bf16=bf16_in) for b in range(2)]
    x = synth.activations(720 + m, m, k, out, scale=1.5, bf16=bf16_in)  # beyond the calibrated range
    w = synth.weights(730 + m, n, k, bf16=bf16_in)
    g = gpu_layer(xc, w, x, 0.5, out_bf16=bf16_out)
    r = ORACLE.layer_forward(xc, w, x, 0.5, bf16_out=bf16_out)
    check_layer(g, r, bf16_out)


@pytest.mark.parametrize("alpha", [0.0, 0.25, 0.75, 1.0])
def test_alpha_values(alpha):
    m, n, k = 33, 200, 512
    out = synth.outlier_channels(800, k)
    x = synth.activations(801, m, k, out)
    w = synth.weights(802, n, k)
    g = gpu_layer([x], w, x, alpha, out_bf16=True)
    r = ORACLE.layer_forward([x], w, x, alpha, bf16_out=True)
    check_layer(g, r, True)


# ---- single entry points -------------------------------------------------------------

def test_absmax_cases():
    import torch
    d = dev()
    for k, bf16 in [(1088, True), (1088, False), (64, True), (13824, True)]:
        chunks = [synth.activations(900 + i, rows, k, synth.outlier_channels(899, k), bf16=bf16)
                  for i, rows in enumerate([1, 17, 333])]
        am = torch.empty(k, dtype=torch.float32, device=d)
        ref = np.zeros(k, np.float32)
        for i, c in enumerate(chunks):
            capi.sq_calib_absmax(synth.to_torch(c, d), am, accumulate=i > 0)
            ORACLE.calib_absmax(c, ref)
        torch.cuda.synchronize()
        assert_bitexact(f"absmax k={k}", synth.from_torch(am), ref)
    # zero rows, overwrite: all zeros
    am = torch.full((128,), 7.0, dtype=torch.float32, device=d)
    capi.sq_calib_absmax(torch.empty((0, 128), dtype=torch.bfloat16, device=d), am, accumulate=False)
    torch.cuda.synchronize()
    assert not am.any()


@pytest.mark.parametrize("k,bf16", [(2048, True), (4096, True), (5120, True), (8192, True), (13824, True),
                                    (16384, True), (28672, True), (33792, True), (66560, True), (1024, False),
                                    (2560, False), (4096, False), (8192, False), (16384, False), (20480, False),
                                    (40960, False), (66560, False), (11008, True), (6144, False),
                                    # each side of the row classes of the whole-row kernel (1024 and
                                    # 4096 16-byte vectors) and the shortest row
                                    (64, True), (8256, True), (32768, True), (32832, True), (64, False),
                                    (4160, False), (16448, False)])
def test_quant_weight_paths(k, bf16):
    import torch
    d = dev()
    n = 5
    g = synth.rng(1000 + k)
    w = synth.weights(1001 + k, n, k, std=1.0, bf16=False)
    w[2] = 0.0
    w[3, 7] = 1e4
    w = synth.to_bf16_bits(w) if bf16 else w
    s = g.uniform(0.1, 10.0, k).astype(np.float32)
    wq = torch.empty((n, k), dtype=torch.int8, device=d)
    ws = torch.empty(n, dtype=torch.float32, device=d)
    capi.sq_quant_weight(synth.to_torch(w, d), synth.to_torch(s, d), wq, ws)
    torch.cuda.synchronize()
    rq, rs = ORACLE.quant_weight(w, s)
    assert_bitexact("wq", synth.from_torch(wq), rq)
    assert_bitexact("w_scale", synth.from_torch(ws), rs)


@pytest.mark.parametrize("m,k,bf16", [(1, 64, True), (7, 1088, True), (33, 5120, True), (300, 4096, False),
                                      (1000, 11008, True),
                                      # more than 65535 blocks of 32 rows: taller blocks, ragged last one
                                      (65535 * 32 + 37, 64, True)])
def test_quant_act_cases(m, k, bf16):
    import torch
    d = dev()
    g = synth.rng(1100 + m)
    x = synth.activations(1101 + m, m, k, synth.outlier_channels(1102, k), bf16=bf16)
    inv_s = g.uniform(0.01, 2.0, k).astype(np.float32)
    xf = synth.bf16_bits_to_f32(x) if bf16 else x
    # a scale at half the largest smoothed value, so saturation is exercised
    a = np.array([0.5 * np.abs(xf * inv_s).max() / 127.0, 0, 0, 0], np.float32)
    xq = torch.empty((m, k), dtype=torch.int8, device=d)
    capi.sq_smooth_quant_act(synth.to_torch(x, d), synth.to_torch(inv_s, d), synth.to_torch(a, d), xq)
    torch.cuda.synchronize()
    ref = ORACLE.quant_act(x, inv_s, a[0])
    assert_bitexact("xq", synth.from_torch(xq), ref)
    assert np.abs(ref.astype(np.int32)).max() == 127  # saturation is exercised


def test_quant_act_ties():
    """Exact .5 ties round to even, +-200 saturate at +-127 (s = 1, scale 1)."""
    import torch
    d = dev()
    k = 64
    vals = [2.5, 3.5, -2.5, 0.5, 1.5, -0.5, -1.5, 200.0, -200.0, 126.5, -127.5, 127.49, -126.5, 4.5, 5.5, 0.0]
    x = np.zeros((3, k), np.float32)
    x[1, :len(vals)] = vals
    x[2] = -x[1]
    ones = np.ones(k, np.float32)
    a = np.array([1.0, 0, 0, 0], np.float32)
    xq = torch.empty((3, k), dtype=torch.int8, device=d)
    capi.sq_smooth_quant_act(synth.to_torch(x, d), synth.to_torch(ones, d), synth.to_torch(a, d), xq)
    torch.cuda.synchronize()
    assert_bitexact("ties", synth.from_torch(xq), ORACLE.quant_act(x, ones, a[0]))


GEMM_CASES = [(1, 16, 64), (5, 48, 1088), (129, 257, 320), (300, 600, 2048), (512, 8192, 128),
              (1024, 8192, 256), (2100, 4112, 192), (2048, 7168, 64), (2048, 11008, 128), (4096, 4096, 64),
              (4000, 4100, 64), (1000, 11008, 320),
              # the split LDS rings of the wide tiles over several K steps, ragged m and n and a
              # half last step: 256 x 256 (1100 x 12000) and 256 x 224 (1500 x 9000)
              (1100, 12000, 704), (1500, 9000, 448),
              # decode widths: 17-32 and 33-64 rows, 8-wave blocks (>= 512 column blocks) and
              # 16-wave blocks, K steps not a multiple of waves x steps in flight
              (24, 8200, 192), (17, 1000, 4160), (40, 8192, 320), (64, 300, 704), (9, 8208, 1344),
              # the vector-ALU kernel (m <= 4): 2 and 4 activation rows, ragged weight-row blocks, a
              # partial last 1 KB chunk, up to 4 chunks per wave in flight and, past 16 KB of K,
              # a second group of chunks
              (2, 1003, 4160), (3, 4100, 11008), (4, 262, 20480), (1, 4097, 13824)]


def reachable_tilings():
    """Block tiles the library picks over a broad grid of output shapes."""
    ms = [1, 8, 16, 64, 100, 128, 200, 256, 512, 1000, 1024, 1500, 2048, 3000, 4096, 8192, 16384]
    ns = [16, 128, 512, 1024, 2048, 3000, 4096, 5120, 7168, 8192, 11008, 13824, 28672]
    return {capi.sq_gemm_tiling(m, n) for m in ms for n in ns}


def test_gemm_cases_cover_every_tiling():
    """The GEMM cases below exercise every block tile the library can pick."""
    used = {capi.sq_gemm_tiling(m, n) for m, n, _ in GEMM_CASES}
    assert reachable_tilings() <= used, (reachable_tilings(), used)


@pytest.mark.parametrize("m,n,k", GEMM_CASES)
@pytest.mark.parametrize("bf16_out", [False, True])
def test_gemm_cases(m, n, k, bf16_out):
    import torch
    d = dev()
    g = synth.rng(1200 + m + n + k)
    xq = g.integers(-127, 128, (m, k), dtype=np.int8)
    wq = g.integers(-127, 128, (n, k), dtype=np.int8)
    ws = g.uniform(1e-4, 1e-2, n).astype(np.float32)
    a = np.array([0.0213, 0, 0, 0], np.float32)
    y = torch.empty((m, n), dtype=torch.bfloat16 if bf16_out else torch.float32, device=d)
    acc = torch.empty((m, n), dtype=torch.int32, device=d)
    capi.sq_w8a8_gemm(synth.to_torch(xq, d), synth.to_torch(wq, d), synth.to_torch(a, d), synth.to_torch(ws, d),
                      y, acc)
    torch.cuda.synchronize()
    racc = ORACLE.gemm_i32(xq, wq)
    assert_bitexact("acc", synth.from_torch(acc), racc)
    assert_bitexact("y", synth.from_torch(y), ORACLE.dequant(racc, a[0], ws, bf16=bf16_out))


def test_gemm_extremes_and_empty():
    import torch
    d = dev()
    k = 28672
    xq = np.full((3, k), 127, np.int8)
    xq[1] = -127
    xq[2, ::2] = -127
    wq = np.full((20, k), 127, np.int8)
    wq[5] = -127
    ws = np.full(20, 1e-3, np.float32)
    a = np.array([2e-3, 0, 0, 0], np.float32)
    y = torch.empty((3, 20), dtype=torch.float32, device=d)
    acc = torch.empty((3, 20), dtype=torch.int32, device=d)
    capi.sq_w8a8_gemm(synth.to_torch(xq, d), synth.to_torch(wq, d), synth.to_torch(a, d), synth.to_torch(ws, d),
                      y, acc)
    torch.cuda.synchronize()
    racc = ORACLE.gemm_i32(xq, wq)
    assert racc[0, 0] == k * 127 * 127
    assert_bitexact("acc", synth.from_torch(acc), racc)
    assert_bitexact("y", synth.from_torch(y), ORACLE.dequant(racc, a[0], ws))
    # an empty batch is a no-op
    y0 = torch.empty((0, 20), dtype=torch.float32, device=d)
    capi.sq_w8a8_gemm(torch.empty((0, k), dtype=torch.int8, device=d), synth.to_torch(wq, d),
                      synth.to_torch(a, d), synth.to_torch(ws, d), y0)
    torch.cuda.synchronize()
