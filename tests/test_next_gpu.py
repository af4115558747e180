"""GPU parity of the widened activation-side entry points against the CPU
oracle: the dynamic per-tensor scale, the averaged per-sample maxima, RMSNorm
and the norm with 1/s folded into its weight feeding the quantizer.

Bar: statistics, scales and int8 codes bit-exact. The RMSNorm factor r is a
fp64 sum of squares in an order the kernel chooses, rounded once to fp32, so
it may differ from the oracle's sequential sum by one fp32 ulp; everything
after r is checked bit-exactly against the oracle fed with the GPU's own r
(the same stage-wise rule as for s).
"""
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


def _x(seed, m, k, bf16, outliers=True):
    out = synth.outlier_channels(seed, k) if outliers else None
    return synth.activations(seed + 1, m, k, out, bf16=bf16)


def _inv_s(seed, k):
    return synth.rng(seed).uniform(0.02, 3.0, k).astype(np.float32)


def _t(a):
    return synth.to_torch(a, dev())


def _host(t):
    return synth.from_torch(t)


# ---- sq_act_scale and the dynamic mode ------------------------------------------

def test_act_scale_entry():
    import torch
    k = 5120
    g = synth.rng(501)
    act_max = (g.uniform(0.1, 5.0, k) * (g.random(k) < 0.99) + 0).astype(np.float32)  # some zeros: floor
    inv_s = _inv_s(502, k)
    a = torch.empty(4, dtype=torch.float32, device=dev())
    capi.sq_act_scale(_t(act_max), _t(inv_s), a)
    torch.cuda.synchronize()
    assert_bitexact("act_scale", _host(a)[:1], np.array([ORACLE.act_scale(act_max, inv_s)], np.float32))


@pytest.mark.parametrize("m,k,bf16", [(300, 1088, True), (2048, 5120, True), (16, 1024, False), (1, 64, True),
                                      (4099, 320, False)])
def test_dynamic_quant_act(m, k, bf16):
    import torch
    x = _x(510 + m, m, k, bf16)
    inv_s = _inv_s(511, k)
    live = torch.empty(k, dtype=torch.float32, device=dev())
    a = torch.empty(4, dtype=torch.float32, device=dev())
    xq = torch.empty((m, k), dtype=torch.int8, device=dev())
    capi.sq_dynamic_quant_act(_t(x), _t(inv_s), live, a, xq)
    torch.cuda.synchronize()
    rq, ra = ORACLE.dynamic_quant_act(x, inv_s)
    assert_bitexact("live_max", _host(live), ORACLE.calib_absmax(x))
    assert_bitexact("act_scale", _host(a)[:1], np.array([ra], np.float32))
    assert_bitexact("xq", _host(xq), rq)


def test_dynamic_quant_act_empty_batch():
    import torch
    k = 256
    inv_s = _inv_s(520, k)
    live = torch.full((k,), 7.0, dtype=torch.float32, device=dev())
    a = torch.empty(4, dtype=torch.float32, device=dev())
    xq = torch.empty((0, k), dtype=torch.int8, device=dev())
    x = torch.empty((0, k), dtype=torch.bfloat16, device=dev())
    capi.sq_dynamic_quant_act(x, _t(inv_s), live, a, xq)
    torch.cuda.synchronize()
    assert not _host(live).any()
    _, ra = ORACLE.dynamic_quant_act(np.zeros((1, k), np.float32), inv_s)
    assert_bitexact("act_scale (floor)", _host(a)[:1], np.array([ra], np.float32))


# ---- averaged per-sample maxima ------------------------------------------------------

@pytest.mark.parametrize("samples,rows,k,bf16", [(24, 50, 1088, True), (7, 33, 320, False), (512, 64, 5120, True),
                                                 (3, 1, 64, True)])
def test_sample_max_mean(samples, rows, k, bf16):
    import torch
    x = _x(530 + samples, samples * rows, k, bf16)
    smax = torch.empty((samples, k), dtype=torch.float32, device=dev())
    total = torch.zeros(k, dtype=torch.float64, device=dev())
    # two calls: the first third of the samples, then the rest (running sum)
    s1 = samples // 3
    tx = _t(x)
    if s1:
        capi.sq_calib_sample_max_sum(tx[: s1 * rows], s1, smax[:s1], total)
    capi.sq_calib_sample_max_sum(tx[s1 * rows:], samples - s1, smax[s1:], total)
    act_max = torch.empty(k, dtype=torch.float32, device=dev())
    capi.sq_calib_mean_finalize(total, samples, act_max)
    torch.cuda.synchronize()
    per = np.stack([ORACLE.calib_absmax(np.ascontiguousarray(x[b * rows:(b + 1) * rows])) for b in range(samples)])
    assert_bitexact("sample_max", _host(smax), per)
    ref_sum = ORACLE.calib_sample_max_sum(x, samples)
    got_sum = _host(total)
    assert np.array_equal(got_sum.view(np.uint64), ref_sum.view(np.uint64)), "fp64 running sum differs"
    assert_bitexact("act_max (mean of maxima)", _host(act_max), ORACLE.calib_mean_finalize(ref_sum, samples))


# ---- RMSNorm and the folded norm + quantizer -------------------------------------------

def _norm_inputs(seed, m, k, bf16):
    g = synth.rng(seed)
    h = (g.standard_normal((m, k)) * g.uniform(0.05, 30.0, (m, 1))).astype(np.float32)
    h[:, g.integers(0, k, 3)] *= 40.0  # outlier channels
    if bf16:
        h = synth.to_bf16_bits(h)
    gamma = g.uniform(0.2, 2.0, k).astype(np.float32)
    return h, gamma


def _check_r(r_gpu, r_ref):
    d = np.abs(r_gpu.view(np.int32).astype(np.int64) - r_ref.view(np.int32).astype(np.int64))
    assert d.max() <= 1, f"r differs by {d.max()} ulp"
    assert (d != 0).mean() <= 0.01, f"r differs in {(d != 0).mean():.3%} of the rows"


# every launch shape: 1..8 vectors per thread (8, 4, 2, 2, 1, 1 rows per block, ragged row counts) and
# the streamed long rows
NORM_CASES = [(37, 320, False, False), (300, 5120, True, True), (5, 20480, True, True), (64, 8192, True, False),
              (1, 64, False, True), (129, 4096, True, True), (17, 12288, True, True), (9, 6144, False, False),
              (6, 33024, False, True), (3, 16384, True, False), (7, 10240, True, True), (13, 2048, True, True)]


@pytest.mark.parametrize("m,k,bf16_in,bf16_out", NORM_CASES)
def test_rmsnorm(m, k, bf16_in, bf16_out):
    import torch
    eps = 1e-5
    h, gamma = _norm_inputs(540 + m, m, k, bf16_in)
    y = torch.empty((m, k), dtype=torch.bfloat16 if bf16_out else torch.float32, device=dev())
    r = torch.empty(m, dtype=torch.float32, device=dev())
    capi.sq_rmsnorm(_t(h), _t(gamma), eps, y, r)
    torch.cuda.synchronize()
    rg = _host(r)
    _check_r(rg, ORACLE.rms_inv(h, eps))
    assert_bitexact("y", _host(y), ORACLE.rmsnorm_apply(h, rg, gamma, bf16=bf16_out))


@pytest.mark.parametrize("m,k,bf16_in,_unused", NORM_CASES)
def test_rmsnorm_quant_act(m, k, bf16_in, _unused):
    import torch
    eps = 1e-5
    h, gamma = _norm_inputs(560 + m, m, k, bf16_in)
    inv_s = _inv_s(561, k)
    gf = torch.empty(k, dtype=torch.float32, device=dev())
    capi.sq_fold_norm_weight(_t(gamma), _t(inv_s), gf)
    # a static scale from the plain norm output of this batch (as a calibration would give)
    r_ref = ORACLE.rms_inv(h, eps)
    a = ORACLE.act_scale(ORACLE.calib_absmax(ORACLE.rmsnorm_apply(h, r_ref, gamma)), inv_s)
    ta = torch.tensor([a, 0, 0, 0], dtype=torch.float32, device=dev())
    xq = torch.empty((m, k), dtype=torch.int8, device=dev())
    r = torch.empty(m, dtype=torch.float32, device=dev())
    capi.sq_rmsnorm_quant_act(_t(h), gf, eps, ta, xq, r)
    torch.cuda.synchronize()
    gf_h = _host(gf)
    assert_bitexact("gamma_folded", gf_h, ORACLE.fold_norm_weight(gamma, inv_s))
    rg = _host(r)
    _check_r(rg, r_ref)
    assert_bitexact("xq", _host(xq), ORACLE.norm_quant_apply(h, rg, gf_h, a))


def test_rmsnorm_quant_act_empty_and_no_r():
    import torch
    k = 512
    h, gamma = _norm_inputs(580, 8, k, True)
    gf = _t(gamma)
    ta = torch.tensor([0.05, 0, 0, 0], dtype=torch.float32, device=dev())
    xq = torch.full((8, k), 5, dtype=torch.int8, device=dev())
    capi.sq_rmsnorm_quant_act(_t(h)[:0], gf, 1e-5, ta, xq[:0])
    torch.cuda.synchronize()
    assert (_host(xq) == 5).all()
    capi.sq_rmsnorm_quant_act(_t(h), gf, 1e-5, ta, xq)  # r_out = NULL
    torch.cuda.synchronize()
    r_ref = ORACLE.rms_inv(h, 1e-5)
    ref = ORACLE.norm_quant_apply(h, r_ref, gamma, np.float32(0.05))
    got = _host(xq)
    # with r unchecked, rows whose r differs by one ulp may differ by one code step
    assert np.abs(got.astype(np.int32) - ref.astype(np.int32)).max() <= 1


# ---- nearest-rank percentile -----------------------------------------------------------

@pytest.mark.parametrize("rows,k,bf16,qs", [
    (1000, 320, True, (0.999, 0.5, 0.9995, 1.0, 0.0)),
    (777, 64, False, (0.999, 0.25, 1.0)),
    (65536, 1024, True, (0.999,)),
    (4099, 128, False, (0.9, 0.999)),
])
def test_percentile(rows, k, bf16, qs):
    import torch
    x = _x(600 + rows, rows, k, bf16)
    tx = _t(x)
    ws = torch.empty(capi.sq_calib_percentile_workspace(k, capi.SQ_BF16 if bf16 else capi.SQ_F32),
                     dtype=torch.uint8, device=dev())
    out = torch.empty(k, dtype=torch.float32, device=dev())
    for q in qs:
        capi.sq_calib_percentile(tx, q, ws, out)
        torch.cuda.synchronize()
        assert_bitexact(f"percentile q={q}", _host(out), ORACLE.calib_percentile(x, q))


def test_percentile_ties_and_signs():
    import torch
    g = synth.rng(620)
    rows, k = 3000, 64
    # few distinct magnitudes with both signs, zeros and negative zeros: ties everywhere
    x = (g.integers(-3, 4, (rows, k)) * 0.5).astype(np.float32)
    x[g.random((rows, k)) < 0.05] = -0.0
    x[7, :] = -1000.0
    xb = synth.to_bf16_bits(x)
    ws = torch.empty(capi.sq_calib_percentile_workspace(k, capi.SQ_F32), dtype=torch.uint8, device=dev())
    out = torch.empty(k, dtype=torch.float32, device=dev())
    for arr in (x, xb):
        for q in (0.999, 0.9996, 0.5, 1.0, 1.0 / rows):
            capi.sq_calib_percentile(_t(arr), q, ws, out)
            torch.cuda.synchronize()
            assert_bitexact(f"ties q={q}", _host(out), ORACLE.calib_percentile(arr, q))


@pytest.mark.parametrize("m,k,bf16,n", [(37, 5120, True, 3), (2048, 5120, True, 3), (100, 8192, True, 2),
                                        (64, 2048, False, 4), (5, 16384, True, 3), (300, 64, True, 2),
                                        (9, 4096, False, 1)])
def test_rmsnorm_quant_multi_equals_single(m, k, bf16, n):
    """Several consumers of one norm output in one call: every consumer's
    codes and r equal the single-consumer call's, bit for bit (one pass over
    h, or one per consumer when the row is too long for all weights in
    registers, e.g. k = 16384 with three consumers)."""
    import torch
    g = synth.rng(5200 + m + n)
    h = _t(_x(5201 + m, m, k, bf16))
    gam = [_t(g.uniform(0.2, 3.0, k).astype(np.float32)) for _ in range(n)]
    a = [torch.tensor([g.uniform(0.005, 0.05), 0, 0, 0], dtype=torch.float32, device=dev()) for _ in range(n)]
    one = [torch.empty((m, k), dtype=torch.int8, device=dev()) for _ in range(n)]
    r1 = torch.empty(m, dtype=torch.float32, device=dev())
    for c in range(n):
        capi.sq_rmsnorm_quant_act(h, gam[c], 1e-5, a[c], one[c], r_out=r1)
    two = [torch.full((m, k), 99, dtype=torch.int8, device=dev()) for _ in range(n)]
    r2 = torch.zeros(m, dtype=torch.float32, device=dev())
    capi.sq_rmsnorm_quant_act_multi(h, gam, 1e-5, a, two, r_out=r2)
    torch.cuda.synchronize()
    assert torch.equal(r1, r2)
    for c in range(n):
        assert torch.equal(one[c], two[c]), c
