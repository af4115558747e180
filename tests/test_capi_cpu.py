"""CPU: libsq.so loads, exports every entry point include/sq.h declares, and
rejects invalid arguments with the documented status before launching
anything (every call here fails validation, so no GPU is touched)."""
import ctypes
import math

import pytest

from w8a8_post_quantization_channel_amd import build as sqbuild
from w8a8_post_quantization_channel_amd import capi, ceiling

OK, NULL, SHAPE, DTYPE, ALPHA, WORKSPACE, HIP, ALIGN = range(8)
A = 0x10000   # a fake, 16-byte-aligned device address (never dereferenced)
MIS = 0x10004  # a fake misaligned address
P = ctypes.c_void_p


@pytest.fixture(scope="module")
def lib():
    if sqbuild.stale():
        sqbuild.build()
    return capi.load()


def test_exports_every_declared_symbol(lib):
    names = capi.declared_functions()
    assert set(names) >= {"sq_calib_absmax", "sq_smooth_factors", "sq_quant_weight", "sq_smooth_quant_act",
                          "sq_w8a8_gemm", "sq_alpha_search", "sq_alpha_search_workspace", "sq_status_string",
                          "sq_gemm_tiling", "sq_gemm_batched_tiling"}
    for name in names:
        assert hasattr(lib, name), name


def test_measurement_probes_live_in_their_own_library(lib):
    """libsq.so exports the path only; the measured-ceiling probes are in
    libsq_ceiling.so, which exports every function include/sq_ceiling.h declares."""
    names = ceiling.declared_functions()
    assert names == ["sq_ceiling_copy", "sq_ceiling_mfma", "sq_ceiling_narrow", "sq_ceiling_read"]
    clib = ceiling.load()
    for name in names:
        assert hasattr(clib, name), name
        assert not hasattr(lib, name), name
    assert not any(n.startswith("sq_ceiling") for n in capi.declared_functions())


def test_status_strings(lib):
    for code in range(9):
        assert lib.sq_status_string(code)
    assert lib.sq_status_string(99) == b"unknown status"


def test_calib_absmax_validation(lib):
    f = lib.sq_calib_absmax
    assert f(P(A), 1, 16, 1024, None, 0, None) == NULL
    assert f(None, 1, 16, 1024, P(A), 0, None) == NULL
    assert f(P(A), 2, 16, 1024, P(A), 0, None) == DTYPE
    assert f(P(A), 1, -1, 1024, P(A), 0, None) == SHAPE
    assert f(P(A), 1, 16, 1000, P(A), 0, None) == SHAPE
    assert f(P(A), 1, 16, 0, P(A), 0, None) == SHAPE
    assert f(P(MIS), 1, 16, 1024, P(A), 0, None) == ALIGN
    assert f(P(A), 1, 16, 1024, P(MIS), 0, None) == ALIGN
    # zero rows into a running max is a no-op (x may be NULL)
    assert f(None, 1, 0, 1024, P(A), 1, None) == OK


def test_smooth_factors_validation(lib):
    f = lib.sq_smooth_factors
    args = [P(A), P(A), 1024, 0.5, P(A), P(A), P(A), None]
    for bad in (float("nan"), float("inf"), -0.01, 1.01):
        a = list(args)
        a[3] = bad
        assert f(*a) == ALPHA
    a = list(args)
    a[4] = None
    assert f(*a) == NULL
    a = list(args)
    a[2] = 96
    assert f(*a) == SHAPE
    a = list(args)
    a[6] = P(MIS)
    assert f(*a) == ALIGN


def test_quant_weight_validation(lib):
    f = lib.sq_quant_weight
    assert f(P(A), 1, 8, 1024, None, P(A), P(A), None) == NULL
    assert f(P(A), 7, 8, 1024, P(A), P(A), P(A), None) == DTYPE
    assert f(P(A), 1, -8, 1024, P(A), P(A), P(A), None) == SHAPE
    assert f(P(A), 1, 8, 1056, P(A), P(A), P(A), None) == SHAPE
    assert f(P(A), 1, 8, 1024, P(A), P(MIS), P(A), None) == ALIGN


def test_quant_act_validation(lib):
    f = lib.sq_smooth_quant_act
    assert f(P(A), 1, 8, 1024, P(A), None, P(A), None) == NULL
    assert f(None, 1, 8, 1024, P(A), P(A), P(A), None) == NULL
    assert f(P(A), 1, 8, 1024 + 32, P(A), P(A), P(A), None) == SHAPE
    assert f(P(MIS), 1, 8, 1024, P(A), P(A), P(A), None) == ALIGN


def test_gemm_validation(lib):
    f = lib.sq_w8a8_gemm
    base = [P(A), P(A), 16, 32, 1024, P(A), P(A), P(A), 1, None, None]
    a = list(base)
    a[5] = None
    assert f(*a) == NULL
    a = list(base)
    a[8] = 3
    assert f(*a) == DTYPE
    a = list(base)
    a[4] = 131072 + 64
    assert f(*a) == SHAPE
    a = list(base)
    a[4] = 100
    assert f(*a) == SHAPE
    a = list(base)
    a[2] = -1
    assert f(*a) == SHAPE
    a = list(base)
    a[9] = P(MIS)
    assert f(*a) == ALIGN
    # an empty product launches nothing and succeeds
    a = list(base)
    a[2] = 0
    assert f(*a) == OK


def test_gemm_tiling_query(lib):
    bm, bn = ctypes.c_int(0), ctypes.c_int(0)
    assert lib.sq_gemm_tiling(16, 32, None, ctypes.byref(bn)) == NULL
    assert lib.sq_gemm_tiling(-1, 32, ctypes.byref(bm), ctypes.byref(bn)) == SHAPE
    assert lib.sq_gemm_tiling(2048, 5120, ctypes.byref(bm), ctypes.byref(bn)) == OK
    assert bm.value in (128, 256) and bn.value in (128, 160, 192, 224, 256)


def test_gemm_batched_tiling_query(lib):
    """One width for the products of a grouped launch, chosen for the group,
    except that a 256 x 256 launch may run up to its last three products (never
    all of them) on 256 x 128 tiles; decode and small products keep their
    single-call tiles; argument errors are statuses."""
    blk = [(2048, 5120, 5120)] * 4 + [(2048, 13824, 5120)] * 2 + [(2048, 5120, 13824)]
    for order in (blk, blk[::-1]):
        tiles = capi.sq_gemm_batched_tiling(order)
        assert tiles[0] == (256, 256) and set(tiles) <= {(256, 256), (256, 128)}, tiles
        narrow = [i for i, t in enumerate(tiles) if t == (256, 128)]
        assert len(narrow) <= 3 and narrow == list(range(len(tiles) - len(narrow), len(tiles))), tiles
    # one product: the single call's choice
    for m, n, k in [(2048, 5120, 5120), (4096, 8192, 8192), (300, 600, 2048), (16, 4096, 4096), (1, 4096, 4096)]:
        assert capi.sq_gemm_batched_tiling([(m, n, k)]) == [capi.sq_gemm_tiling(m, n)]
    # decode products and empty ones keep their own tiles beside a grouped launch
    mixed = [(1, 4096, 4096), (16, 4096, 4096), (2048, 5120, 5120), (0, 512, 64), (2048, 13824, 5120)]
    got = capi.sq_gemm_batched_tiling(mixed)
    assert got[0] == capi.sq_gemm_tiling(1, 4096) and got[1] == capi.sq_gemm_tiling(16, 4096)
    assert got[2] == got[4] and got[2][0] == 256
    m, n, k = (ctypes.c_int64 * 2)(2048, 2048), (ctypes.c_int64 * 2)(5120, 5120), (ctypes.c_int64 * 2)(64, 64)
    bm, bn = (ctypes.c_int * 2)(), (ctypes.c_int * 2)()
    assert lib.sq_gemm_batched_tiling(2, m, n, None, bm, bn) == NULL
    assert lib.sq_gemm_batched_tiling(0, m, n, k, bm, bn) == SHAPE
    assert lib.sq_gemm_batched_tiling(17, m, n, k, bm, bn) == SHAPE
    k[1] = 0
    assert lib.sq_gemm_batched_tiling(2, m, n, k, bm, bn) == SHAPE
    k[1] = 64
    assert lib.sq_gemm_batched_tiling(2, m, n, k, bm, bn) == OK and bm[0] == bm[1] and bn[0] == bn[1]


def test_alpha_search_validation(lib):
    ws = ctypes.c_size_t(0)
    assert lib.sq_alpha_search_workspace(8, 2048, 11008, 4096, 4, None) == NULL
    assert lib.sq_alpha_search_workspace(0, 2048, 11008, 4096, 4, ctypes.byref(ws)) == SHAPE
    assert lib.sq_alpha_search_workspace(8, 2048, 11008, 4000, 4, ctypes.byref(ws)) == SHAPE
    assert lib.sq_alpha_search_workspace(8, 2048, 11008, 4096, 17, ctypes.byref(ws)) == SHAPE
    assert lib.sq_alpha_search_workspace(8, 2048, 11008, 4096, 4, ctypes.byref(ws)) == OK
    need = ws.value
    # at least the reference outputs and the int8 weight
    assert need >= 8 * 2048 * 11008 * 4 + 11008 * 4096
    small = ctypes.c_size_t(0)
    assert lib.sq_alpha_search_workspace(1, 128, 256, 512, 4, ctypes.byref(small)) == OK
    assert small.value < need

    xb = (ctypes.c_void_p * 2)(A, A)
    al = (ctypes.c_float * 4)(0.25, 0.5, 0.75, 1.0)
    mse = (ctypes.c_double * 4)()
    best = ctypes.c_int(-1)

    def call(batches=xb, xt=1, wt=1, alphas=al, na=4, wsp=A, wsb=None):
        return lib.sq_alpha_search(ctypes.cast(batches, P), xt, 2, 128, 512, P(A), wt, 256,
                                   ctypes.cast(alphas, P), na, P(wsp), need if wsb is None else wsb,
                                   ctypes.cast(mse, P), ctypes.byref(best), None)

    assert call(xt=1, wt=0) == DTYPE
    assert call(na=0) == SHAPE
    bad = (ctypes.c_float * 4)(0.25, 0.5, math.nan, 1.0)
    assert call(alphas=bad) == ALPHA
    assert call(wsb=16) == WORKSPACE
    assert call(wsp=0) == WORKSPACE
    nb = (ctypes.c_void_p * 2)(A, 0)
    assert call(batches=nb) == NULL
    mb = (ctypes.c_void_p * 2)(A, MIS)
    assert call(batches=mb) == ALIGN
    assert best.value == -1  # nothing written on error


def test_new_entries_exported(lib):
    for name in ("sq_act_scale", "sq_dynamic_quant_act", "sq_calib_sample_max_sum", "sq_calib_mean_finalize",
                 "sq_rmsnorm", "sq_fold_norm_weight", "sq_rmsnorm_quant_act"):
        assert name in capi.declared_functions()
        assert hasattr(lib, name)


def test_act_scale_and_dynamic_validation(lib):
    f = lib.sq_act_scale
    assert f(None, P(A), 1024, P(A), None) == NULL
    assert f(P(A), P(A), 1000, P(A), None) == SHAPE
    assert f(P(A), P(A), 1024, P(MIS), None) == ALIGN
    g = lib.sq_dynamic_quant_act
    base = [P(A), 1, 16, 1024, P(A), P(A), P(A), P(A), None]
    for i, code in ((4, NULL), (5, NULL), (6, NULL), (7, NULL)):
        a = list(base)
        a[i] = None
        assert g(*a) == code
    a = list(base)
    a[1] = 5
    assert g(*a) == DTYPE
    a = list(base)
    a[2] = -1
    assert g(*a) == SHAPE
    a = list(base)
    a[3] = 96
    assert g(*a) == SHAPE
    a = list(base)
    a[5] = P(MIS)
    assert g(*a) == ALIGN


def test_sample_max_validation(lib):
    f = lib.sq_calib_sample_max_sum
    base = [P(A), 1, 4, 512, 1024, P(A), P(A), None]
    a = list(base)
    a[6] = None
    assert f(*a) == NULL
    a = list(base)
    a[5] = None
    assert f(*a) == NULL
    a = list(base)
    a[3] = 0
    assert f(*a) == SHAPE
    a = list(base)
    a[2] = -1
    assert f(*a) == SHAPE
    a = list(base)
    a[6] = P(MIS)
    assert f(*a) == ALIGN
    # zero samples: nothing to do, x and sample_max may be NULL
    assert f(None, 1, 0, 512, 1024, None, P(A), None) == OK
    g = lib.sq_calib_mean_finalize
    assert g(P(A), 0, 1024, P(A), None) == SHAPE
    assert g(None, 4, 1024, P(A), None) == NULL
    assert g(P(A), 4, 1024, P(MIS), None) == ALIGN


def test_norm_validation(lib):
    f = lib.sq_rmsnorm
    base = [P(A), 1, 8, 1024, P(A), 1e-5, P(A), 1, None, None]
    a = list(base)
    a[4] = None
    assert f(*a) == NULL
    a = list(base)
    a[7] = 9
    assert f(*a) == DTYPE
    for bad in (float("nan"), float("inf"), -1e-6):
        a = list(base)
        a[5] = bad
        assert f(*a) == SHAPE
    a = list(base)
    a[8] = P(MIS)
    assert f(*a) == ALIGN
    g = lib.sq_fold_norm_weight
    assert g(P(A), None, 1024, P(A), None) == NULL
    assert g(P(A), P(A), 100, P(A), None) == SHAPE
    h = lib.sq_rmsnorm_quant_act
    base = [P(A), 1, 8, 1024, P(A), 1e-5, P(A), P(A), None, None]
    a = list(base)
    a[6] = None
    assert h(*a) == NULL
    a = list(base)
    a[3] = 1000
    assert h(*a) == SHAPE
    a = list(base)
    a[7] = P(MIS)
    assert h(*a) == ALIGN
    a = list(base)
    a[2] = 0
    assert h(*a) == OK


def test_percentile_validation(lib):
    n = ctypes.c_size_t(0)
    assert lib.sq_calib_percentile_workspace(1, 1024, None) == NULL
    assert lib.sq_calib_percentile_workspace(5, 1024, ctypes.byref(n)) == DTYPE
    assert lib.sq_calib_percentile_workspace(1, 1000, ctypes.byref(n)) == SHAPE
    assert lib.sq_calib_percentile_workspace(1, 1024, ctypes.byref(n)) == OK
    need = n.value
    assert need >= 2 * 1024 * 256 * 4
    f4 = ctypes.c_size_t(0)
    assert lib.sq_calib_percentile_workspace(0, 1024, ctypes.byref(f4)) == OK and f4.value > need
    f = lib.sq_calib_percentile
    base = [P(A), 1, 4096, 1024, 0.999, P(A), need, P(A), None]
    a = list(base)
    a[0] = None
    assert f(*a) == NULL
    for bad in (float("nan"), -0.1, 1.5):
        a = list(base)
        a[4] = bad
        assert f(*a) == SHAPE
    a = list(base)
    a[2] = 0
    assert f(*a) == SHAPE
    a = list(base)
    a[6] = need - 1
    assert f(*a) == WORKSPACE
    a = list(base)
    a[5] = None
    assert f(*a) == WORKSPACE
    a = list(base)
    a[7] = P(MIS)
    assert f(*a) == ALIGN


def test_fp8_validation(lib):
    for name in ("sq_act_scale_fp8", "sq_quant_weight_fp8", "sq_smooth_quant_act_fp8", "sq_fp8_gemm"):
        assert name in capi.declared_functions() and hasattr(lib, name)
    assert lib.sq_act_scale_fp8(P(A), None, 1024, P(A), None) == NULL
    assert lib.sq_act_scale_fp8(P(A), P(A), 1000, P(A), None) == SHAPE
    f = lib.sq_quant_weight_fp8
    assert f(P(A), 1, 8, 1024, None, P(A), P(A), None) == NULL
    assert f(P(A), 4, 8, 1024, P(A), P(A), P(A), None) == DTYPE
    assert f(P(A), 1, 8, 1056, P(A), P(A), P(A), None) == SHAPE
    assert f(P(A), 1, 8, 1024, P(A), P(MIS), P(A), None) == ALIGN
    g = lib.sq_smooth_quant_act_fp8
    assert g(P(A), 1, 8, 1024, P(A), None, P(A), None) == NULL
    assert g(P(MIS), 1, 8, 1024, P(A), P(A), P(A), None) == ALIGN
    assert g(None, 1, 0, 1024, P(A), P(A), None, None) == OK
    h = lib.sq_fp8_gemm
    base = [P(A), P(A), 16, 32, 1024, P(A), P(A), P(A), 1, None, None]
    a = list(base)
    a[5] = None
    assert h(*a) == NULL
    a = list(base)
    a[4] = 131072 + 64
    assert h(*a) == SHAPE
    a = list(base)
    a[9] = P(MIS)
    assert h(*a) == ALIGN
    a = list(base)
    a[3] = 0
    assert h(*a) == OK


def _arr(ctype, values):
    a = (ctype * len(values))(*values)
    return a, ctypes.cast(a, P)


def test_batched_validation(lib):
    for name in ("sq_calib_absmax_batched", "sq_smooth_factors_batched", "sq_quant_weight_batched"):
        assert name in capi.declared_functions() and hasattr(lib, name)
    B = 0x100000  # a second fake address, 1 MiB past A
    i64, i32, f32 = ctypes.c_int64, ctypes.c_int, ctypes.c_float

    # absmax: two bf16 inputs of 16 x 1024
    def absmax(count, xs, dts, rows, ks, outs, acc=0):
        keep = [_arr(P, xs), _arr(i32, dts), _arr(i64, rows), _arr(i64, ks), _arr(P, outs)]
        return lib.sq_calib_absmax_batched(count, *[p for _, p in keep], acc, None)

    good = ([A, B], [1, 1], [16, 16], [1024, 1024], [A + 0x40000, B + 0x40000])
    assert lib.sq_calib_absmax_batched(2, None, None, None, None, None, 0, None) == NULL
    assert absmax(0, *good) == SHAPE
    assert absmax(17, *[v * 9 for v in good]) == SHAPE
    bad = [list(v) for v in good]
    bad[1][1] = 7  # item 1: dtype
    assert absmax(2, *bad) == DTYPE
    bad = [list(v) for v in good]
    bad[3][0] = 1000  # item 0: k
    bad[4][1] = MIS   # item 1: misaligned (item 0 fails first)
    assert absmax(2, *bad) == SHAPE
    bad = [list(v) for v in good]
    bad[4][1] = bad[4][0] + 16  # outputs of items 0 and 1 overlap
    assert absmax(2, *bad) == SHAPE
    bad = [list(v) for v in good]
    bad[4][1] = A + 64  # item 1 writes into item 0's input
    assert absmax(2, *bad) == SHAPE
    # zero rows into running maxima: nothing to launch
    assert absmax(2, [0, 0], [1, 1], [0, 0], [1024, 1024], good[4], acc=1) == OK

    # smoothing: outputs of two items overlapping, alpha of item 1 invalid
    def smooth(count, am, wm, ks, al, s, inv, sc):
        keep = [_arr(P, am), _arr(P, wm), _arr(i64, ks), _arr(f32, al), _arr(P, s), _arr(P, inv), _arr(P, sc)]
        return lib.sq_smooth_factors_batched(count, *[p for _, p in keep], None)

    sg = ([A, A], [A + 0x1000, A + 0x2000], [256, 256], [0.5, 0.5], [B, B + 0x1000], [B + 0x2000, B + 0x3000],
          [B + 0x4000, B + 0x4010])
    assert lib.sq_smooth_factors_batched(2, *([None] * 7), None) == NULL
    bad = [list(v) for v in sg]
    bad[3][1] = 1.5
    assert smooth(2, *bad) == ALPHA
    bad = [list(v) for v in sg]
    bad[6][1] = bad[6][0]  # both items write one act_scale
    assert smooth(2, *bad) == SHAPE
    bad = [list(v) for v in sg]
    bad[4][1] = A  # item 1's s over the shared statistic act_max
    assert smooth(2, *bad) == SHAPE

    # weight quant
    def qw(count, w, wt, n, ks, s, wq, wsc):
        keep = [_arr(P, w), _arr(i32, wt), _arr(i64, n), _arr(i64, ks), _arr(P, s), _arr(P, wq), _arr(P, wsc)]
        return lib.sq_quant_weight_batched(count, *[p for _, p in keep], None)

    qg = ([A, A + 0x10000], [1, 1], [8, 8], [1024, 1024], [B, B], [B + 0x1000, B + 0x4000], [B + 0x8000, B + 0x8100])
    assert lib.sq_quant_weight_batched(2, *([None] * 7), None) == NULL
    bad = [list(v) for v in qg]
    bad[2][1] = -1
    assert qw(2, *bad) == SHAPE
    bad = [list(v) for v in qg]
    bad[5][1] = bad[5][0] + 8192  # 8 x 1024 codes of item 0 end exactly where item 1's start: no overlap ...
    bad[6][1] = bad[6][0] + 16    # ... but the w_scale ranges (32 bytes each) overlap
    assert qw(2, *bad) == SHAPE
    bad = [list(v) for v in qg]
    bad[4][1] = MIS
    assert qw(2, *bad) == ALIGN


def test_batched_act_and_gemm_validation(lib):
    for name in ("sq_smooth_quant_act_batched", "sq_w8a8_gemm_batched"):
        assert name in capi.declared_functions() and hasattr(lib, name)
    B = 0x100000
    i64, i32 = ctypes.c_int64, ctypes.c_int

    def act(count, xs, dts, ms, ks, inv, sc, xq):
        keep = [_arr(P, xs), _arr(i32, dts), _arr(i64, ms), _arr(i64, ks), _arr(P, inv), _arr(P, sc), _arr(P, xq)]
        return lib.sq_smooth_quant_act_batched(count, *[p for _, p in keep], None)

    # two consumers of one input (shared x is allowed)
    ag = ([A, A], [1, 1], [16, 16], [1024, 1024], [B, B + 0x1000], [B + 0x2000, B + 0x2010],
          [B + 0x10000, B + 0x20000])
    assert lib.sq_smooth_quant_act_batched(2, *([None] * 7), None) == NULL
    assert act(0, *ag) == SHAPE
    bad = [list(v) for v in ag]
    bad[3][1] = 1000
    assert act(2, *bad) == SHAPE
    bad = [list(v) for v in ag]
    bad[6][1] = bad[6][0] + 8192  # 16 x 1024 codes of item 0 overlap item 1's output
    assert act(2, *bad) == SHAPE
    bad = [list(v) for v in ag]
    bad[6][1] = A + 1024  # item 1 writes into the input
    assert act(2, *bad) == SHAPE
    bad = [list(v) for v in ag]
    bad[1][0] = 5
    assert act(2, *bad) == DTYPE

    def gemm(count, xq, wq, ms, ns, ks, sc, ws, ys, yts, acc):
        keep = [_arr(P, xq), _arr(P, wq), _arr(i64, ms), _arr(i64, ns), _arr(i64, ks), _arr(P, sc), _arr(P, ws),
                _arr(P, ys), _arr(i32, yts)]
        acc_arr = _arr(P, acc) if acc is not None else (None, None)
        return lib.sq_w8a8_gemm_batched(count, *[p for _, p in keep], acc_arr[1], None)

    gg = ([A, A], [A + 0x40000, A + 0x80000], [64, 64], [128, 128], [1024, 1024], [B, B], [B + 0x100, B + 0x300],
          [B + 0x10000, B + 0x20000], [1, 1], None)
    assert lib.sq_w8a8_gemm_batched(2, *([None] * 10), None, None) == NULL
    assert gemm(17, *[v * 9 if isinstance(v, list) else v for v in gg]) == SHAPE
    bad = [list(v) if isinstance(v, list) else v for v in gg]
    bad[4][0] = 131072 + 64  # k above SQ_MAX_GEMM_K, the exact-accumulator limit
    assert gemm(2, *bad) == SHAPE
    bad = [list(v) if isinstance(v, list) else v for v in gg]
    bad[7][1] = bad[7][0] + 64  # the two outputs overlap
    assert gemm(2, *bad) == SHAPE
    bad = [list(v) if isinstance(v, list) else v for v in gg]
    bad[9] = [None, MIS]  # item 1's acc_out misaligned
    assert gemm(2, *bad) == ALIGN
    bad = [list(v) if isinstance(v, list) else v for v in gg]
    bad[9] = [bad[7][1], None]  # item 0's acc_out over item 1's y
    assert gemm(2, *bad) == SHAPE


def test_rmsnorm_quant_multi_validation(lib):
    PP = ctypes.c_void_p * 3
    f = lib.sq_rmsnorm_quant_act_multi
    H, G0, G1, G2, S0, S1, S2, Q0, Q1, Q2 = (A + i * 0x1000000 for i in range(10))
    base = dict(h=H, ht=1, m=8, k=1024, eps=1e-5, n=3, g=PP(G0, G1, G2), a=PP(S0, S1, S2), q=PP(Q0, Q1, Q2), r=None)

    def call(**ch):
        v = dict(base, **ch)
        return f(P(v["h"]) if v["h"] is not None else None, v["ht"], v["m"], v["k"], ctypes.c_float(v["eps"]), v["n"],
                 v["g"], v["a"], v["q"], P(v["r"]) if v["r"] is not None else None, None)
    assert call(g=None) == NULL
    assert call(h=None) == NULL
    assert call(q=PP(Q0, None, Q2)) == NULL
    assert call(ht=9) == DTYPE
    assert call(n=0) == SHAPE
    assert call(n=5) == SHAPE
    assert call(k=1000) == SHAPE
    assert call(eps=-1.0) == SHAPE
    assert call(h=H + 8) == ALIGN
    assert call(q=PP(Q0, Q1 + 4, Q2)) == ALIGN
    assert call(q=PP(Q0, Q0 + 4096, Q2)) == SHAPE   # two consumers' codes overlap
    assert call(q=PP(Q0, G1, Q2)) == SHAPE          # codes on a consumer's folded weight
    assert call(q=PP(Q0, Q1, H + 1024)) == SHAPE    # codes on h
    assert call(r=G2) == SHAPE                      # r on a folded weight


def test_act_scale_batched_validation(lib):
    PP = ctypes.c_void_p * 2
    I64 = ctypes.c_int64 * 2
    a, b = A, A + 0x100000
    f = lib.sq_act_scale_batched
    assert f(2, None, PP(a, b), I64(64, 64), PP(a + 0x200000, b + 0x200000), None) == NULL
    assert f(0, PP(a, b), PP(a, b), I64(64, 64), PP(a + 0x200000, b + 0x200000), None) == SHAPE
    assert f(2, PP(a, b), PP(a, b), I64(64, 100), PP(a + 0x200000, b + 0x200000), None) == SHAPE
    assert f(2, PP(a, MIS), PP(a, b), I64(64, 64), PP(a + 0x200000, b + 0x200000), None) == ALIGN
    assert f(2, PP(a, b), PP(a, b), I64(64, 64), PP(a + 0x200000, a), None) == SHAPE  # item 1's scale on item 0's act_max


def test_fp8_batched_validation(lib):
    """The batched FP8 forms share the int8 batched forms' checks."""
    PP = ctypes.c_void_p * 2
    I64 = ctypes.c_int64 * 2
    F = ctypes.c_float * 2
    I = ctypes.c_int * 2
    a, b = A, A + 0x100000
    ptrs = lambda *v: PP(*v)
    k = I64(1024, 1024)
    assert lib.sq_smooth_factors_fp8_batched(2, None, ptrs(a, b), k, F(0.5, 0.5), ptrs(a, b), ptrs(a, b),
                                             ptrs(a, b), None) == NULL
    assert lib.sq_smooth_factors_fp8_batched(17, ptrs(a, b), ptrs(a, b), k, F(0.5, 0.5), ptrs(a, b), ptrs(a, b),
                                             ptrs(a, b), None) == SHAPE
    assert lib.sq_smooth_factors_fp8_batched(2, ptrs(a, b), ptrs(a, b), k, F(0.5, 1.5), ptrs(a, b), ptrs(a, b),
                                             ptrs(a, b), None) == ALPHA
    assert lib.sq_quant_weight_fp8_batched(2, ptrs(a, b), I(1, 7), I64(8, 8), k, ptrs(a, b), ptrs(a, b),
                                           ptrs(a, b), None) == DTYPE
    assert lib.sq_smooth_quant_act_fp8_batched(2, ptrs(a, b), I(1, 1), I64(8, 8), I64(1024, 1000), ptrs(a, b),
                                               ptrs(a, b), ptrs(a, b), None) == SHAPE
    assert lib.sq_fp8_gemm_batched(2, ptrs(a, b), ptrs(a, b), I64(8, 8), I64(16, 16), k, ptrs(a, b), ptrs(a, b),
                                   ptrs(a + 4, b), I(1, 1), None, None) == ALIGN
    # item 1's output on item 0's weight codes
    x0, w0, y0, x1, w1 = (A + i * 0x100000 for i in range(5))
    assert lib.sq_fp8_gemm_batched(2, ptrs(x0, x1), ptrs(w0, w1), I64(8, 8), I64(16, 16), k,
                                   ptrs(A + 0x600000, A + 0x700000), ptrs(A + 0x800000, A + 0x900000),
                                   ptrs(y0, w0), I(1, 1), None, None) == SHAPE


def test_f16_scale_validation(lib):
    """The fp16-scale entry points: the fp32 forms' checks; smoothing writes
    no inv_s (none is taken); the overlap rule counts 2-byte scales."""
    names = ("sq_smooth_factors_f16", "sq_quant_weight_f16", "sq_smooth_quant_act_f16", "sq_w8a8_gemm_f16",
             "sq_smooth_factors_f16_batched", "sq_quant_weight_f16_batched", "sq_smooth_quant_act_f16_batched",
             "sq_w8a8_gemm_f16_batched")
    for name in names:
        assert name in capi.declared_functions() and hasattr(lib, name)
    sf = lib.sq_smooth_factors_f16
    assert sf(P(A), P(A), 1024, 0.5, None, P(A), None) == NULL
    assert sf(P(A), P(A), 1024, 0.5, P(A), None, None) == NULL
    assert sf(P(A), P(A), 1000, 0.5, P(A), P(A), None) == SHAPE
    assert sf(P(A), P(A), 1024, 1.5, P(A), P(A), None) == ALPHA
    assert sf(P(A), P(A), 1024, float("nan"), P(A), P(A), None) == ALPHA
    assert sf(P(A), P(A), 1024, 0.5, P(A), P(MIS), None) == ALIGN
    f = lib.sq_quant_weight_f16
    assert f(P(A), 1, 8, 1024, None, P(A), P(A), None) == NULL
    assert f(P(A), 4, 8, 1024, P(A), P(A), P(A), None) == DTYPE
    assert f(P(A), 1, 8, 1056, P(A), P(A), P(A), None) == SHAPE
    assert f(P(A), 1, -1, 1024, P(A), P(A), P(A), None) == SHAPE
    assert f(P(A), 1, 8, 1024, P(A), P(A), P(MIS), None) == ALIGN
    assert f(None, 1, 0, 1024, P(A), None, None, None) == OK
    g = lib.sq_smooth_quant_act_f16
    assert g(P(A), 1, 8, 1024, P(A), None, P(A), None) == NULL
    assert g(P(A), 1, 8, 1024, P(MIS), P(A), P(A), None) == ALIGN
    assert g(None, 1, 0, 1024, P(A), P(A), None, None) == OK
    h = lib.sq_w8a8_gemm_f16
    base = [P(A), P(A), 16, 32, 1024, P(A), P(A), P(A), 1, None, None]
    for idx, val, want in ((5, None, NULL), (4, 131072 + 64, SHAPE), (8, 5, DTYPE), (6, P(MIS), ALIGN),
                           (3, 0, OK)):
        a = list(base)
        a[idx] = val
        assert h(*a) == want, (idx, val)
    PP = ctypes.c_void_p * 2
    I64 = ctypes.c_int64 * 2
    F = ctypes.c_float * 2
    I = ctypes.c_int * 2
    a, b = A, A + 0x100000
    k = I64(1024, 1024)
    assert lib.sq_smooth_factors_f16_batched(2, PP(a, b), PP(a, b), k, F(0.5, 0.5), None, PP(a, b), None) == NULL
    assert lib.sq_smooth_factors_f16_batched(17, PP(a, b), PP(a, b), k, F(0.5, 0.5), PP(a, b), PP(a, b),
                                             None) == SHAPE
    assert lib.sq_smooth_factors_f16_batched(2, PP(a, b), PP(a, b), k, F(0.5, -0.5), PP(a, b), PP(a, b),
                                             None) == ALPHA
    # s of item 1 (2 KB of binary16) starting 1 KB into s of item 0: overlap
    assert lib.sq_smooth_factors_f16_batched(2, PP(A, A + 0x4000), PP(A + 0x8000, A + 0xc000), k, F(0.5, 0.5),
                                             PP(A + 0x10000, A + 0x10400), PP(A + 0x20000, A + 0x20010),
                                             None) == SHAPE
    # the same 2 KB apart: no overlap -- rejected only by a bad alpha, so no launch
    assert lib.sq_smooth_factors_f16_batched(2, PP(A, A + 0x4000), PP(A + 0x8000, A + 0xc000), k, F(0.5, 2.0),
                                             PP(A + 0x10000, A + 0x10800), PP(A + 0x20000, A + 0x20010),
                                             None) == ALPHA
    assert lib.sq_quant_weight_f16_batched(2, PP(a, b), I(1, 7), I64(8, 8), k, PP(a, b), PP(a, b), PP(a, b),
                                           None) == DTYPE
    assert lib.sq_smooth_quant_act_f16_batched(2, PP(a, b), I(1, 1), I64(8, 8), I64(1024, 1000), PP(a, b),
                                               PP(a, b), PP(a, b), None) == SHAPE
    assert lib.sq_w8a8_gemm_f16_batched(2, PP(a, b), PP(a, b), I64(8, 8), I64(16, 16), k, PP(a, b), PP(a, b),
                                        PP(a + 4, b), I(1, 1), None, None) == ALIGN


def test_ceiling_validation(lib):
    lib = ceiling.load()
    for name in ("sq_ceiling_mfma", "sq_ceiling_copy", "sq_ceiling_read", "sq_ceiling_narrow"):
        assert name in ceiling.declared_functions() and hasattr(lib, name)
    ops = ctypes.c_int64(0)
    assert lib.sq_ceiling_mfma(100, 1, P(A), None, ctypes.byref(ops), None) == NULL
    assert lib.sq_ceiling_mfma(100, 1, None, P(A), ctypes.byref(ops), None) == NULL
    assert lib.sq_ceiling_mfma(100, 1, P(A), P(A), None, None) == NULL
    assert lib.sq_ceiling_mfma(0, 1, P(A), P(A), ctypes.byref(ops), None) == SHAPE
    assert lib.sq_ceiling_mfma((1 << 24) + 1, 1, P(A), P(A), ctypes.byref(ops), None) == SHAPE
    assert lib.sq_ceiling_mfma(100, 9, P(A), P(A), ctypes.byref(ops), None) == SHAPE
    assert lib.sq_ceiling_mfma(100, 1, P(A), P(A + 2), ctypes.byref(ops), None) == ALIGN
    assert lib.sq_ceiling_mfma(100, 1, P(MIS), P(A), ctypes.byref(ops), None) == ALIGN
    assert lib.sq_ceiling_copy(None, P(A), 1024, None) == NULL
    assert lib.sq_ceiling_copy(P(A), P(A + 0x1000), 1000, None) == SHAPE
    assert lib.sq_ceiling_copy(P(A), P(A + 512), 1024, None) == SHAPE  # overlapping
    assert lib.sq_ceiling_copy(P(MIS), P(A + 0x1000), 1024, None) == ALIGN
    assert lib.sq_ceiling_copy(None, None, 0, None) == OK
    assert lib.sq_ceiling_read(P(A), 1024, None, None) == NULL
    assert lib.sq_ceiling_read(None, 1024, P(A), None) == NULL
    assert lib.sq_ceiling_read(P(A), 1000, P(A), None) == SHAPE
    assert lib.sq_ceiling_read(P(MIS), 1024, P(A), None) == ALIGN
    assert lib.sq_ceiling_read(P(A), 1024, P(A + 2), None) == ALIGN
    assert lib.sq_ceiling_read(None, 0, P(A), None) == OK
    assert lib.sq_ceiling_narrow(None, P(A), 1024, None) == NULL
    assert lib.sq_ceiling_narrow(P(A), P(A + 0x1000), 1000, None) == SHAPE
    assert lib.sq_ceiling_narrow(P(A), P(A + 256), 1024, None) == SHAPE  # dst inside src
    assert lib.sq_ceiling_narrow(P(A + 0x1000), P(A + 0x1000 - 256), 1024, None) == SHAPE  # dst runs into src
    assert lib.sq_ceiling_narrow(P(MIS), P(A + 0x1000), 1024, None) == ALIGN
    assert lib.sq_ceiling_narrow(P(A), P(A + 0x1004), 1024, None) == ALIGN
    assert lib.sq_ceiling_narrow(None, None, 0, None) == OK


def test_ceiling_chain_dots():
    """The host side of the MFMA loop's check: all-ones operands give 32 per
    chain; one nonzero byte pair at lane 32 lands in its own chain only; bytes
    of lanes other than 0 and 32 do not enter element 0."""
    import numpy as np
    assert ceiling.ceiling_chain_dots(np.ones(16384, np.int8)) == [32] * 8
    o = np.zeros((16, 64, 16), np.int8)
    o[2 * 3, 32, 5], o[2 * 3 + 1, 32, 5] = -7, 9
    o[2 * 5, 1, 0], o[2 * 5 + 1, 1, 0] = 100, 100  # lane 1: row 1 of A, column 1 of B
    o[2 * 6, 0, 2], o[2 * 6 + 1, 0, 3] = 50, 50  # different K positions
    assert ceiling.ceiling_chain_dots(o.reshape(-1)) == [0, 0, 0, -63, 0, 0, 0, 0]
    assert ceiling.ceiling_expected_sink(o.reshape(-1), 3, 10) == (-63 * 30) % (1 << 32)


# ---- the Python binding checks every tensor against the sizes it passes ------------------

def _expect_value_error(call, *words):
    with pytest.raises(ValueError) as e:
        call()
    msg = str(e.value)
    for w in words:
        assert w in msg, (w, msg)


def test_binding_rejects_mismatched_outputs_before_launch():
    """Wrong output shapes, element types and sizes raise ValueError naming the
    argument; CPU tensors with every size right fail only at the GPU check.
    No call reaches the library (these are CPU tensors)."""
    import torch
    bf, f32, i8, u8, i32 = torch.bfloat16, torch.float32, torch.int8, torch.uint8, torch.int32
    m, n, k = 64, 32, 128
    x = torch.zeros(m, k, dtype=bf)
    xq, wq = torch.zeros(m, k, dtype=i8), torch.zeros(n, k, dtype=i8)
    a, ws, y = torch.ones(4), torch.ones(n), torch.zeros(m, n, dtype=bf)
    e = _expect_value_error
    e(lambda: capi.sq_calib_absmax(x, torch.zeros(k - 64)), "absmax", "shape")
    e(lambda: capi.sq_calib_absmax(x, torch.zeros(k, dtype=torch.float64)), "absmax", "dtype")
    e(lambda: capi.sq_smooth_factors(torch.ones(k), torch.ones(k), 0.5, torch.ones(k), torch.ones(k - 1), a),
      "inv_s", "shape")
    e(lambda: capi.sq_smooth_factors(torch.ones(k), torch.ones(k), 0.5, torch.ones(k), torch.ones(k), torch.ones(0)),
      "act_scale", "elements")
    e(lambda: capi.sq_quant_weight(x, torch.ones(k), torch.zeros(m, k, dtype=u8), torch.ones(m)), "wq", "dtype")
    e(lambda: capi.sq_quant_weight(x, torch.ones(k), torch.zeros(m, k, dtype=i8), torch.ones(m - 1)), "w_scale")
    e(lambda: capi.sq_smooth_quant_act(x, torch.ones(k), a, torch.zeros(m, k - 64, dtype=i8)), "xq", "shape")
    e(lambda: capi.sq_smooth_quant_act(x, torch.ones(k), a, torch.zeros(m, k, dtype=u8)), "xq", "dtype")
    e(lambda: capi.sq_w8a8_gemm(xq, wq, a, ws, torch.zeros(m, n - 1, dtype=bf)), "y", "shape")
    e(lambda: capi.sq_w8a8_gemm(xq, torch.zeros(n, k + 64, dtype=i8), a, ws, y), "wq", "k")
    e(lambda: capi.sq_w8a8_gemm(xq, wq, a, torch.ones(n - 16), y), "w_scale", "shape")
    e(lambda: capi.sq_w8a8_gemm(xq, wq, a, ws, y, torch.zeros(m, n, dtype=f32)), "acc_out", "dtype")
    e(lambda: capi.sq_w8a8_gemm(xq, wq, a, ws, torch.zeros(m, n, dtype=torch.float16)), "y", "dtype")
    e(lambda: capi.sq_dynamic_quant_act(x, torch.ones(k), torch.ones(k - 64), a, xq), "live_max")
    e(lambda: capi.sq_rmsnorm(x, torch.ones(k), 1e-5, torch.zeros(m, k + 64, dtype=bf)), "y", "shape")
    e(lambda: capi.sq_rmsnorm_quant_act(x, torch.ones(k), 1e-5, a, xq, torch.ones(m - 1)), "r_out")
    e(lambda: capi.sq_calib_sample_max_sum(x, 4, torch.zeros(4, k), torch.zeros(k)), "sum", "dtype")
    e(lambda: capi.sq_calib_sample_max_sum(x, 4, torch.zeros(2, k), torch.zeros(k, dtype=torch.float64)),
      "sample_max")
    e(lambda: capi.sq_calib_percentile(x, 0.999, torch.zeros(16, dtype=u8), torch.zeros(k - 64)), "act_max")
    # FP8 variant: codes are uint8, accumulators fp32
    xq8, wq8 = torch.zeros(m, k, dtype=u8), torch.zeros(n, k, dtype=u8)
    e(lambda: capi.sq_fp8_gemm(xq, wq, a, ws, y), "xq", "dtype")
    e(lambda: capi.sq_fp8_gemm(xq8, wq8, a, ws, y, torch.zeros(m, n, dtype=i32)), "acc_out", "dtype")
    e(lambda: capi.sq_quant_weight_fp8(x, torch.ones(k), torch.zeros(m, k, dtype=i8), torch.ones(m)), "wq")
    # fp16 scale storage: every scale a float16 tensor
    f16 = torch.float16
    s16, a16, ws16 = torch.ones(k, dtype=f16), torch.ones(4, dtype=f16), torch.ones(n, dtype=f16)
    e(lambda: capi.sq_smooth_factors_f16(torch.ones(k), torch.ones(k), 0.5, torch.ones(k), a16), "s", "dtype")
    e(lambda: capi.sq_smooth_factors_f16(torch.ones(k), torch.ones(k), 0.5, s16, torch.ones(0, dtype=f16)),
      "act_scale", "elements")
    e(lambda: capi.sq_quant_weight_f16(x, torch.ones(k), torch.zeros(m, k, dtype=i8), torch.ones(m, dtype=f16)),
      "s", "dtype")
    e(lambda: capi.sq_quant_weight_f16(x, s16, torch.zeros(m, k, dtype=i8), torch.ones(m)), "w_scale", "dtype")
    e(lambda: capi.sq_smooth_quant_act_f16(x, s16, a, xq), "act_scale", "dtype")
    e(lambda: capi.sq_w8a8_gemm_f16(xq, wq, a16, ws, y), "w_scale", "dtype")
    e(lambda: capi.sq_w8a8_gemm_f16(xq, wq, a16, torch.ones(n - 1, dtype=f16), y), "w_scale", "shape")
    e(lambda: capi.sq_w8a8_gemm_f16_batched([xq], [wq], [a], [ws16], [y]), "act_scale[0]", "dtype")
    e(lambda: capi.sq_smooth_quant_act_f16_batched([x], [torch.ones(k)], [a16], [xq]), "inv_ss[0]", "dtype")
    e(lambda: capi.sq_quant_weight_f16_batched([x], [s16], [torch.zeros(m, k, dtype=i8)], [torch.ones(m)]),
      "w_scales[0]", "dtype")
    e(lambda: capi.sq_smooth_factors_f16_batched([torch.ones(k)], [torch.ones(k)], [0.5], [torch.ones(k)], [a16]),
      "ss[0]", "dtype")
    e(lambda: capi.sq_w8a8_gemm_f16(xq, wq, a16, ws16, y), "GPU")
    # batched forms name the item
    e(lambda: capi.sq_w8a8_gemm_batched([xq, xq], [wq, wq], [a, a], [ws, ws], [y, torch.zeros(m, n + 1, dtype=bf)]),
      "y[1]", "shape")
    e(lambda: capi.sq_calib_absmax_batched([x, x], [torch.zeros(k), torch.zeros(k + 64)]), "absmaxes[1]")
    e(lambda: capi.sq_quant_weight_batched([x], [torch.ones(k)], [torch.zeros(m, k, dtype=u8)], [torch.ones(m)]),
      "wqs[0]", "dtype")
    e(lambda: capi.sq_quant_weight_fp8_batched([x], [torch.ones(k)], [torch.zeros(m, k, dtype=i8)],
                                               [torch.ones(m)]), "wqs[0]", "dtype")
    e(lambda: capi.sq_smooth_quant_act_batched([x], [torch.ones(k)], [a], [torch.zeros(m, k, dtype=u8)]), "xqs[0]")
    e(lambda: capi.sq_act_scale_batched([torch.ones(k)], [torch.ones(k + 64)], [a]), "inv_ss[0]")
    e(lambda: capi.sq_w8a8_gemm_batched([], [], [], [], []), "at least one")
    e(lambda: capi.sq_rmsnorm_quant_act_multi(x, [torch.ones(k), torch.ones(k - 64)], 1e-5, [a, a], [xq, xq]),
      "gammas_folded[1]")
    # everything right, but host tensors: rejected at the GPU check, still before any launch
    e(lambda: capi.sq_w8a8_gemm(xq, wq, a, ws, y), "GPU")
    e(lambda: capi.sq_calib_absmax(x, torch.zeros(k)), "GPU")


def test_percentile_noalloc_validation(lib):
    """The allocation-free percentile: the percentile's argument rules, and
    problems whose scratch exceeds the static array rejected before launch."""
    f = lib.sq_calib_percentile_noalloc
    assert f(None, 1, 1024, 1024, 0.999, P(A), None) == NULL
    assert f(P(A), 1, 1024, 1024, 0.999, None, None) == NULL
    assert f(P(A), 3, 1024, 1024, 0.999, P(A), None) == DTYPE
    assert f(P(A), 1, 0, 1024, 0.999, P(A), None) == SHAPE
    assert f(P(A), 1, 1024, 1000, 0.999, P(A), None) == SHAPE
    assert f(P(A), 1, 1024, 1024, 1.5, P(A), None) == SHAPE
    assert f(P(A), 1, 1024, 1024, float("nan"), P(A), None) == SHAPE
    SCRATCH = 8
    assert capi.SQ_PERCENTILE_SCRATCH_BYTES == 32 << 20
    # the largest widths that fit (bf16: 2 digit passes, fp32: 4) and the next ones
    for dt, kmax in ((1, 16320), (0, 8128)):
        assert capi.sq_calib_percentile_workspace(kmax, dt) <= capi.SQ_PERCENTILE_SCRATCH_BYTES
        assert capi.sq_calib_percentile_workspace(kmax + 64, dt) > capi.SQ_PERCENTILE_SCRATCH_BYTES
        assert f(P(A), dt, 1024, kmax + 64, 0.999, P(A), None) == SCRATCH
    assert f(P(MIS), 1, 1024, 1024, 0.999, P(A), None) == ALIGN
    assert lib.sq_status_string(SCRATCH) != b"unknown status"
