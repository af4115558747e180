"""Thin Python binding over libsq's C ABI (include/sq.h).

Argument marshalling only: each function takes torch tensors that already
live on the GPU, checks dtype/contiguity, and passes raw device pointers, the
shapes and the current HIP stream to the entry point of the same name. Every
step of the computation runs in the library's HIP kernels. There is no
fallback: if libsq.so is missing or fails to load, the call raises.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsq.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "sq.h")

SQ_F32, SQ_BF16 = 0, 1
STATUS = {0: "SQ_OK", 1: "SQ_ERR_NULL", 2: "SQ_ERR_SHAPE", 3: "SQ_ERR_DTYPE", 4: "SQ_ERR_ALPHA",
          5: "SQ_ERR_WORKSPACE", 6: "SQ_ERR_HIP", 7: "SQ_ERR_ALIGN"}
ALPHA_GRID = (0.25, 0.5, 0.75, 1.0)

_lib = None
_lock = threading.Lock()


class SQError(RuntimeError):
    def __init__(self, name: str, status: int, message: str):
        super().__init__(f"{name}: {STATUS.get(status, status)} ({message})")
        self.status = status


def declared_functions(header: str = HEADER) -> list[str]:
    """Names of the functions include/sq.h declares."""
    text = open(header).read()
    return sorted(set(re.findall(r"^\s*(?:sq_status|const char\*)\s+(sq_\w+)\s*\(", text, re.M)))


def _declare(lib):
    c = ctypes
    P, i64, St = c.c_void_p, c.c_int64, c.c_int
    sigs = {
        "sq_calib_absmax": [P, c.c_int, i64, i64, P, c.c_int, P],
        "sq_smooth_factors": [P, P, i64, c.c_float, P, P, P, P],
        "sq_quant_weight": [P, c.c_int, i64, i64, P, P, P, P],
        "sq_smooth_quant_act": [P, c.c_int, i64, i64, P, P, P, P],
        "sq_w8a8_gemm": [P, P, i64, i64, i64, P, P, P, c.c_int, P, P],
        "sq_alpha_search_workspace": [c.c_int, i64, i64, i64, c.c_int, P],
        "sq_gemm_tiling": [i64, i64, P, P],
        "sq_alpha_search": [P, c.c_int, c.c_int, i64, i64, P, c.c_int, i64, P, c.c_int, P, c.c_size_t, P, P, P],
        "sq_act_scale": [P, P, i64, P, P],
        "sq_dynamic_quant_act": [P, c.c_int, i64, i64, P, P, P, P, P],
        "sq_calib_sample_max_sum": [P, c.c_int, i64, i64, i64, P, P, P],
        "sq_calib_mean_finalize": [P, i64, i64, P, P],
        "sq_calib_percentile_workspace": [c.c_int, i64, P],
        "sq_calib_percentile": [P, c.c_int, i64, i64, c.c_double, P, c.c_size_t, P, P],
        "sq_rmsnorm": [P, c.c_int, i64, i64, P, c.c_float, P, c.c_int, P, P],
        "sq_act_scale_fp8": [P, P, i64, P, P],
        "sq_quant_weight_fp8": [P, c.c_int, i64, i64, P, P, P, P],
        "sq_smooth_quant_act_fp8": [P, c.c_int, i64, i64, P, P, P, P],
        "sq_fp8_gemm": [P, P, i64, i64, i64, P, P, P, c.c_int, P, P],
        "sq_fold_norm_weight": [P, P, i64, P, P],
        "sq_rmsnorm_quant_act": [P, c.c_int, i64, i64, P, c.c_float, P, P, P, P],
        "sq_calib_absmax_batched": [c.c_int, P, P, P, P, P, c.c_int, P],
        "sq_smooth_factors_batched": [c.c_int, P, P, P, P, P, P, P, P],
        "sq_quant_weight_batched": [c.c_int, P, P, P, P, P, P, P, P],
        "sq_smooth_quant_act_batched": [c.c_int, P, P, P, P, P, P, P, P],
        "sq_w8a8_gemm_batched": [c.c_int, P, P, P, P, P, P, P, P, P, P, P],
        "sq_smooth_factors_fp8_batched": [c.c_int, P, P, P, P, P, P, P, P],
        "sq_act_scale_batched": [c.c_int, P, P, P, P, P],
        "sq_rmsnorm_quant_act_multi": [P, c.c_int, i64, i64, c.c_float, c.c_int, P, P, P, P, P],
        "sq_quant_weight_fp8_batched": [c.c_int, P, P, P, P, P, P, P, P],
        "sq_smooth_quant_act_fp8_batched": [c.c_int, P, P, P, P, P, P, P, P],
        "sq_fp8_gemm_batched": [c.c_int, P, P, P, P, P, P, P, P, P, P, P],
        "sq_ceiling_mfma": [i64, c.c_int, P, P, P, P],
        "sq_ceiling_copy": [P, P, i64, P],
        "sq_ceiling_read": [P, i64, P, P],
        "sq_ceiling_narrow": [P, P, i64, P],
    }
    for name, args in sigs.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = St
    lib.sq_status_string.argtypes = [c.c_int]
    lib.sq_status_string.restype = c.c_char_p
    return lib


def load(path: str = LIB_PATH):
    """Load libsq.so (raises if it is not built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
            _lib = _declare(ctypes.CDLL(path))
    return _lib


def _check(name: str, status: int):
    if status != 0:
        raise SQError(name, status, load().sq_status_string(status).decode())


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return SQ_F32
    if t.dtype == torch.bfloat16:
        return SQ_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t, what: str):
    if not t.is_cuda:
        raise ValueError(f"{what} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def sq_calib_absmax(x, absmax, accumulate: bool = False, stream=None):
    """absmax[j] = max(absmax[j] if accumulate else 0, max_t |x[t, j]|)."""
    rows, k = x.shape
    _check("sq_calib_absmax", load().sq_calib_absmax(_dev(x, "x"), _dtype_code(x), rows, k, _dev(absmax, "absmax"),
                                                     int(bool(accumulate)), _stream(stream)))
    return absmax


def sq_smooth_factors(act_max, w_max, alpha: float, s, inv_s, act_scale, stream=None):
    k = act_max.shape[0]
    _check("sq_smooth_factors", load().sq_smooth_factors(_dev(act_max, "act_max"), _dev(w_max, "w_max"), k,
                                                         float(alpha), _dev(s, "s"), _dev(inv_s, "inv_s"),
                                                         _dev(act_scale, "act_scale"), _stream(stream)))


def sq_quant_weight(w, s, wq, w_scale, stream=None):
    n, k = w.shape
    _check("sq_quant_weight", load().sq_quant_weight(_dev(w, "w"), _dtype_code(w), n, k, _dev(s, "s"),
                                                     _dev(wq, "wq"), _dev(w_scale, "w_scale"), _stream(stream)))


def sq_smooth_quant_act(x, inv_s, act_scale, xq, stream=None):
    m, k = x.shape
    _check("sq_smooth_quant_act", load().sq_smooth_quant_act(_dev(x, "x"), _dtype_code(x), m, k,
                                                             _dev(inv_s, "inv_s"), _dev(act_scale, "act_scale"),
                                                             _dev(xq, "xq"), _stream(stream)))


def sq_w8a8_gemm(xq, wq, act_scale, w_scale, y, acc_out=None, stream=None):
    m, k = xq.shape
    n = wq.shape[0]
    acc = _dev(acc_out, "acc_out") if acc_out is not None else ctypes.c_void_p(0)
    _check("sq_w8a8_gemm", load().sq_w8a8_gemm(_dev(xq, "xq"), _dev(wq, "wq"), m, n, k, _dev(act_scale, "act_scale"),
                                               _dev(w_scale, "w_scale"), _dev(y, "y"), _dtype_code(y), acc,
                                               _stream(stream)))


SQ_MAX_NORM_CONSUMERS = 4


def sq_rmsnorm_quant_act_multi(h, gammas_folded, eps: float, act_scales, xqs, r_out=None, stream=None):
    """sq_rmsnorm_quant_act for several consumers of one norm output (h read
    once when their folded weights fit in registers)."""
    m, k = h.shape
    n = len(gammas_folded)
    if not (len(act_scales) == n and len(xqs) == n):
        raise ValueError("per-consumer lists differ in length")
    g, a, q = _ptrs(gammas_folded, "gammas_folded"), _ptrs(act_scales, "act_scales"), _ptrs(xqs, "xqs")
    _check("sq_rmsnorm_quant_act_multi", load().sq_rmsnorm_quant_act_multi(
        _dev(h, "h"), _dtype_code(h), m, k, float(eps), n, g[1], a[1], q[1], _opt(r_out, "r_out"), _stream(stream)))


def sq_act_scale_batched(act_maxes, inv_ss, act_scales, stream=None):
    """sq_act_scale for several projections in one launch."""
    count = len(act_maxes)
    if not all(len(v) == count for v in (inv_ss, act_scales)):
        raise ValueError("per-item lists differ in length")
    keep = [_ptrs(act_maxes, "act_maxes"), _ptrs(inv_ss, "inv_ss"),
            _host_array(ctypes.c_int64, [t.shape[0] for t in act_maxes]), _ptrs(act_scales, "act_scales")]
    _check("sq_act_scale_batched", load().sq_act_scale_batched(count, *[a for _, a in keep], _stream(stream)))


def sq_smooth_factors_fp8_batched(act_maxes, w_maxes, alphas, ss, inv_ss, act_scales, stream=None):
    """sq_smooth_factors_batched with the act scales over 448 (e4m3 codes)."""
    sq_smooth_factors_batched(act_maxes, w_maxes, alphas, ss, inv_ss, act_scales, stream,
                              _name="sq_smooth_factors_fp8_batched")


def sq_quant_weight_fp8_batched(ws, ss, wqs, w_scales, stream=None):
    """sq_quant_weight_fp8 for several weights (uint8 e4m3 codes)."""
    sq_quant_weight_batched(ws, ss, wqs, w_scales, stream, _name="sq_quant_weight_fp8_batched")


def sq_smooth_quant_act_fp8_batched(xs, inv_ss, act_scales, xqs, stream=None):
    """sq_smooth_quant_act_fp8 for several projections in one launch."""
    sq_smooth_quant_act_batched(xs, inv_ss, act_scales, xqs, stream, _name="sq_smooth_quant_act_fp8_batched")


def sq_fp8_gemm_batched(xqs, wqs, act_scales, w_scales, ys, acc_outs=None, stream=None):
    """sq_fp8_gemm for several products (fp32 acc_outs when given)."""
    sq_w8a8_gemm_batched(xqs, wqs, act_scales, w_scales, ys, acc_outs, stream, _name="sq_fp8_gemm_batched")


def sq_gemm_tiling(m: int, n: int) -> tuple[int, int]:
    """Block tile (rows, columns) sq_w8a8_gemm uses for an m x n output."""
    bm, bn = ctypes.c_int(0), ctypes.c_int(0)
    _check("sq_gemm_tiling", load().sq_gemm_tiling(m, n, ctypes.byref(bm), ctypes.byref(bn)))
    return bm.value, bn.value


def sq_alpha_search_workspace(n_batches: int, rows_per_batch: int, n: int, k: int, n_alphas: int = 4) -> int:
    out = ctypes.c_size_t(0)
    _check("sq_alpha_search_workspace",
           load().sq_alpha_search_workspace(n_batches, rows_per_batch, n, k, n_alphas, ctypes.byref(out)))
    return out.value


def sq_alpha_search(x_batches, w, workspace, alphas=ALPHA_GRID, stream=None):
    """Returns (mse list, best index). Synchronises the stream."""
    nb = len(x_batches)
    rows, k = x_batches[0].shape
    n = w.shape[0]
    xt = _dtype_code(x_batches[0])
    for x in x_batches:
        if x.shape != (rows, k) or _dtype_code(x) != xt:
            raise ValueError("all batches must share shape and dtype")
    ptrs = (ctypes.c_void_p * nb)(*[_dev(x, "x_batches[i]").value for x in x_batches])
    al = (ctypes.c_float * len(alphas))(*[float(a) for a in alphas])
    mse = (ctypes.c_double * len(alphas))()
    best = ctypes.c_int(-1)
    _check("sq_alpha_search", load().sq_alpha_search(ctypes.cast(ptrs, ctypes.c_void_p), xt, nb, rows, k, _dev(w, "w"),
                                                     _dtype_code(w), n, ctypes.cast(al, ctypes.c_void_p), len(alphas),
                                                     _dev(workspace, "workspace"), workspace.numel() *
                                                     workspace.element_size(), ctypes.cast(mse, ctypes.c_void_p),
                                                     ctypes.byref(best), _stream(stream)))
    return list(mse), best.value


def _host_array(ctype, values):
    """A host array for a per-item argument of the batched entry points."""
    arr = (ctype * len(values))(*values)
    return arr, ctypes.cast(arr, ctypes.c_void_p)


def _ptrs(tensors, what: str):
    return _host_array(ctypes.c_void_p, [_dev(t, f"{what}[{i}]").value for i, t in enumerate(tensors)])


def sq_calib_absmax_batched(xs, absmaxes, accumulate: bool = False, stream=None):
    """sq_calib_absmax over several inputs in one zero fill + one reduction launch."""
    if len(xs) != len(absmaxes):
        raise ValueError("xs and absmaxes differ in length")
    keep = [_ptrs(xs, "xs"), _host_array(ctypes.c_int, [_dtype_code(x) for x in xs]),
            _host_array(ctypes.c_int64, [x.shape[0] for x in xs]), _host_array(ctypes.c_int64, [x.shape[1] for x in xs]),
            _ptrs(absmaxes, "absmaxes")]
    _check("sq_calib_absmax_batched", load().sq_calib_absmax_batched(len(xs), *[a for _, a in keep],
                                                                     int(bool(accumulate)), _stream(stream)))


def sq_smooth_factors_batched(act_maxes, w_maxes, alphas, ss, inv_ss, act_scales, stream=None,
                              _name="sq_smooth_factors_batched"):
    """sq_smooth_factors for several projections in two launches."""
    count = len(act_maxes)
    if not all(len(v) == count for v in (w_maxes, alphas, ss, inv_ss, act_scales)):
        raise ValueError("per-item lists differ in length")
    keep = [_ptrs(act_maxes, "act_maxes"), _ptrs(w_maxes, "w_maxes"),
            _host_array(ctypes.c_int64, [t.shape[0] for t in act_maxes]),
            _host_array(ctypes.c_float, [float(a) for a in alphas]), _ptrs(ss, "ss"), _ptrs(inv_ss, "inv_ss"),
            _ptrs(act_scales, "act_scales")]
    _check(_name, getattr(load(), _name)(count, *[a for _, a in keep], _stream(stream)))


def sq_quant_weight_batched(ws, ss, wqs, w_scales, stream=None, _name="sq_quant_weight_batched"):
    """sq_quant_weight for several weights, one launch per row-length class."""
    count = len(ws)
    if not all(len(v) == count for v in (ss, wqs, w_scales)):
        raise ValueError("per-item lists differ in length")
    keep = [_ptrs(ws, "ws"), _host_array(ctypes.c_int, [_dtype_code(w) for w in ws]),
            _host_array(ctypes.c_int64, [w.shape[0] for w in ws]), _host_array(ctypes.c_int64, [w.shape[1] for w in ws]),
            _ptrs(ss, "ss"), _ptrs(wqs, "wqs"), _ptrs(w_scales, "w_scales")]
    _check(_name, getattr(load(), _name)(count, *[a for _, a in keep], _stream(stream)))


def sq_smooth_quant_act_batched(xs, inv_ss, act_scales, xqs, stream=None, _name="sq_smooth_quant_act_batched"):
    """sq_smooth_quant_act for several projections in one launch (a shared
    input tensor is read once for all of its consumers)."""
    count = len(xs)
    if not all(len(v) == count for v in (inv_ss, act_scales, xqs)):
        raise ValueError("per-item lists differ in length")
    keep = [_ptrs(xs, "xs"), _host_array(ctypes.c_int, [_dtype_code(x) for x in xs]),
            _host_array(ctypes.c_int64, [x.shape[0] for x in xs]), _host_array(ctypes.c_int64, [x.shape[1] for x in xs]),
            _ptrs(inv_ss, "inv_ss"), _ptrs(act_scales, "act_scales"), _ptrs(xqs, "xqs")]
    _check(_name, getattr(load(), _name)(count, *[a for _, a in keep], _stream(stream)))


def sq_w8a8_gemm_batched(xqs, wqs, act_scales, w_scales, ys, acc_outs=None, stream=None,
                         _name="sq_w8a8_gemm_batched"):
    """sq_w8a8_gemm for several products; those with the same large tile and
    output type share one launch."""
    count = len(xqs)
    if not all(len(v) == count for v in (wqs, act_scales, w_scales, ys)):
        raise ValueError("per-item lists differ in length")
    keep = [_ptrs(xqs, "xqs"), _ptrs(wqs, "wqs"), _host_array(ctypes.c_int64, [x.shape[0] for x in xqs]),
            _host_array(ctypes.c_int64, [w.shape[0] for w in wqs]), _host_array(ctypes.c_int64, [x.shape[1] for x in xqs]),
            _ptrs(act_scales, "act_scales"), _ptrs(w_scales, "w_scales"), _ptrs(ys, "ys"),
            _host_array(ctypes.c_int, [_dtype_code(y) for y in ys])]
    acc = None
    if acc_outs is not None:
        if len(acc_outs) != count:
            raise ValueError("acc_outs differs in length")
        acc = _host_array(ctypes.c_void_p, [_opt(a, f"acc_outs[{i}]").value for i, a in enumerate(acc_outs)])
    _check(_name, getattr(load(), _name)(count, *[a for _, a in keep], acc[1] if acc else ctypes.c_void_p(0),
                                         _stream(stream)))


CEILING_OPERAND_BYTES = 16384


def sq_ceiling_mfma(iters: int, blocks_per_cu: int, operands, sink, stream=None) -> int:
    """MFMA-only loop on every compute unit over the 16 KiB of register
    operands in `operands`; returns the int8 ops it issues."""
    if operands.numel() * operands.element_size() != CEILING_OPERAND_BYTES:
        raise ValueError(f"operands must hold {CEILING_OPERAND_BYTES} bytes")
    ops = ctypes.c_int64(0)
    _check("sq_ceiling_mfma", load().sq_ceiling_mfma(iters, blocks_per_cu, _dev(operands, "operands"),
                                                     _dev(sink, "sink"), ctypes.byref(ops), _stream(stream)))
    return ops.value


def ceiling_chain_dots(operands) -> list:
    """Per chain, the dot product sq_ceiling_mfma adds to its sink per
    iteration: element 0 of a v_mfma_i32_32x32x32_i8 accumulator is row 0 of A
    times column 0 of B, whose 32 bytes are lanes 0 and 32 of each operand
    (the same byte order on both sides, so the pairing does not depend on how
    the instruction numbers K). `operands` is the host copy (16384 int8)."""
    import numpy as np
    o = np.asarray(operands, dtype=np.int8).reshape(16, 64, 16).astype(np.int64)
    return [int((np.concatenate([o[2 * c, 0], o[2 * c, 32]]) *
                 np.concatenate([o[2 * c + 1, 0], o[2 * c + 1, 32]])).sum()) for c in range(8)]


def ceiling_expected_sink(operands, iters: int, waves: int) -> int:
    """sink[0] after one sq_ceiling_mfma call from zero (mod 2^32)."""
    return (waves * iters * sum(ceiling_chain_dots(operands))) % (1 << 32)


def sq_ceiling_copy(src, dst, stream=None):
    """16-byte vector copy of src into dst (same number of bytes)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst differ in size")
    _check("sq_ceiling_copy", load().sq_ceiling_copy(_dev(src, "src"), _dev(dst, "dst"), nbytes, _stream(stream)))


def sq_ceiling_narrow(src, dst, stream=None):
    """Reads src, writes the first 8 bytes of every 16-byte vector of it to
    dst (half src's size)."""
    nbytes = src.numel() * src.element_size()
    if 2 * dst.numel() * dst.element_size() != nbytes:
        raise ValueError("dst must hold half of src's bytes")
    _check("sq_ceiling_narrow", load().sq_ceiling_narrow(_dev(src, "src"), _dev(dst, "dst"), nbytes,
                                                         _stream(stream)))


def sq_ceiling_read(src, sink, stream=None):
    """16-byte vector read of src, every 32-bit word XORed into sink[0]."""
    _check("sq_ceiling_read", load().sq_ceiling_read(_dev(src, "src"), src.numel() * src.element_size(),
                                                     _dev(sink, "sink"), _stream(stream)))


def _opt(t, what: str):
    return _dev(t, what) if t is not None else ctypes.c_void_p(0)


def sq_act_scale(act_max, inv_s, act_scale, stream=None):
    k = act_max.shape[0]
    _check("sq_act_scale", load().sq_act_scale(_dev(act_max, "act_max"), _dev(inv_s, "inv_s"), k,
                                               _dev(act_scale, "act_scale"), _stream(stream)))


def sq_dynamic_quant_act(x, inv_s, live_max, act_scale, xq, stream=None):
    m, k = x.shape
    _check("sq_dynamic_quant_act", load().sq_dynamic_quant_act(_dev(x, "x"), _dtype_code(x), m, k,
                                                               _dev(inv_s, "inv_s"), _dev(live_max, "live_max"),
                                                               _dev(act_scale, "act_scale"), _dev(xq, "xq"),
                                                               _stream(stream)))


def sq_calib_sample_max_sum(x, samples: int, sample_max, total, stream=None):
    rows, k = x.shape
    if samples < 1 or rows % samples:
        raise ValueError("rows must be a whole number of samples")
    _check("sq_calib_sample_max_sum", load().sq_calib_sample_max_sum(_dev(x, "x"), _dtype_code(x), samples,
                                                                     rows // samples, k,
                                                                     _dev(sample_max, "sample_max"),
                                                                     _dev(total, "sum"), _stream(stream)))


def sq_calib_mean_finalize(total, count: int, act_max, stream=None):
    k = total.shape[0]
    _check("sq_calib_mean_finalize", load().sq_calib_mean_finalize(_dev(total, "sum"), count, k,
                                                                   _dev(act_max, "act_max"), _stream(stream)))


def sq_rmsnorm(h, gamma, eps: float, y, r_out=None, stream=None):
    m, k = h.shape
    _check("sq_rmsnorm", load().sq_rmsnorm(_dev(h, "h"), _dtype_code(h), m, k, _dev(gamma, "gamma"), float(eps),
                                           _dev(y, "y"), _dtype_code(y), _opt(r_out, "r_out"), _stream(stream)))


def sq_fold_norm_weight(gamma, inv_s, gamma_folded, stream=None):
    k = gamma.shape[0]
    _check("sq_fold_norm_weight", load().sq_fold_norm_weight(_dev(gamma, "gamma"), _dev(inv_s, "inv_s"), k,
                                                             _dev(gamma_folded, "gamma_folded"), _stream(stream)))


def sq_rmsnorm_quant_act(h, gamma_folded, eps: float, act_scale, xq, r_out=None, stream=None):
    m, k = h.shape
    _check("sq_rmsnorm_quant_act", load().sq_rmsnorm_quant_act(_dev(h, "h"), _dtype_code(h), m, k,
                                                               _dev(gamma_folded, "gamma_folded"), float(eps),
                                                               _dev(act_scale, "act_scale"), _dev(xq, "xq"),
                                                               _opt(r_out, "r_out"), _stream(stream)))


def sq_calib_percentile_workspace(k: int, dtype_code: int = SQ_BF16) -> int:
    out = ctypes.c_size_t(0)
    _check("sq_calib_percentile_workspace", load().sq_calib_percentile_workspace(dtype_code, k, ctypes.byref(out)))
    return out.value


def sq_calib_percentile(x, q: float, workspace, act_max, stream=None):
    """act_max[j] = nearest-rank q-quantile of |x[:, j]|."""
    rows, k = x.shape
    _check("sq_calib_percentile", load().sq_calib_percentile(_dev(x, "x"), _dtype_code(x), rows, k, float(q),
                                                             _dev(workspace, "workspace"),
                                                             workspace.numel() * workspace.element_size(),
                                                             _dev(act_max, "act_max"), _stream(stream)))


# ---- FP8 (OCP E4M3) variant: codes are torch.uint8 tensors --------------------------

def sq_act_scale_fp8(act_max, inv_s, act_scale, stream=None):
    k = act_max.shape[0]
    _check("sq_act_scale_fp8", load().sq_act_scale_fp8(_dev(act_max, "act_max"), _dev(inv_s, "inv_s"), k,
                                                       _dev(act_scale, "act_scale"), _stream(stream)))


def sq_quant_weight_fp8(w, s, wq, w_scale, stream=None):
    n, k = w.shape
    _check("sq_quant_weight_fp8", load().sq_quant_weight_fp8(_dev(w, "w"), _dtype_code(w), n, k, _dev(s, "s"),
                                                             _dev(wq, "wq"), _dev(w_scale, "w_scale"),
                                                             _stream(stream)))


def sq_smooth_quant_act_fp8(x, inv_s, act_scale, xq, stream=None):
    m, k = x.shape
    _check("sq_smooth_quant_act_fp8", load().sq_smooth_quant_act_fp8(_dev(x, "x"), _dtype_code(x), m, k,
                                                                     _dev(inv_s, "inv_s"),
                                                                     _dev(act_scale, "act_scale"), _dev(xq, "xq"),
                                                                     _stream(stream)))


def sq_fp8_gemm(xq, wq, act_scale, w_scale, y, acc_out=None, stream=None):
    m, k = xq.shape
    n = wq.shape[0]
    _check("sq_fp8_gemm", load().sq_fp8_gemm(_dev(xq, "xq"), _dev(wq, "wq"), m, n, k, _dev(act_scale, "act_scale"),
                                             _dev(w_scale, "w_scale"), _dev(y, "y"), _dtype_code(y),
                                             _opt(acc_out, "acc_out"), _stream(stream)))
