"""Thin Python binding over libsq's C ABI (include/sq.h).

Argument marshalling only: each function takes torch tensors that already
live on the GPU, checks every tensor's element type, shape (or size), device
and contiguity against the sizes it passes (the C ABI trusts them), and passes
raw device pointers, the shapes and the current HIP stream to the entry point
of the same name. Every
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
          5: "SQ_ERR_WORKSPACE", 6: "SQ_ERR_HIP", 7: "SQ_ERR_ALIGN", 8: "SQ_ERR_SCRATCH"}
SQ_PERCENTILE_SCRATCH_BYTES = 32 << 20
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
        "sq_gemm_batched_tiling": [c.c_int, P, P, P, P, P],
        "sq_alpha_search": [P, c.c_int, c.c_int, i64, i64, P, c.c_int, i64, P, c.c_int, P, c.c_size_t, P, P, P],
        "sq_act_scale": [P, P, i64, P, P],
        "sq_dynamic_quant_act": [P, c.c_int, i64, i64, P, P, P, P, P],
        "sq_calib_sample_max_sum": [P, c.c_int, i64, i64, i64, P, P, P],
        "sq_calib_mean_finalize": [P, i64, i64, P, P],
        "sq_calib_percentile_workspace": [c.c_int, i64, P],
        "sq_calib_percentile": [P, c.c_int, i64, i64, c.c_double, P, c.c_size_t, P, P],
        "sq_calib_percentile_noalloc": [P, c.c_int, i64, i64, c.c_double, P, P],
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
        "sq_smooth_factors_f16": [P, P, i64, c.c_float, P, P, P],
        "sq_quant_weight_f16": [P, c.c_int, i64, i64, P, P, P, P],
        "sq_smooth_quant_act_f16": [P, c.c_int, i64, i64, P, P, P, P],
        "sq_w8a8_gemm_f16": [P, P, i64, i64, i64, P, P, P, c.c_int, P, P],
        "sq_smooth_factors_f16_batched": [c.c_int, P, P, P, P, P, P, P],
        "sq_quant_weight_f16_batched": [c.c_int, P, P, P, P, P, P, P, P],
        "sq_smooth_quant_act_f16_batched": [c.c_int, P, P, P, P, P, P, P, P],
        "sq_w8a8_gemm_f16_batched": [c.c_int, P, P, P, P, P, P, P, P, P, P, P],
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


def _dtypes(name: str):
    import torch
    return {"f32": (torch.float32,), "bf16": (torch.bfloat16,), "act": (torch.float32, torch.bfloat16),
            "i8": (torch.int8,), "u8": (torch.uint8,), "i32": (torch.int32,), "f64": (torch.float64,),
            "f16": (torch.float16,)}[name]


def _sdt(name: str) -> str:
    """Scale storage of a batched entry point: binary16 for the _f16 forms
    (torch.float16 tensors hold the bit patterns), fp32 otherwise."""
    return "f16" if "_f16" in name else "f32"


def _arg(t, what: str, dtype: str, shape=None, numel: int | None = None, device=None):
    """Check one tensor argument against what the entry point will read or
    write -- element type, exact shape (or at least `numel` elements), device
    (the first input's), contiguity -- and return its device pointer. Shape and
    type are checked first, so a mismatch raises ValueError before anything is
    launched (the C ABI sizes every buffer from the scalar sizes passed to it)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch.Tensor")
    if t.dtype not in _dtypes(dtype):
        raise ValueError(f"{what}: dtype {t.dtype}, expected {' or '.join(str(d) for d in _dtypes(dtype))}")
    if shape is not None and tuple(t.shape) != tuple(int(v) for v in shape):
        raise ValueError(f"{what}: shape {tuple(t.shape)}, expected {tuple(int(v) for v in shape)}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{what}: {t.numel()} elements, at least {numel} needed")
    if device is not None and t.device != device:
        raise ValueError(f"{what} is on {t.device}, the call's inputs on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _call(name: str, anchor, *args, stream=None):
    """Call entry point `name` once every argument has been checked: the
    anchor input (every other tensor was checked to share its device) must be
    a GPU tensor; the stream is resolved last."""
    if not anchor.is_cuda:
        raise ValueError(f"{name}: inputs must be GPU tensors (got {anchor.device})")
    _check(name, getattr(load(), name)(*args, _stream(stream)))


def _shape2(t, what: str):
    if t.dim() != 2:
        raise ValueError(f"{what} must be 2-D, got shape {tuple(t.shape)}")
    return t.shape[0], t.shape[1]


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def sq_calib_absmax(x, absmax, accumulate: bool = False, stream=None):
    """absmax[j] = max(absmax[j] if accumulate else 0, max_t |x[t, j]|)."""
    rows, k = _shape2(x, "x")
    px = _arg(x, "x", "act")
    pa = _arg(absmax, "absmax", "f32", (k,), device=x.device)
    _call("sq_calib_absmax", x, px, _dtype_code(x), rows, k, pa, int(bool(accumulate)), stream=stream)
    return absmax


def sq_smooth_factors(act_max, w_max, alpha: float, s, inv_s, act_scale, stream=None):
    k = act_max.shape[0]
    d = act_max.device
    _call("sq_smooth_factors", act_max, _arg(act_max, "act_max", "f32", (k,)), _arg(w_max, "w_max", "f32", (k,), device=d), k, float(alpha),
        _arg(s, "s", "f32", (k,), device=d), _arg(inv_s, "inv_s", "f32", (k,), device=d),
        _arg(act_scale, "act_scale", "f32", numel=1, device=d), stream=stream)


def sq_quant_weight(w, s, wq, w_scale, stream=None):
    n, k = _shape2(w, "w")
    pw, d = _arg(w, "w", "act"), w.device
    _call("sq_quant_weight", w, pw, _dtype_code(w), n, k, _arg(s, "s", "f32", (k,), device=d),
                                                     _arg(wq, "wq", "i8", (n, k), device=d),
                                                     _arg(w_scale, "w_scale", "f32", (n,), device=d), stream=stream)


def sq_smooth_quant_act(x, inv_s, act_scale, xq, stream=None):
    m, k = _shape2(x, "x")
    px, d = _arg(x, "x", "act"), x.device
    _call("sq_smooth_quant_act", x, px, _dtype_code(x), m, k, _arg(inv_s, "inv_s", "f32", (k,), device=d),
        _arg(act_scale, "act_scale", "f32", numel=1, device=d), _arg(xq, "xq", "i8", (m, k), device=d), stream=stream)


def _gemm_args(xq, wq, act_scale, w_scale, y, acc_out, code: str, acc_code: str, tag: str = "", sdt: str = "f32"):
    """Pointers and sizes of one product: xq [m,k], wq [n,k] (same code type),
    act_scale [>=1], w_scale [n] (fp32, or float16 for sdt "f16"), y [m,n]
    fp32/bf16, acc_out [m,n] or None (`tag` names the item of a batched call in
    error messages)."""
    m, k = _shape2(xq, f"xq{tag}")
    n, kw = _shape2(wq, f"wq{tag}")
    if kw != k:
        raise ValueError(f"wq{tag}: shape {tuple(wq.shape)} does not share k = {k} with xq{tag}")
    d = xq.device
    return (m, n, k, _arg(xq, f"xq{tag}", code), _arg(wq, f"wq{tag}", code, device=d),
            _arg(act_scale, f"act_scale{tag}", sdt, numel=1, device=d),
            _arg(w_scale, f"w_scale{tag}", sdt, (n,), device=d), _arg(y, f"y{tag}", "act", (m, n), device=d),
            _arg(acc_out, f"acc_out{tag}", acc_code, (m, n), device=d) if acc_out is not None else ctypes.c_void_p(0))


def sq_w8a8_gemm(xq, wq, act_scale, w_scale, y, acc_out=None, stream=None):
    m, n, k, px, pw, pa, ps, py, pacc = _gemm_args(xq, wq, act_scale, w_scale, y, acc_out, "i8", "i32")
    _call("sq_w8a8_gemm", xq, px, pw, m, n, k, pa, ps, py, _dtype_code(y), pacc, stream=stream)


# ---- fp16 scale storage: every scale a torch.float16 tensor (binary16) ----------

def sq_smooth_factors_f16(act_max, w_max, alpha: float, s, act_scale, stream=None):
    """s = f16(fp32 s_j); act_scale = f16(closed form from the stored s)."""
    k = act_max.shape[0]
    d = act_max.device
    _call("sq_smooth_factors_f16", act_max, _arg(act_max, "act_max", "f32", (k,)),
          _arg(w_max, "w_max", "f32", (k,), device=d), k, float(alpha), _arg(s, "s", "f16", (k,), device=d),
          _arg(act_scale, "act_scale", "f16", numel=1, device=d), stream=stream)


def sq_quant_weight_f16(w, s, wq, w_scale, stream=None):
    n, k = _shape2(w, "w")
    pw, d = _arg(w, "w", "act"), w.device
    _call("sq_quant_weight_f16", w, pw, _dtype_code(w), n, k, _arg(s, "s", "f16", (k,), device=d),
          _arg(wq, "wq", "i8", (n, k), device=d), _arg(w_scale, "w_scale", "f16", (n,), device=d), stream=stream)


def sq_smooth_quant_act_f16(x, s, act_scale, xq, stream=None):
    m, k = _shape2(x, "x")
    px, d = _arg(x, "x", "act"), x.device
    _call("sq_smooth_quant_act_f16", x, px, _dtype_code(x), m, k, _arg(s, "s", "f16", (k,), device=d),
          _arg(act_scale, "act_scale", "f16", numel=1, device=d), _arg(xq, "xq", "i8", (m, k), device=d),
          stream=stream)


def sq_w8a8_gemm_f16(xq, wq, act_scale, w_scale, y, acc_out=None, stream=None):
    m, n, k, px, pw, pa, ps, py, pacc = _gemm_args(xq, wq, act_scale, w_scale, y, acc_out, "i8", "i32", sdt="f16")
    _call("sq_w8a8_gemm_f16", xq, px, pw, m, n, k, pa, ps, py, _dtype_code(y), pacc, stream=stream)


SQ_MAX_NORM_CONSUMERS = 4


def sq_rmsnorm_quant_act_multi(h, gammas_folded, eps: float, act_scales, xqs, r_out=None, stream=None):
    """sq_rmsnorm_quant_act for several consumers of one norm output (h read
    once when their folded weights fit in registers)."""
    m, k = _shape2(h, "h")
    ph, d = _arg(h, "h", "act"), h.device
    n = len(gammas_folded)
    if not (len(act_scales) == n and len(xqs) == n):
        raise ValueError("per-consumer lists differ in length")
    g = _ptrs(gammas_folded, "gammas_folded", "f32", lambda i: (k,), d)
    a = _ptrs(act_scales, "act_scales", "f32", None, d, numel=1)
    q = _ptrs(xqs, "xqs", "i8", lambda i: (m, k), d)
    pr = _arg(r_out, "r_out", "f32", (m,), device=d) if r_out is not None else ctypes.c_void_p(0)
    _call("sq_rmsnorm_quant_act_multi", h, ph, _dtype_code(h), m, k, float(eps), n, g[1], a[1], q[1], pr, stream=stream)


def sq_act_scale_batched(act_maxes, inv_ss, act_scales, stream=None):
    """sq_act_scale for several projections in one launch."""
    count = _items(len(act_maxes), "act_maxes")
    if not all(len(v) == count for v in (inv_ss, act_scales)):
        raise ValueError("per-item lists differ in length")
    ks = [t.shape[0] for t in act_maxes]
    d = act_maxes[0].device if count else None
    keep = [_ptrs(act_maxes, "act_maxes", "f32", lambda i: (ks[i],), d),
            _ptrs(inv_ss, "inv_ss", "f32", lambda i: (ks[i],), d),
            _host_array(ctypes.c_int64, ks), _ptrs(act_scales, "act_scales", "f32", None, d, numel=1)]
    _call("sq_act_scale_batched", act_maxes[0], count, *[a for _, a in keep], stream=stream)


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


def sq_gemm_batched_tiling(shapes) -> list[tuple[int, int]]:
    """Block tile (rows, columns) of each product of an sq_w8a8_gemm_batched
    call with these (m, n, k) shapes (one output type and scale storage)."""
    count = len(shapes)
    ms, ns, ks = (_host_array(ctypes.c_int64, [int(s[i]) for s in shapes]) for i in range(3))
    bm, bn = (ctypes.c_int * max(count, 1))(), (ctypes.c_int * max(count, 1))()
    _check("sq_gemm_batched_tiling", load().sq_gemm_batched_tiling(count, ms[1], ns[1], ks[1], bm, bn))
    return [(bm[i], bn[i]) for i in range(count)]


def sq_alpha_search_workspace(n_batches: int, rows_per_batch: int, n: int, k: int, n_alphas: int = 4) -> int:
    out = ctypes.c_size_t(0)
    _check("sq_alpha_search_workspace",
           load().sq_alpha_search_workspace(n_batches, rows_per_batch, n, k, n_alphas, ctypes.byref(out)))
    return out.value


def sq_alpha_search(x_batches, w, workspace, alphas=ALPHA_GRID, stream=None):
    """Returns (mse list, best index). Synchronises the stream."""
    nb = len(x_batches)
    rows, k = _shape2(x_batches[0], "x_batches[0]")
    n, kw = _shape2(w, "w")
    if kw != k:
        raise ValueError(f"w: shape {tuple(w.shape)} does not share k = {k} with the batches")
    xt = _dtype_code(x_batches[0])
    d = x_batches[0].device
    for x in x_batches:
        if tuple(x.shape) != (rows, k) or _dtype_code(x) != xt:
            raise ValueError("all batches must share shape and dtype")
    _arg(w, "w", "act", device=d)
    need = sq_alpha_search_workspace(nb, rows, n, k, len(alphas))
    if workspace.device != d:
        raise ValueError(f"workspace is on {workspace.device}, the call's inputs on {d}")
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace: {workspace.numel() * workspace.element_size()} bytes, {need} needed")
    ptrs = (ctypes.c_void_p * nb)(*[_arg(x, f"x_batches[{i}]", "act", device=d).value for i, x in enumerate(x_batches)])
    al = (ctypes.c_float * len(alphas))(*[float(a) for a in alphas])
    mse = (ctypes.c_double * len(alphas))()
    best = ctypes.c_int(-1)
    if not x_batches[0].is_cuda:
        raise ValueError(f"sq_alpha_search: inputs must be GPU tensors (got {x_batches[0].device})")
    _check("sq_alpha_search", load().sq_alpha_search(ctypes.cast(ptrs, ctypes.c_void_p), xt, nb, rows, k, _dev(w, "w"),
                                                     _dtype_code(w), n, ctypes.cast(al, ctypes.c_void_p), len(alphas),
                                                     _dev(workspace, "workspace"), workspace.numel() *
                                                     workspace.element_size(), ctypes.cast(mse, ctypes.c_void_p),
                                                     ctypes.byref(best), _stream(stream)))
    return list(mse), best.value


def _items(n: int, what: str) -> int:
    if n < 1:
        raise ValueError(f"{what}: at least one item is needed")
    return n


def _host_array(ctype, values):
    """A host array for a per-item argument of the batched entry points."""
    arr = (ctype * len(values))(*values)
    return arr, ctypes.cast(arr, ctypes.c_void_p)


def _ptrs(tensors, what: str, dtype: str | None = None, shape_of=None, device=None, numel: int | None = None):
    """Host array of the tensors' device pointers, each checked with _arg
    (shape_of(i) gives item i's expected shape, or None)."""
    if dtype is None:
        return _host_array(ctypes.c_void_p, [_dev(t, f"{what}[{i}]").value for i, t in enumerate(tensors)])
    return _host_array(ctypes.c_void_p, [
        _arg(t, f"{what}[{i}]", dtype, shape_of(i) if shape_of else None, numel, device).value
        for i, t in enumerate(tensors)])


def sq_calib_absmax_batched(xs, absmaxes, accumulate: bool = False, stream=None):
    """sq_calib_absmax over several inputs in one zero fill + one reduction launch."""
    if len(xs) != len(absmaxes):
        raise ValueError("xs and absmaxes differ in length")
    _items(len(xs), "xs")
    shp = [_shape2(x, f"xs[{i}]") for i, x in enumerate(xs)]
    d = xs[0].device if xs else None
    keep = [_ptrs(xs, "xs", "act", None, d), _host_array(ctypes.c_int, [_dtype_code(x) for x in xs]),
            _host_array(ctypes.c_int64, [r for r, _ in shp]), _host_array(ctypes.c_int64, [k for _, k in shp]),
            _ptrs(absmaxes, "absmaxes", "f32", lambda i: (shp[i][1],), d)]
    _call("sq_calib_absmax_batched", xs[0], len(xs), *[a for _, a in keep], int(bool(accumulate)), stream=stream)


def sq_smooth_factors_batched(act_maxes, w_maxes, alphas, ss, inv_ss, act_scales, stream=None,
                              _name="sq_smooth_factors_batched"):
    """sq_smooth_factors for several projections in two launches (the _f16
    form stores no inv_s: pass inv_ss=None)."""
    count = _items(len(act_maxes), "act_maxes")
    sdt = _sdt(_name)
    if (inv_ss is None) != (sdt == "f16"):
        raise ValueError("inv_ss is written by the fp32 forms only")
    if not all(len(v) == count for v in (w_maxes, alphas, ss, act_scales) + ((inv_ss,) if inv_ss is not None else ())):
        raise ValueError("per-item lists differ in length")
    ks = [t.shape[0] for t in act_maxes]
    d = act_maxes[0].device if count else None
    kk = lambda i: (ks[i],)  # noqa: E731
    keep = [_ptrs(act_maxes, "act_maxes", "f32", kk, d), _ptrs(w_maxes, "w_maxes", "f32", kk, d),
            _host_array(ctypes.c_int64, ks),
            _host_array(ctypes.c_float, [float(a) for a in alphas]), _ptrs(ss, "ss", sdt, kk, d)]
    if inv_ss is not None:
        keep.append(_ptrs(inv_ss, "inv_ss", "f32", kk, d))
    keep.append(_ptrs(act_scales, "act_scales", sdt, None, d, numel=1))
    _call(_name, act_maxes[0], count, *[a for _, a in keep], stream=stream)


def sq_smooth_factors_f16_batched(act_maxes, w_maxes, alphas, ss, act_scales, stream=None):
    sq_smooth_factors_batched(act_maxes, w_maxes, alphas, ss, None, act_scales, stream,
                              _name="sq_smooth_factors_f16_batched")


def sq_quant_weight_batched(ws, ss, wqs, w_scales, stream=None, _name="sq_quant_weight_batched"):
    """sq_quant_weight for several weights, one launch per row-length class."""
    count = _items(len(ws), "ws")
    if not all(len(v) == count for v in (ss, wqs, w_scales)):
        raise ValueError("per-item lists differ in length")
    shp = [_shape2(w, f"ws[{i}]") for i, w in enumerate(ws)]
    d = ws[0].device if count else None
    code, sdt = "u8" if "fp8" in _name else "i8", _sdt(_name)
    keep = [_ptrs(ws, "ws", "act", None, d), _host_array(ctypes.c_int, [_dtype_code(w) for w in ws]),
            _host_array(ctypes.c_int64, [n for n, _ in shp]), _host_array(ctypes.c_int64, [k for _, k in shp]),
            _ptrs(ss, "ss", sdt, lambda i: (shp[i][1],), d), _ptrs(wqs, "wqs", code, lambda i: shp[i], d),
            _ptrs(w_scales, "w_scales", sdt, lambda i: (shp[i][0],), d)]
    _call(_name, ws[0], count, *[a for _, a in keep], stream=stream)


def sq_quant_weight_f16_batched(ws, ss, wqs, w_scales, stream=None):
    sq_quant_weight_batched(ws, ss, wqs, w_scales, stream, _name="sq_quant_weight_f16_batched")


def sq_smooth_quant_act_batched(xs, inv_ss, act_scales, xqs, stream=None, _name="sq_smooth_quant_act_batched"):
    """sq_smooth_quant_act for several projections in one launch (a shared
    input tensor is read once for all of its consumers)."""
    count = _items(len(xs), "xs")
    if not all(len(v) == count for v in (inv_ss, act_scales, xqs)):
        raise ValueError("per-item lists differ in length")
    shp = [_shape2(x, f"xs[{i}]") for i, x in enumerate(xs)]
    d = xs[0].device if count else None
    code, sdt = "u8" if "fp8" in _name else "i8", _sdt(_name)
    keep = [_ptrs(xs, "xs", "act", None, d), _host_array(ctypes.c_int, [_dtype_code(x) for x in xs]),
            _host_array(ctypes.c_int64, [m for m, _ in shp]), _host_array(ctypes.c_int64, [k for _, k in shp]),
            _ptrs(inv_ss, "inv_ss", sdt, lambda i: (shp[i][1],), d),
            _ptrs(act_scales, "act_scales", sdt, None, d, numel=1), _ptrs(xqs, "xqs", code, lambda i: shp[i], d)]
    _call(_name, xs[0], count, *[a for _, a in keep], stream=stream)


def sq_smooth_quant_act_f16_batched(xs, ss, act_scales, xqs, stream=None):
    """The binary16 form: ss are the stored s (the kernel forms 1 / s)."""
    sq_smooth_quant_act_batched(xs, ss, act_scales, xqs, stream, _name="sq_smooth_quant_act_f16_batched")


def sq_w8a8_gemm_batched(xqs, wqs, act_scales, w_scales, ys, acc_outs=None, stream=None,
                         _name="sq_w8a8_gemm_batched"):
    """sq_w8a8_gemm for several products; those with the same large tile and
    output type share one launch."""
    count = _items(len(xqs), "xqs")
    if not all(len(v) == count for v in (wqs, act_scales, w_scales, ys)):
        raise ValueError("per-item lists differ in length")
    if acc_outs is not None and len(acc_outs) != count:
        raise ValueError("acc_outs differs in length")
    fp8 = "fp8" in _name
    args = [_gemm_args(xqs[i], wqs[i], act_scales[i], w_scales[i], ys[i],
                       acc_outs[i] if acc_outs is not None else None, "u8" if fp8 else "i8", "f32" if fp8 else "i32",
                       f"[{i}]", _sdt(_name))
            for i in range(count)]
    d = xqs[0].device if count else None
    for i in range(1, count):
        if xqs[i].device != d:
            raise ValueError(f"xqs[{i}] is on {xqs[i].device}, the call's inputs on {d}")
    keep = [_host_array(ctypes.c_void_p, [a[3].value for a in args]), _host_array(ctypes.c_void_p, [a[4].value for a in args]),
            _host_array(ctypes.c_int64, [a[0] for a in args]), _host_array(ctypes.c_int64, [a[1] for a in args]),
            _host_array(ctypes.c_int64, [a[2] for a in args]), _host_array(ctypes.c_void_p, [a[5].value for a in args]),
            _host_array(ctypes.c_void_p, [a[6].value for a in args]), _host_array(ctypes.c_void_p, [a[7].value for a in args]),
            _host_array(ctypes.c_int, [_dtype_code(y) for y in ys])]
    acc = None
    if acc_outs is not None:
        acc = _host_array(ctypes.c_void_p, [a[8].value for a in args])
    _call(_name, xqs[0], count, *[a for _, a in keep], acc[1] if acc else ctypes.c_void_p(0), stream=stream)


def sq_w8a8_gemm_f16_batched(xqs, wqs, act_scales, w_scales, ys, acc_outs=None, stream=None):
    sq_w8a8_gemm_batched(xqs, wqs, act_scales, w_scales, ys, acc_outs, stream, _name="sq_w8a8_gemm_f16_batched")


def _opt(t, what: str):
    return _dev(t, what) if t is not None else ctypes.c_void_p(0)


def sq_act_scale(act_max, inv_s, act_scale, stream=None):
    k, d = act_max.shape[0], act_max.device
    _call("sq_act_scale", act_max, _arg(act_max, "act_max", "f32", (k,)),
                                               _arg(inv_s, "inv_s", "f32", (k,), device=d), k,
                                               _arg(act_scale, "act_scale", "f32", numel=1, device=d), stream=stream)


def sq_dynamic_quant_act(x, inv_s, live_max, act_scale, xq, stream=None):
    m, k = _shape2(x, "x")
    px, d = _arg(x, "x", "act"), x.device
    _call("sq_dynamic_quant_act", x, px, _dtype_code(x), m, k, _arg(inv_s, "inv_s", "f32", (k,), device=d),
        _arg(live_max, "live_max", "f32", (k,), device=d), _arg(act_scale, "act_scale", "f32", numel=1, device=d),
        _arg(xq, "xq", "i8", (m, k), device=d), stream=stream)


def sq_calib_sample_max_sum(x, samples: int, sample_max, total, stream=None):
    rows, k = _shape2(x, "x")
    if samples < 1 or rows % samples:
        raise ValueError("rows must be a whole number of samples")
    px, d = _arg(x, "x", "act"), x.device
    _call("sq_calib_sample_max_sum", x, px, _dtype_code(x), samples, rows // samples, k,
        _arg(sample_max, "sample_max", "f32", (samples, k), device=d), _arg(total, "sum", "f64", (k,), device=d), stream=stream)


def sq_calib_mean_finalize(total, count: int, act_max, stream=None):
    k, d = total.shape[0], total.device
    _call("sq_calib_mean_finalize", total, _arg(total, "sum", "f64", (k,)), count, k,
                                                                   _arg(act_max, "act_max", "f32", (k,), device=d), stream=stream)


def sq_rmsnorm(h, gamma, eps: float, y, r_out=None, stream=None):
    m, k = _shape2(h, "h")
    ph, d = _arg(h, "h", "act"), h.device
    pr = _arg(r_out, "r_out", "f32", (m,), device=d) if r_out is not None else ctypes.c_void_p(0)
    _call("sq_rmsnorm", h, ph, _dtype_code(h), m, k, _arg(gamma, "gamma", "f32", (k,), device=d),
                                           float(eps), _arg(y, "y", "act", (m, k), device=d), _dtype_code(y), pr, stream=stream)


def sq_fold_norm_weight(gamma, inv_s, gamma_folded, stream=None):
    k, d = gamma.shape[0], gamma.device
    _call("sq_fold_norm_weight", gamma, _arg(gamma, "gamma", "f32", (k,)), _arg(inv_s, "inv_s", "f32", (k,), device=d), k,
        _arg(gamma_folded, "gamma_folded", "f32", (k,), device=d), stream=stream)


def sq_rmsnorm_quant_act(h, gamma_folded, eps: float, act_scale, xq, r_out=None, stream=None):
    m, k = _shape2(h, "h")
    ph, d = _arg(h, "h", "act"), h.device
    pr = _arg(r_out, "r_out", "f32", (m,), device=d) if r_out is not None else ctypes.c_void_p(0)
    _call("sq_rmsnorm_quant_act", h, ph, _dtype_code(h), m, k, _arg(gamma_folded, "gamma_folded", "f32", (k,), device=d), float(eps),
        _arg(act_scale, "act_scale", "f32", numel=1, device=d), _arg(xq, "xq", "i8", (m, k), device=d), pr, stream=stream)


def sq_calib_percentile_workspace(k: int, dtype_code: int = SQ_BF16) -> int:
    out = ctypes.c_size_t(0)
    _check("sq_calib_percentile_workspace", load().sq_calib_percentile_workspace(dtype_code, k, ctypes.byref(out)))
    return out.value


def sq_calib_percentile(x, q: float, workspace, act_max, stream=None):
    """act_max[j] = nearest-rank q-quantile of |x[:, j]|."""
    rows, k = _shape2(x, "x")
    px, d = _arg(x, "x", "act"), x.device
    pa = _arg(act_max, "act_max", "f32", (k,), device=d)
    if workspace.device != d:
        raise ValueError(f"workspace is on {workspace.device}, the call's inputs on {d}")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    _call("sq_calib_percentile", x, px, _dtype_code(x), rows, k, float(q), ctypes.c_void_p(workspace.data_ptr()),
          workspace.numel() * workspace.element_size(), pa, stream=stream)


def sq_calib_percentile_noalloc(x, q: float, act_max, stream=None):
    """sq_calib_percentile with the library's static scratch (no workspace,
    no allocation); calls that overlap on one GPU race."""
    rows, k = _shape2(x, "x")
    px, d = _arg(x, "x", "act"), x.device
    _call("sq_calib_percentile_noalloc", x, px, _dtype_code(x), rows, k, float(q),
          _arg(act_max, "act_max", "f32", (k,), device=d), stream=stream)


# ---- FP8 (OCP E4M3) variant: codes are torch.uint8 tensors --------------------------

def sq_act_scale_fp8(act_max, inv_s, act_scale, stream=None):
    k, d = act_max.shape[0], act_max.device
    _call("sq_act_scale_fp8", act_max, _arg(act_max, "act_max", "f32", (k,)),
                                                       _arg(inv_s, "inv_s", "f32", (k,), device=d), k,
                                                       _arg(act_scale, "act_scale", "f32", numel=1, device=d), stream=stream)


def sq_quant_weight_fp8(w, s, wq, w_scale, stream=None):
    n, k = _shape2(w, "w")
    pw, d = _arg(w, "w", "act"), w.device
    _call("sq_quant_weight_fp8", w, pw, _dtype_code(w), n, k, _arg(s, "s", "f32", (k,), device=d), _arg(wq, "wq", "u8", (n, k), device=d),
        _arg(w_scale, "w_scale", "f32", (n,), device=d), stream=stream)


def sq_smooth_quant_act_fp8(x, inv_s, act_scale, xq, stream=None):
    m, k = _shape2(x, "x")
    px, d = _arg(x, "x", "act"), x.device
    _call("sq_smooth_quant_act_fp8", x, px, _dtype_code(x), m, k, _arg(inv_s, "inv_s", "f32", (k,), device=d),
        _arg(act_scale, "act_scale", "f32", numel=1, device=d), _arg(xq, "xq", "u8", (m, k), device=d), stream=stream)


def sq_fp8_gemm(xq, wq, act_scale, w_scale, y, acc_out=None, stream=None):
    m, n, k, px, pw, pa, ps, py, pacc = _gemm_args(xq, wq, act_scale, w_scale, y, acc_out, "u8", "f32")
    _call("sq_fp8_gemm", xq, px, pw, m, n, k, pa, ps, py, _dtype_code(y), pacc, stream=stream)
