"""ctypes wrapper over the plain C oracle (oracle/sq_oracle.c).

TEST INFRASTRUCTURE ONLY. Only tests/, the smoke check in __graft_entry__ and
the CPU-baseline leg of bench.py may import this module. It shares nothing
with the GPU library. Arrays are numpy; bf16 data is carried as uint16 bit
patterns (dtype ``np.uint16``), fp32 as ``np.float32``.

Each wrapper names the oracle step it runs; the steps and the passages they
follow are listed in oracle/sq_oracle.h.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sq_oracle.c")
LIB = os.path.join(HERE, "libsq_oracle.so")

F32, BF16 = 0, 1
_lock = threading.Lock()
_lib = None

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
          "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(src: str = SRC, out: str = LIB) -> str:
    """Compile the oracle with gcc (plain scalar code, no FMA contraction)."""
    cmd = ["gcc", *CFLAGS, "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True, cwd=os.path.dirname(src))
    return out


def _declare(lib):
    c = ctypes
    P = c.c_void_p
    i64 = c.c_int64
    lib.sqo_num_threads.restype = c.c_int
    lib.sqo_set_num_threads.argtypes = [c.c_int]
    lib.sqo_set_num_threads.restype = None
    lib.sqo_calib_absmax.argtypes = [P, c.c_int, i64, i64, P, c.c_int]
    lib.sqo_act_scale.argtypes = [P, P, i64]
    lib.sqo_act_scale.restype = c.c_float
    lib.sqo_smooth_factors.argtypes = [P, P, i64, c.c_double, P, P, P]
    lib.sqo_quant_weight.argtypes = [P, c.c_int, i64, i64, P, P, P]
    lib.sqo_quant_act.argtypes = [P, c.c_int, i64, i64, P, c.c_float, P]
    lib.sqo_gemm_i32.argtypes = [P, P, i64, i64, i64, P]
    lib.sqo_dequant.argtypes = [P, i64, i64, c.c_float, P, c.c_int, P]
    lib.sqo_ref_gemm.argtypes = [P, c.c_int, P, c.c_int, i64, i64, i64, P]
    lib.sqo_sse.argtypes = [P, P, i64, i64]
    lib.sqo_sse.restype = c.c_double
    lib.sqo_alpha_search.argtypes = [P, c.c_int, c.c_int, i64, i64, P, c.c_int, i64, P, c.c_int, P]
    lib.sqo_alpha_search.restype = c.c_int
    lib.sqo_dynamic_quant_act.argtypes = [P, c.c_int, i64, i64, P, P, P]
    lib.sqo_calib_sample_max_sum.argtypes = [P, c.c_int, i64, i64, i64, P]
    lib.sqo_calib_mean_finalize.argtypes = [P, i64, i64, P]
    lib.sqo_percentile_rank.argtypes = [c.c_double, i64]
    lib.sqo_percentile_rank.restype = i64
    lib.sqo_calib_percentile.argtypes = [P, c.c_int, i64, i64, c.c_double, P]
    lib.sqo_rms_inv.argtypes = [P, c.c_int, i64, i64, c.c_float, P]
    lib.sqo_rmsnorm_apply.argtypes = [P, c.c_int, i64, i64, P, P, c.c_int, P]
    lib.sqo_fold_norm_weight.argtypes = [P, P, i64, P]
    lib.sqo_norm_quant_apply.argtypes = [P, c.c_int, i64, i64, P, P, c.c_float, P]
    lib.sqo_e4m3_encode.argtypes = [c.c_float]
    lib.sqo_e4m3_encode.restype = c.c_uint8
    lib.sqo_e4m3_decode.argtypes = [c.c_uint8]
    lib.sqo_e4m3_decode.restype = c.c_float
    lib.sqo_quant_weight_fp8.argtypes = [P, c.c_int, i64, i64, P, P, P]
    lib.sqo_act_scale_fp8.argtypes = [P, P, i64]
    lib.sqo_act_scale_fp8.restype = c.c_float
    lib.sqo_quant_act_fp8.argtypes = [P, c.c_int, i64, i64, P, c.c_float, P]
    lib.sqo_gemm_fp8.argtypes = [P, P, i64, i64, i64, c.c_float, P, c.c_int, P, P, P]
    lib.sqo_dequant_f32.argtypes = [P, i64, i64, c.c_float, P, c.c_int, P]
    lib.sqo_f16_encode.argtypes = [c.c_float]
    lib.sqo_f16_encode.restype = c.c_uint16
    lib.sqo_f16_decode.argtypes = [c.c_uint16]
    lib.sqo_f16_decode.restype = c.c_float
    lib.sqo_scale_f16.argtypes = [c.c_float]
    lib.sqo_scale_f16.restype = c.c_uint16
    lib.sqo_f16_encode_array.argtypes = [P, i64, P]
    lib.sqo_f16_decode_array.argtypes = [P, i64, P]
    lib.sqo_smooth_factors_h.argtypes = [P, P, i64, c.c_double, P, P]
    lib.sqo_quant_weight_h.argtypes = [P, c.c_int, i64, i64, P, P, P]
    lib.sqo_quant_act_h.argtypes = [P, c.c_int, i64, i64, P, c.c_uint16, P]
    lib.sqo_dequant_h.argtypes = [P, i64, i64, c.c_uint16, P, c.c_int, P]
    return lib


def load(path: str | None = None):
    """Load the oracle library, building it first if it is missing or stale.

    ``path`` loads a different build of the same source (mutation tests)."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if (not os.path.exists(LIB)) or os.path.getmtime(LIB) < max(
                    os.path.getmtime(SRC), os.path.getmtime(os.path.join(HERE, "sq_oracle.h"))):
                build()
            _lib = _declare(ctypes.CDLL(LIB))
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def _ftype(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"unsupported float storage {a.dtype}")


class Oracle:
    """Thin numpy front end; one instance per loaded library."""

    def __init__(self, lib=None):
        self.lib = lib if lib is not None else load()

    def num_threads(self) -> int:
        return int(self.lib.sqo_num_threads())

    def set_num_threads(self, n: int) -> None:
        """Threads for later calls from this thread (timing only: results do
        not depend on the count)."""
        self.lib.sqo_set_num_threads(int(n))

    # O1 / O2
    def calib_absmax(self, x: np.ndarray, absmax: np.ndarray | None = None) -> np.ndarray:
        rows, k = x.shape
        acc = absmax is not None
        out = absmax if acc else np.zeros(k, np.float32)
        self.lib.sqo_calib_absmax(_ptr(x), _ftype(x), rows, k, _ptr(out), int(acc))
        return out

    # O6
    def act_scale(self, act_max: np.ndarray, inv_s: np.ndarray) -> np.float32:
        return np.float32(self.lib.sqo_act_scale(_ptr(act_max), _ptr(inv_s), act_max.shape[0]))

    # O3 - O6
    def smooth_factors(self, act_max: np.ndarray, w_max: np.ndarray, alpha: float):
        k = act_max.shape[0]
        s = np.empty(k, np.float32)
        inv_s = np.empty(k, np.float32)
        a = np.empty(1, np.float32)
        self.lib.sqo_smooth_factors(_ptr(act_max), _ptr(w_max), k, float(alpha), _ptr(s), _ptr(inv_s), _ptr(a))
        return s, inv_s, a[0]

    # O7
    def quant_weight(self, w: np.ndarray, s: np.ndarray):
        n, k = w.shape
        wq = np.empty((n, k), np.int8)
        ws = np.empty(n, np.float32)
        self.lib.sqo_quant_weight(_ptr(w), _ftype(w), n, k, _ptr(s), _ptr(wq), _ptr(ws))
        return wq, ws

    # O8
    def quant_act(self, x: np.ndarray, inv_s: np.ndarray, act_scale) -> np.ndarray:
        m, k = x.shape
        xq = np.empty((m, k), np.int8)
        self.lib.sqo_quant_act(_ptr(x), _ftype(x), m, k, _ptr(inv_s), float(np.float32(act_scale)), _ptr(xq))
        return xq

    # O9
    def gemm_i32(self, xq: np.ndarray, wq: np.ndarray) -> np.ndarray:
        m, k = xq.shape
        n = wq.shape[0]
        assert wq.shape[1] == k
        acc = np.empty((m, n), np.int32)
        self.lib.sqo_gemm_i32(_ptr(xq), _ptr(wq), m, n, k, _ptr(acc))
        return acc

    # O10
    def dequant(self, acc: np.ndarray, act_scale, w_scale: np.ndarray, bf16: bool = False) -> np.ndarray:
        m, n = acc.shape
        y = np.empty((m, n), np.uint16 if bf16 else np.float32)
        self.lib.sqo_dequant(_ptr(acc), m, n, float(np.float32(act_scale)), _ptr(w_scale), BF16 if bf16 else F32, _ptr(y))
        return y

    def ref_gemm(self, x: np.ndarray, w: np.ndarray) -> np.ndarray:
        m, k = x.shape
        n = w.shape[0]
        y = np.empty((m, n), np.float32)
        self.lib.sqo_ref_gemm(_ptr(x), _ftype(x), _ptr(w), _ftype(w), m, n, k, _ptr(y))
        return y

    def sse(self, y: np.ndarray, yref: np.ndarray) -> float:
        m, n = y.shape
        return float(self.lib.sqo_sse(_ptr(y), _ptr(yref), m, n))

    # O11
    def alpha_search(self, x_batches, w: np.ndarray, alphas=(0.25, 0.5, 0.75, 1.0)):
        nb = len(x_batches)
        rows, k = x_batches[0].shape
        n = w.shape[0]
        ptrs = (ctypes.c_void_p * nb)(*[x.ctypes.data for x in x_batches])
        al = np.asarray(alphas, np.float64)
        mse = np.empty(len(al), np.float64)
        best = self.lib.sqo_alpha_search(ctypes.cast(ptrs, ctypes.c_void_p), _ftype(x_batches[0]), nb, rows, k,
                                         _ptr(w), _ftype(w), n, _ptr(al), len(al), _ptr(mse))
        return mse, int(best)

    # O13
    def dynamic_quant_act(self, x: np.ndarray, inv_s: np.ndarray):
        m, k = x.shape
        xq = np.empty((m, k), np.int8)
        a = np.empty(1, np.float32)
        self.lib.sqo_dynamic_quant_act(_ptr(x), _ftype(x), m, k, _ptr(inv_s), _ptr(xq), _ptr(a))
        return xq, a[0]

    # O14
    def calib_sample_max_sum(self, x: np.ndarray, samples: int, total: np.ndarray | None = None) -> np.ndarray:
        rows, k = x.shape
        assert rows % samples == 0
        out = total if total is not None else np.zeros(k, np.float64)
        self.lib.sqo_calib_sample_max_sum(_ptr(x), _ftype(x), samples, rows // samples, k, _ptr(out))
        return out

    def calib_mean_finalize(self, total: np.ndarray, count: int) -> np.ndarray:
        k = total.shape[0]
        out = np.empty(k, np.float32)
        self.lib.sqo_calib_mean_finalize(_ptr(total), count, k, _ptr(out))
        return out

    # O15
    def percentile_rank(self, q: float, rows: int) -> int:
        return int(self.lib.sqo_percentile_rank(float(q), rows))

    def calib_percentile(self, x: np.ndarray, q: float) -> np.ndarray:
        rows, k = x.shape
        out = np.empty(k, np.float32)
        self.lib.sqo_calib_percentile(_ptr(x), _ftype(x), rows, k, float(q), _ptr(out))
        return out

    # O16
    def rms_inv(self, h: np.ndarray, eps: float) -> np.ndarray:
        m, k = h.shape
        r = np.empty(m, np.float32)
        self.lib.sqo_rms_inv(_ptr(h), _ftype(h), m, k, float(np.float32(eps)), _ptr(r))
        return r

    def rmsnorm_apply(self, h: np.ndarray, r: np.ndarray, gamma: np.ndarray, bf16: bool = False) -> np.ndarray:
        m, k = h.shape
        y = np.empty((m, k), np.uint16 if bf16 else np.float32)
        self.lib.sqo_rmsnorm_apply(_ptr(h), _ftype(h), m, k, _ptr(r), _ptr(gamma), BF16 if bf16 else F32, _ptr(y))
        return y

    # O17
    def fold_norm_weight(self, gamma: np.ndarray, inv_s: np.ndarray) -> np.ndarray:
        out = np.empty_like(gamma, dtype=np.float32)
        self.lib.sqo_fold_norm_weight(_ptr(gamma), _ptr(inv_s), gamma.shape[0], _ptr(out))
        return out

    # O18
    def norm_quant_apply(self, h: np.ndarray, r: np.ndarray, gamma_folded: np.ndarray, act_scale) -> np.ndarray:
        m, k = h.shape
        xq = np.empty((m, k), np.int8)
        self.lib.sqo_norm_quant_apply(_ptr(h), _ftype(h), m, k, _ptr(r), _ptr(gamma_folded),
                                      float(np.float32(act_scale)), _ptr(xq))
        return xq

    # O16 + O18: the fused norm + quantizer for one batch
    def rmsnorm_quant_act(self, h: np.ndarray, gamma_folded: np.ndarray, eps: float, act_scale):
        r = self.rms_inv(h, eps)
        return self.norm_quant_apply(h, r, gamma_folded, act_scale), r

    # O19
    def e4m3_encode(self, v) -> np.ndarray:
        v = np.asarray(v, np.float32)
        return np.array([self.lib.sqo_e4m3_encode(float(x)) for x in v.ravel()], np.uint8).reshape(v.shape)

    def e4m3_decode(self, b) -> np.ndarray:
        b = np.asarray(b, np.uint8)
        return np.array([self.lib.sqo_e4m3_decode(int(x)) for x in b.ravel()], np.float32).reshape(b.shape)

    # O20
    def quant_weight_fp8(self, w: np.ndarray, s: np.ndarray):
        n, k = w.shape
        wq = np.empty((n, k), np.uint8)
        ws = np.empty(n, np.float32)
        self.lib.sqo_quant_weight_fp8(_ptr(w), _ftype(w), n, k, _ptr(s), _ptr(wq), _ptr(ws))
        return wq, ws

    # O21
    def act_scale_fp8(self, act_max: np.ndarray, inv_s: np.ndarray) -> np.float32:
        return np.float32(self.lib.sqo_act_scale_fp8(_ptr(act_max), _ptr(inv_s), act_max.shape[0]))

    # O22
    def quant_act_fp8(self, x: np.ndarray, inv_s: np.ndarray, act_scale) -> np.ndarray:
        m, k = x.shape
        xq = np.empty((m, k), np.uint8)
        self.lib.sqo_quant_act_fp8(_ptr(x), _ftype(x), m, k, _ptr(inv_s), float(np.float32(act_scale)), _ptr(xq))
        return xq

    # O23
    def gemm_fp8(self, xq: np.ndarray, wq: np.ndarray, act_scale, w_scale: np.ndarray, bf16: bool = False):
        m, k = xq.shape
        n = wq.shape[0]
        y = np.empty((m, n), np.uint16 if bf16 else np.float32)
        acc = np.empty((m, n), np.float64)
        absacc = np.empty((m, n), np.float64)
        self.lib.sqo_gemm_fp8(_ptr(xq), _ptr(wq), m, n, k, float(np.float32(act_scale)), _ptr(w_scale),
                              BF16 if bf16 else F32, _ptr(y), _ptr(acc), _ptr(absacc))
        return y, acc, absacc

    # O24
    def dequant_f32(self, acc: np.ndarray, act_scale, w_scale: np.ndarray, bf16: bool = False) -> np.ndarray:
        m, n = acc.shape
        y = np.empty((m, n), np.uint16 if bf16 else np.float32)
        self.lib.sqo_dequant_f32(_ptr(acc), m, n, float(np.float32(act_scale)), _ptr(w_scale),
                                 BF16 if bf16 else F32, _ptr(y))
        return y

    # O25: binary16 values as uint16 bit patterns
    def f16_encode(self, v) -> np.ndarray:
        v = np.ascontiguousarray(np.asarray(v, np.float32))
        out = np.empty(v.shape, np.uint16)
        self.lib.sqo_f16_encode_array(_ptr(v), v.size, _ptr(out))
        return out

    def f16_decode(self, h) -> np.ndarray:
        h = np.ascontiguousarray(np.asarray(h, np.uint16))
        out = np.empty(h.shape, np.float32)
        self.lib.sqo_f16_decode_array(_ptr(h), h.size, _ptr(out))
        return out

    def scale_f16(self, v: float) -> np.uint16:
        return np.uint16(self.lib.sqo_scale_f16(float(np.float32(v))))

    # O26
    def smooth_factors_h(self, act_max: np.ndarray, w_max: np.ndarray, alpha: float):
        k = act_max.shape[0]
        s16 = np.empty(k, np.uint16)
        a16 = np.zeros(1, np.uint16)
        self.lib.sqo_smooth_factors_h(_ptr(act_max), _ptr(w_max), k, float(alpha), _ptr(s16), _ptr(a16))
        return s16, np.uint16(a16[0])

    # O27
    def quant_weight_h(self, w: np.ndarray, s16: np.ndarray):
        n, k = w.shape
        wq = np.empty((n, k), np.int8)
        ws16 = np.empty(n, np.uint16)
        self.lib.sqo_quant_weight_h(_ptr(w), _ftype(w), n, k, _ptr(s16), _ptr(wq), _ptr(ws16))
        return wq, ws16

    # O28
    def quant_act_h(self, x: np.ndarray, s16: np.ndarray, act_scale16) -> np.ndarray:
        m, k = x.shape
        xq = np.empty((m, k), np.int8)
        self.lib.sqo_quant_act_h(_ptr(x), _ftype(x), m, k, _ptr(s16), int(act_scale16), _ptr(xq))
        return xq

    # O29
    def dequant_h(self, acc: np.ndarray, act_scale16, w_scale16: np.ndarray, bf16: bool = False) -> np.ndarray:
        m, n = acc.shape
        y = np.empty((m, n), np.uint16 if bf16 else np.float32)
        self.lib.sqo_dequant_h(_ptr(np.ascontiguousarray(acc, np.int32)), m, n, int(act_scale16), _ptr(w_scale16),
                               BF16 if bf16 else F32, _ptr(y))
        return y

    # the layer with fp16 scale storage (O26-O29) for one runtime input (helper for tests)
    def layer_forward_h(self, x_calib_batches, w: np.ndarray, x: np.ndarray, alpha: float, bf16_out: bool = False):
        k = w.shape[1]
        act_max = np.zeros(k, np.float32)
        for xc in x_calib_batches:
            self.calib_absmax(xc, act_max)
        w_max = self.calib_absmax(w)
        s16, a16 = self.smooth_factors_h(act_max, w_max, alpha)
        wq, ws16 = self.quant_weight_h(w, s16)
        xq = self.quant_act_h(x, s16, a16)
        acc = self.gemm_i32(xq, wq)
        y = self.dequant_h(acc, a16, ws16, bf16=bf16_out)
        return dict(act_max=act_max, w_max=w_max, s16=s16, act_scale16=a16, wq=wq, w_scale16=ws16, xq=xq,
                    acc=acc, y=y)

    # the whole layer, O1..O10, for one runtime input (helper for tests)
    def layer_forward(self, x_calib_batches, w: np.ndarray, x: np.ndarray, alpha: float, bf16_out: bool = False):
        k = w.shape[1]
        act_max = np.zeros(k, np.float32)
        for xc in x_calib_batches:
            self.calib_absmax(xc, act_max)
        w_max = self.calib_absmax(w)
        s, inv_s, a = self.smooth_factors(act_max, w_max, alpha)
        wq, ws = self.quant_weight(w, s)
        xq = self.quant_act(x, inv_s, a)
        acc = self.gemm_i32(xq, wq)
        y = self.dequant(acc, a, ws, bf16=bf16_out)
        return dict(act_max=act_max, w_max=w_max, s=s, inv_s=inv_s, act_scale=a,
                    wq=wq, w_scale=ws, xq=xq, acc=acc, y=y)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (h.astype(np.uint32) << 16).view(np.float32)
