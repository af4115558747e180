"""Binding of libsq_ceiling.so (include/sq_ceiling.h): the measured-ceiling
probes (an MFMA-only loop, a 16-byte copy, a 2:1 narrowing copy and a 16-byte
read) that bound the path's kernels on their rooflines. They are not steps of
the method and live in a library of their own beside libsq.so. Argument
marshalling only; raises if the library is not built."""
from __future__ import annotations

import ctypes
import os
import re
import threading

from .capi import SQError, STATUS, _dev, _stream

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsq_ceiling.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "sq_ceiling.h")

_lib = None
_lock = threading.Lock()


def declared_functions(header: str = HEADER) -> list[str]:
    """Names of the functions include/sq_ceiling.h declares."""
    text = open(header).read()
    return sorted(set(re.findall(r"^\s*sq_status\s+(sq_\w+)\s*\(", text, re.M)))


def load(path: str = LIB_PATH):
    """Load libsq_ceiling.so (raises if it is not built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
            lib = ctypes.CDLL(path)
            c = ctypes
            P, i64 = c.c_void_p, c.c_int64
            for name, args in {"sq_ceiling_mfma": [i64, c.c_int, P, P, P, P], "sq_ceiling_copy": [P, P, i64, P],
                               "sq_ceiling_read": [P, i64, P, P], "sq_ceiling_narrow": [P, P, i64, P]}.items():
                f = getattr(lib, name)
                f.argtypes = args
                f.restype = c.c_int
            _lib = lib
    return _lib


def _check(name: str, status: int):
    if status != 0:
        raise SQError(name, status, STATUS.get(status, str(status)))


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


