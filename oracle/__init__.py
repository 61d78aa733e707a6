"""Reference oracle for the row normalizations: a plain fp64 CPU implementation.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The product library
(the HIP path) never imports, links or calls anything here, and this package
imports nothing from the product.

``oracle.c`` holds the arithmetic (RMSNorm, LayerNorm and the dual q/k head
RMSNorm, all in IEEE double).  This module compiles it with gcc and exposes
it through ctypes.  ``exact_tiny`` holds an exact-rational second definition
for tiny rows that pins the fp64 code.

Inputs are numpy arrays: ``float32`` for fp32 data, ``uint16`` holding
bfloat16 bit patterns for bf16 data, ``float16`` for fp16 data (decoded by the
oracle's own binary16 code).  Outputs are ``float64``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32 = 0
BF16 = 1
F16 = 2


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile ``oracle.c`` with gcc into a shared library (plain -O2, no
    fast-math, so every double operation is IEEE-exact as written)."""
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-shared",
           "-fPIC", "-std=c99", "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def _needs_build(lib: str, src: str) -> bool:
    return (not os.path.exists(lib)) or os.path.getmtime(lib) < os.path.getmtime(src)


_P = ctypes.c_void_p
_I64 = ctypes.c_int64


class Oracle:
    """ctypes handle on a compiled oracle library."""

    def __init__(self, path: str | None = None):
        if path is None:
            path = _LIB
            if _needs_build(path, _SRC):
                build()
        self.path = path
        lib = ctypes.CDLL(path)
        lib.oracle_rms.argtypes = [_P, _P, ctypes.c_int, _I64, _I64, ctypes.c_float, _P]
        lib.oracle_rms.restype = None
        lib.oracle_layer.argtypes = [_P, _P, _P, ctypes.c_int, _I64, _I64, ctypes.c_float, _P]
        lib.oracle_layer.restype = None
        lib.oracle_dual_head_rms.argtypes = [_P, _P, _P, _P, ctypes.c_int, _I64, _I64, _I64,
                                             ctypes.c_float, _P, _P]
        lib.oracle_dual_head_rms.restype = None
        lib.oracle_rope_rows.argtypes = [_P, _I64, _I64, _I64, _I64, ctypes.c_int,
                                         ctypes.c_float, ctypes.c_float, _I64, _P]
        lib.oracle_rope_rows.restype = None
        lib.oracle_dual_head_rms_rope.argtypes = [_P, _P, _P, _P, ctypes.c_int, _I64, _I64, _I64,
                                                  _I64, ctypes.c_float, _I64, ctypes.c_int,
                                                  ctypes.c_float, ctypes.c_float, _I64, _P, _P,
                                                  _P]
        lib.oracle_dual_head_rms_rope.restype = None
        lib.oracle_rms_swiglu.argtypes = [_P, _P, _P, ctypes.c_int, _I64, _I64, ctypes.c_float,
                                          _P]
        lib.oracle_rms_swiglu.restype = None
        self._lib = lib

    @staticmethod
    def _dtype_code(a: np.ndarray) -> int:
        if a.dtype == np.float32:
            return F32
        if a.dtype == np.uint16:
            return BF16
        if a.dtype == np.float16:
            return F16
        raise TypeError(f"oracle takes float32, uint16 (bf16 bits) or float16, got {a.dtype}")

    @staticmethod
    def _ptr(a):
        return None if a is None else a.ctypes.data_as(ctypes.c_void_p)

    def rms(self, x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
        """RMSNorm over the last axis; returns float64 of x's shape."""
        x = np.ascontiguousarray(x)
        w = np.ascontiguousarray(w)
        code = self._dtype_code(x)
        if w.dtype != x.dtype:
            raise TypeError("x and w must share a dtype")
        width = x.shape[-1]
        rows = x.size // width if width else 0
        if w.shape != (width,):
            raise ValueError("w must have shape (width,)")
        y = np.empty(x.shape, dtype=np.float64)
        self._lib.oracle_rms(self._ptr(x), self._ptr(w), code, rows, width,
                             ctypes.c_float(eps), self._ptr(y))
        return y

    def rms_swiglu(self, x: np.ndarray, g: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
        """RMSNorm over the last axis times SiLU(g), g of x's shape; float64."""
        x = np.ascontiguousarray(x)
        g = np.ascontiguousarray(g)
        w = np.ascontiguousarray(w)
        code = self._dtype_code(x)
        if w.dtype != x.dtype or g.dtype != x.dtype:
            raise TypeError("x, g and w must share a dtype")
        width = x.shape[-1]
        rows = x.size // width if width else 0
        if w.shape != (width,) or g.shape != x.shape:
            raise ValueError("w must have shape (width,) and g the shape of x")
        y = np.empty(x.shape, dtype=np.float64)
        self._lib.oracle_rms_swiglu(self._ptr(x), self._ptr(g), self._ptr(w), code, rows, width,
                                    ctypes.c_float(eps), self._ptr(y))
        return y

    def layer(self, x: np.ndarray, w: np.ndarray, b: np.ndarray | None, eps: float) -> np.ndarray:
        """LayerNorm over the last axis (bias optional); returns float64."""
        x = np.ascontiguousarray(x)
        w = np.ascontiguousarray(w)
        code = self._dtype_code(x)
        width = x.shape[-1]
        rows = x.size // width if width else 0
        if w.dtype != x.dtype or (b is not None and b.dtype != x.dtype):
            raise TypeError("x, w and b must share a dtype")
        if w.shape != (width,) or (b is not None and b.shape != (width,)):
            raise ValueError("w and b must have shape (width,)")
        if b is not None:
            b = np.ascontiguousarray(b)
        y = np.empty(x.shape, dtype=np.float64)
        self._lib.oracle_layer(self._ptr(x), self._ptr(w), self._ptr(b), code, rows, width,
                               ctypes.c_float(eps), self._ptr(y))
        return y

    def dual_head_rms(self, q: np.ndarray, k: np.ndarray, qw: np.ndarray, kw: np.ndarray,
                      eps: float) -> tuple[np.ndarray, np.ndarray]:
        """Dual q/k head RMSNorm; returns (queries, keys) as float64."""
        q = np.ascontiguousarray(q)
        k = np.ascontiguousarray(k)
        qw = np.ascontiguousarray(qw)
        kw = np.ascontiguousarray(kw)
        code = self._dtype_code(q)
        if not (k.dtype == qw.dtype == kw.dtype == q.dtype):
            raise TypeError("q, k, qw and kw must share a dtype")
        hd = q.shape[-1]
        if k.shape[-1] != hd or qw.shape != (hd,) or kw.shape != (hd,):
            raise ValueError("q, k, qw, kw must share the head dimension")
        qy = np.empty(q.shape, dtype=np.float64)
        ky = np.empty(k.shape, dtype=np.float64)
        self._lib.oracle_dual_head_rms(self._ptr(q), self._ptr(k), self._ptr(qw), self._ptr(kw),
                                       code, q.size // hd, k.size // hd, hd,
                                       ctypes.c_float(eps), self._ptr(qy), self._ptr(ky))
        return qy, ky


    def rope_rows(self, v: np.ndarray, heads: int, dims: int, traditional: bool, base: float,
                  scale: float, offset: int, freqs: np.ndarray | None = None) -> np.ndarray:
        """Rotary embedding of fp64 head vectors v [rows, head_dim] (a copy is
        rotated and returned); row r is token r // heads."""
        out = np.array(v, dtype=np.float64, order="C", copy=True)
        hd = out.shape[-1]
        rows = out.size // hd
        if dims % 2 or not 2 <= dims <= hd:
            raise ValueError("dims must be even, 2 <= dims <= head_dim")
        fr = None if freqs is None else np.ascontiguousarray(freqs, dtype=np.float32)
        if fr is not None and fr.shape != (dims // 2,):
            raise ValueError("freqs must have dims/2 entries")
        self._lib.oracle_rope_rows(self._ptr(out), rows, heads, hd, dims, int(traditional),
                                   ctypes.c_float(base), ctypes.c_float(scale), offset,
                                   self._ptr(fr))
        return out

    def dual_head_rms_rope(self, q, k, qw, kw, eps, dims, traditional, base, scale, offset,
                           freqs=None):
        """Dual head RMSNorm then rotary embedding; q [tokens, q_heads, hd],
        k [tokens, k_heads, hd]; returns (queries, keys) in float64."""
        q = np.ascontiguousarray(q)
        k = np.ascontiguousarray(k)
        code = self._dtype_code(q)
        tokens, qh, hd = q.shape
        kh = k.shape[1]
        if k.shape[0] != tokens or k.shape[2] != hd:
            raise ValueError("q and k must share tokens and head_dim")
        fr = None if freqs is None else np.ascontiguousarray(freqs, dtype=np.float32)
        qy = np.empty(q.shape, np.float64)
        ky = np.empty(k.shape, np.float64)
        self._lib.oracle_dual_head_rms_rope(
            self._ptr(q), self._ptr(k), self._ptr(np.ascontiguousarray(qw)),
            self._ptr(np.ascontiguousarray(kw)), code, tokens, qh, kh, hd, ctypes.c_float(eps),
            dims, int(traditional), ctypes.c_float(base), ctypes.c_float(scale), offset,
            self._ptr(fr), self._ptr(qy), self._ptr(ky))
        return qy, ky


_default: Oracle | None = None


def default() -> Oracle:
    """The oracle built from this package's ``oracle.c``."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
