"""The f16wm oracle: TEST INFRASTRUCTURE ONLY.

A plain scalar CPU implementation (``f16wm_oracle.c``) of the F16-weight
products as the bankML page "bankML/f16.rs -- F16 weights, multiplied as the
shipped ggml b11192 multiplies them" defines them: the f16 rounding of the
activation, the ``vec_dot`` and tinyBLAS reduction orders, the ``takes_sgemm``
choice of path, and the products built from them.  This module only marshals
numpy arrays into it.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import it.  It shares no code with ``f16_weight_matrix_amd``
and never imports it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "f16wm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# -ffp-contract=off: no multiply-add the source does not write; no fast-math.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra", "-pthread"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class Oracle:
    """The oracle's functions bound to one build of f16wm_oracle.c."""

    def __init__(self, path: str = _LIB):
        if path == _LIB and not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        L.oracle_to_f16_one.argtypes = [ctypes.c_float]
        L.oracle_to_f16_one.restype = ctypes.c_uint16
        L.oracle_to_f16.argtypes = [P, P, I64]
        L.oracle_widen.argtypes = [P, P, I64]
        L.oracle_vec_dot.argtypes = [P, P, I64]
        L.oracle_vec_dot.restype = ctypes.c_float
        L.oracle_sgemm_dot.argtypes = [P, P, I64]
        L.oracle_sgemm_dot.restype = ctypes.c_float
        L.oracle_takes_sgemm.argtypes = [I64, I64, I64]
        L.oracle_takes_sgemm.restype = ctypes.c_int
        L.oracle_mat_mul.argtypes = [P, I64, I64, P, I64, P, ctypes.c_int]
        L.oracle_mat_vec.argtypes = [P, I64, I64, P, P, ctypes.c_int]
        L.oracle_mat_mul_at.argtypes = [P, I64, I64, P, I64, P, P, I64, P]
        L.oracle_exact_dot.argtypes = [P, P, I64, P]
        L.oracle_exact_dot.restype = ctypes.c_double
        L.oracle_fp64_at.argtypes = [P, I64, P, P, P, I64, P, P]
        L.oracle_mat_mul_out.argtypes = [P, I64, I64, P, I64, ctypes.c_int, P, ctypes.c_int]
        L.oracle_kq.argtypes = [P, I64, I64, I64, P, I64, P]
        L.oracle_mad.argtypes = [P, P, P, I64, I64]
        L.oracle_scale.argtypes = [P, P, I64, I64]
        self.L = L

    def to_f16(self, x) -> np.ndarray:
        """f32 -> f16 bit patterns, round to nearest even (same shape)."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        y = np.empty(x.shape, dtype=np.uint16)
        self.L.oracle_to_f16(_p(x), _p(y), x.size)
        return y

    def widen(self, h) -> np.ndarray:
        """f16 bit patterns -> exact f32 values."""
        h = _u16(h)
        y = np.empty(h.shape, dtype=np.float32)
        self.L.oracle_widen(_p(h), _p(y), h.size)
        return y

    def vec_dot(self, x, y) -> np.float32:
        x, y = _u16(x), _u16(y)
        assert x.shape == y.shape and x.ndim == 1
        return np.float32(self.L.oracle_vec_dot(_p(x), _p(y), x.size))

    def sgemm_dot(self, x, y) -> np.float32:
        x, y = _u16(x), _u16(y)
        assert x.shape == y.shape and x.ndim == 1 and x.size % 8 == 0
        return np.float32(self.L.oracle_sgemm_dot(_p(x), _p(y), x.size))

    def takes_sgemm(self, rows: int, k: int, n: int) -> bool:
        return bool(self.L.oracle_takes_sgemm(rows, k, n))

    def mat_mul(self, w, a, threads: int = 0) -> np.ndarray:
        """W [rows][k] (f16 bits) times A [n][k] (f16 bits) -> out [n][rows] f32,
        out[c, r] = out[c*rows + r], each element by the shape's path."""
        w, a = _u16(w), _u16(a)
        if a.ndim == 1:
            a = a.reshape(1, -1)
        rows, k = w.shape
        n = a.shape[0]
        assert a.shape[1] == k
        out = np.empty((n, rows), dtype=np.float32)
        self.L.oracle_mat_mul(_p(w), rows, k, _p(a), n, _p(out), threads)
        return out

    def mat_vec(self, w, a, threads: int = 0) -> np.ndarray:
        """out[r] = vec_dot(W[r], a)."""
        w, a = _u16(w), _u16(a)
        rows, k = w.shape
        assert a.shape == (k,)
        out = np.empty(rows, dtype=np.float32)
        self.L.oracle_mat_vec(_p(w), rows, k, _p(a), _p(out), threads)
        return out

    def mat_vec_multi(self, ws, a, threads: int = 0) -> list:
        """Several matrices times one f16 column: one mat_vec per matrix."""
        return [self.mat_vec(w, a, threads) for w in ws]

    def mat_mul_at(self, w, a, rr, cc) -> np.ndarray:
        """Elements (rr[i], cc[i]) of W x A, each by the full shape's path."""
        w, a = _u16(w), _u16(a)
        if a.ndim == 1:
            a = a.reshape(1, -1)
        rows, k = w.shape
        n = a.shape[0]
        rr = np.ascontiguousarray(rr, dtype=np.int64)
        cc = np.ascontiguousarray(cc, dtype=np.int64)
        assert rr.shape == cc.shape
        assert (rr >= 0).all() and (rr < rows).all() and (cc >= 0).all() and (cc < n).all()
        out = np.empty(rr.shape, dtype=np.float32)
        self.L.oracle_mat_mul_at(_p(w), rows, k, _p(a), n, _p(rr), _p(cc), rr.size, _p(out))
        return out

    def exact_dot(self, x, y):
        """(exact sum of x[i]*y[i] rounded once to f64, sum |x[i]*y[i]| likewise)."""
        x, y = _u16(x), _u16(y)
        assert x.shape == y.shape and x.ndim == 1
        sa = ctypes.c_double()
        s = self.L.oracle_exact_dot(_p(x), _p(y), x.size, ctypes.byref(sa))
        return s, sa.value

    def fp64_at(self, w, a, rr, cc):
        """binary64 reference and sum-of-|products| scale at elements (rr, cc)."""
        w, a = _u16(w), _u16(a)
        if a.ndim == 1:
            a = a.reshape(1, -1)
        rows, k = w.shape
        rr = np.ascontiguousarray(rr, dtype=np.int64)
        cc = np.ascontiguousarray(cc, dtype=np.int64)
        assert (rr >= 0).all() and (rr < rows).all() and (cc >= 0).all() and (cc < a.shape[0]).all()
        ref = np.empty(rr.shape, dtype=np.float64)
        scale = np.empty(rr.shape, dtype=np.float64)
        self.L.oracle_fp64_at(_p(w), k, _p(a), _p(rr), _p(cc), rr.size, _p(ref), _p(scale))
        return ref, scale

    # the last layer's output columns (forward page, "Why only the output rows
    # leave the last layer")
    OUT_NONE, OUT_LAST, OUT_ALL = 0, 1, 2

    def mat_mul_out(self, w, a, mode: int, threads: int = 0):
        """The product over the output columns only: mode OUT_NONE -> None,
        OUT_LAST -> out [rows] of the last column (vec_dot), OUT_ALL -> out
        [n][rows] (order by takes_sgemm(rows, k, n))."""
        w, a = _u16(w), _u16(a)
        if a.ndim == 1:
            a = a.reshape(1, -1)
        rows, k = w.shape
        n = a.shape[0]
        assert a.shape[1] == k and mode in (0, 1, 2)
        if mode == 0:
            return None
        out = np.empty((rows,) if mode == 1 else (n, rows), dtype=np.float32)
        self.L.oracle_mat_mul_out(_p(w), rows, k, _p(a), n, mode, _p(out), threads)
        return out

    def kq(self, kc, q):
        """Scores of queries q [n_head][d] against an f16 K cache kc
        [n_kv][n_kv_head][d]: out [n_head][n_kv], vec_dot order."""
        kc, q = _u16(kc), _u16(q)
        n_kv, n_kv_head, d = kc.shape
        n_head = q.shape[0]
        assert q.shape == (n_head, d) and n_head % n_kv_head == 0
        out = np.empty((n_head, n_kv), dtype=np.float32)
        self.L.oracle_kq(_p(kc), n_kv, n_kv_head, d, _p(q), n_head, _p(out))
        return out

    def mad(self, acc, v, w):
        """acc [nvec][n] f16 updated in a copy: to_f16(fma(v, w[b], acc))."""
        acc = _u16(acc).copy()
        v = _u16(v)
        if acc.ndim == 1:
            acc, v = acc.reshape(1, -1), v.reshape(1, -1)
        w = np.ascontiguousarray(np.atleast_1d(w), dtype=np.float32)
        assert acc.shape == v.shape and w.shape == (acc.shape[0],)
        self.L.oracle_mad(_p(acc), _p(v), _p(w), acc.shape[0], acc.shape[1])
        return acc

    def scale(self, acc, s):
        """acc [nvec][n] f16 scaled in a copy: to_f16(acc * s[b])."""
        acc = _u16(acc).copy()
        if acc.ndim == 1:
            acc = acc.reshape(1, -1)
        s = np.ascontiguousarray(np.atleast_1d(s), dtype=np.float32)
        assert s.shape == (acc.shape[0],)
        self.L.oracle_scale(_p(acc), _p(s), acc.shape[0], acc.shape[1])
        return acc


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError("expected f16 bit patterns as uint16 or float16, got %s" % a.dtype)
    return np.ascontiguousarray(a)


_default = None


def default() -> Oracle:
    """The oracle built from oracle/f16wm_oracle.c (built on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def __getattr__(name):
    # module-level access (oracle.vec_dot, ...) goes to the default build
    if name in ("to_f16", "widen", "vec_dot", "sgemm_dot", "takes_sgemm", "mat_mul", "mat_vec",
                "mat_vec_multi", "mat_mul_at", "exact_dot", "fp64_at", "mat_mul_out", "kq", "mad", "scale"):
        return getattr(default(), name)
    raise AttributeError(name)
