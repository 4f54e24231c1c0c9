"""f16wm: F16-weight matrix products for AMD MI355X (gfx950).

A thin binding over the C ABI in ``include/f16wm.h`` (``libf16wm.so``, built
by ``python -m f16_weight_matrix_amd.build``).  Every step of every product runs
in the library's HIP kernels; this module only checks tensors and passes their
device pointers and the current HIP stream.  PyTorch supplies device memory
and streams, nothing else.  There is no CPU fallback: if the library is not
built, importing the functions raises.

Tensors: f16 data (weights ``[rows, k]``, rounded activations ``[n, k]``) is
``torch.float16`` (or ``int16``/``uint16`` holding the same bit patterns),
contiguous, on a gfx950 device; f32 data is ``torch.float32``.  Outputs of
products are ``[n, rows]`` (``out[c*rows + r]``).
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libf16wm.so")

F16WM_OK = 0
F16WM_EINVAL = -1
F16WM_ENODEV = -2
F16WM_ELAUNCH = -3
F16WM_EUNSUPPORTED = -4
MAX_MULTI = 8


class F16WMError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("%s (code %d)" % (msg, code))
        self.code = code


class _Mat(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("rows", ctypes.c_int64), ("out", ctypes.c_void_p)]


class _Gemv(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("a", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("k", ctypes.c_int64), ("a_f32", ctypes.c_int32)]


MAX_TABLE = 4096


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libf16wm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libf16wm.so is not built (%s); run `python -m f16_weight_matrix_amd.build`"
                               % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        L.f16wm_to_f16.argtypes = [P, P, I64, P]
        L.f16wm_widen.argtypes = [P, P, I64, P]
        L.f16wm_get_rows.argtypes = [P, I64, I64, P, I64, P, P]
        L.f16wm_mat_vec.argtypes = [P, I64, I64, P, P, P]
        L.f16wm_mat_vec_multi.argtypes = [ctypes.POINTER(_Mat), I32, I64, P, P]
        L.f16wm_mat_vec_f32.argtypes = [P, I64, I64, P, P, P]
        L.f16wm_mat_vec_multi_f32.argtypes = [ctypes.POINTER(_Mat), I32, I64, P, P]
        L.f16wm_mat_vec_table.argtypes = [ctypes.POINTER(_Gemv), I32, P]
        L.f16wm_mat_mul.argtypes = [P, I64, I64, P, I64, P, P]
        L.f16wm_mat_mul_mfma.argtypes = [P, I64, I64, P, I64, P, P]
        L.f16wm_mat_mul_multi.argtypes = [ctypes.POINTER(_Mat), I32, I64, P, I64, P]
        L.f16wm_mat_mul_f32.argtypes = [P, I64, I64, P, I64, P, P]
        L.f16wm_mat_mul_multi_f32.argtypes = [ctypes.POINTER(_Mat), I32, I64, P, I64, P]
        L.f16wm_mat_mul_mfma_multi.argtypes = [ctypes.POINTER(_Mat), I32, I64, P, I64, P]
        L.f16wm_takes_sgemm.argtypes = [I64, I64, I64]
        L.f16wm_mat_mul_out.argtypes = [P, I64, I64, P, I64, I32, P, P]
        L.f16wm_kq.argtypes = [P, I64, I64, I64, P, I64, P, P]
        L.f16wm_mad.argtypes = [P, P, P, I64, I64, P]
        L.f16wm_scale.argtypes = [P, P, I64, I64, P]
        for f in ("f16wm_to_f16", "f16wm_widen", "f16wm_get_rows", "f16wm_mat_vec", "f16wm_mat_vec_multi", "f16wm_mat_vec_f32",
                  "f16wm_mat_vec_multi_f32", "f16wm_mat_vec_table", "f16wm_mat_mul", "f16wm_mat_mul_mfma", "f16wm_mat_mul_multi",
                  "f16wm_mat_mul_mfma_multi", "f16wm_mat_mul_f32", "f16wm_mat_mul_multi_f32", "f16wm_takes_sgemm",
                  "f16wm_mat_mul_out", "f16wm_kq", "f16wm_mad", "f16wm_scale"):
            getattr(L, f).restype = ctypes.c_int
        L.f16wm_last_error.restype = ctypes.c_char_p
        L.f16wm_last_error.argtypes = []
        L.f16wm_version.restype = ctypes.c_char_p
        L.f16wm_version.argtypes = []
        _lib = L
    return _lib


def last_error() -> str:
    return lib().f16wm_last_error().decode()


def version() -> str:
    return lib().f16wm_version().decode()


def takes_sgemm(rows: int, k: int, n: int) -> bool:
    """n >= 2 and rows % 4 == 0 and k % 8 == 0: the tinyBLAS order applies."""
    return bool(lib().f16wm_takes_sgemm(rows, k, n))


_F16_DTYPES = (torch.float16, torch.int16, torch.uint16)


def _f16(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a tensor" % name)
    if t.dtype not in _F16_DTYPES:
        raise TypeError("%s must hold f16 bit patterns (float16/int16/uint16), got %s" % (name, t.dtype))
    if not t.is_cuda:
        raise ValueError("%s must be on a GPU" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _f32(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype != torch.float32:
        raise TypeError("%s must be float32, got %s" % (name, t.dtype))
    if not t.is_cuda:
        raise ValueError("%s must be on a GPU" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _check(rc: int):
    if rc != F16WM_OK:
        raise F16WMError(rc, last_error())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def to_f16(x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Round f32 activations to f16 (nearest even): the same shape in float16."""
    _f32(x, "x")
    if out is None:
        out = torch.empty(x.shape, dtype=torch.float16, device=x.device)
    _f16(out, "out")
    if out.numel() != x.numel() or out.device != x.device:
        raise ValueError("out must match x in size and device")
    with torch.cuda.device(x.device):
        _check(lib().f16wm_to_f16(x.data_ptr(), out.data_ptr(), x.numel(), _stream(x.device)))
    return out


def widen(h: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Exact f16 -> f32 (same shape)."""
    _f16(h, "h")
    if out is None:
        out = torch.empty(h.shape, dtype=torch.float32, device=h.device)
    _f32(out, "out")
    if out.numel() != h.numel() or out.device != h.device:
        raise ValueError("out must match h in size and device")
    with torch.cuda.device(h.device):
        _check(lib().f16wm_widen(h.data_ptr(), out.data_ptr(), h.numel(), _stream(h.device)))
    return out


def get_rows(w: torch.Tensor, ids: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Rows ids of W [rows, k] widened to f32: [len(ids), k] (ids int64 on the
    GPU; an id outside [0, rows) gives a row of NaN)."""
    rows, k = _wk(w)
    if not isinstance(ids, torch.Tensor) or ids.dtype != torch.int64 or not ids.is_cuda \
            or not ids.is_contiguous():
        raise TypeError("ids must be a contiguous int64 GPU tensor")
    n = ids.numel()
    if out is None:
        out = torch.empty((n, k), dtype=torch.float32, device=w.device)
    _f32(out, "out")
    if out.numel() != n * k:
        raise ValueError("out must have len(ids)*k elements")
    with torch.cuda.device(w.device):
        _check(lib().f16wm_get_rows(w.data_ptr(), rows, k, ids.data_ptr(), n, out.data_ptr(),
                                    _stream(w.device)))
    return out


def _wk(w: torch.Tensor):
    _f16(w, "w")
    if w.dim() != 2:
        raise ValueError("w must be [rows, k]")
    return w.shape[0], w.shape[1]


def _act(a: torch.Tensor, name: str) -> bool:
    """Check an activation column: f16 bit patterns, or float32 (rounded to f16
    inside the product).  Returns True for float32."""
    if isinstance(a, torch.Tensor) and a.dtype == torch.float32:
        _f32(a, name)
        return True
    _f16(a, name)
    return False


def mat_vec(w: torch.Tensor, a: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """out[r] = vec_dot(W[r], a): W [rows, k] f16, a [k] f16 -> [rows] f32.
    A float32 `a` is rounded to f16 inside the same launch (equal to
    to_f16(a) first, bit for bit)."""
    rows, k = _wk(w)
    f32 = _act(a, "a")
    if a.numel() != k:
        raise ValueError("a must have k = %d elements" % k)
    if out is None:
        out = torch.empty(rows, dtype=torch.float32, device=w.device)
    _f32(out, "out")
    if out.numel() != rows:
        raise ValueError("out must have rows = %d elements" % rows)
    fn = lib().f16wm_mat_vec_f32 if f32 else lib().f16wm_mat_vec
    with torch.cuda.device(w.device):
        _check(fn(w.data_ptr(), rows, k, a.data_ptr(), out.data_ptr(), _stream(w.device)))
    return out


def mat_vec_multi(ws, a: torch.Tensor, outs=None) -> list:
    """Several matrices with the same k times one f16 column, in one launch
    (a float32 column is rounded to f16 inside that launch)."""
    ws = list(ws)
    if not 1 <= len(ws) <= MAX_MULTI:
        raise ValueError("1..%d matrices" % MAX_MULTI)
    k = None
    for w in ws:
        rows, kk = _wk(w)
        if k is None:
            k = kk
        elif kk != k:
            raise ValueError("all matrices must share k")
    f32 = _act(a, "a")
    if a.numel() != k:
        raise ValueError("a must have k = %d elements" % k)
    if outs is None:
        outs = [torch.empty(w.shape[0], dtype=torch.float32, device=w.device) for w in ws]
    outs = list(outs)
    if len(outs) != len(ws):
        raise ValueError("one output per matrix")
    mats = (_Mat * len(ws))()
    for i, (w, o) in enumerate(zip(ws, outs)):
        _f32(o, "outs[%d]" % i)
        if o.numel() != w.shape[0]:
            raise ValueError("outs[%d] must have %d elements" % (i, w.shape[0]))
        mats[i].w = w.data_ptr()
        mats[i].rows = w.shape[0]
        mats[i].out = o.data_ptr()
    dev = ws[0].device
    fn = lib().f16wm_mat_vec_multi_f32 if f32 else lib().f16wm_mat_vec_multi
    with torch.cuda.device(dev):
        _check(fn(mats, len(ws), k, a.data_ptr(), _stream(dev)))
    return outs


class VecTable:
    """A prepared f16wm_mat_vec_table call: the C descriptors of a fixed list
    of independent one-column products, built once so that a decode loop (or
    a HIP graph capture) pays only the library call.  The tensors must stay
    alive and in place while the table is used."""

    def __init__(self, prods):
        prods = list(prods)
        if len(prods) > MAX_TABLE:
            raise ValueError("at most %d products" % MAX_TABLE)
        arr = (_Gemv * max(1, len(prods)))()
        self.outs = []
        self.device = None
        for i, item in enumerate(prods):
            w, a = item[0], item[1]
            out = item[2] if len(item) > 2 else None
            rows, k = _wk(w)
            f32 = _act(a, "a")
            if a.numel() != k:
                raise ValueError("product %d: the column must have k = %d elements" % (i, k))
            if out is None:
                out = torch.empty(rows, dtype=torch.float32, device=w.device)
            _f32(out, "out")
            if out.numel() != rows:
                raise ValueError("product %d: out must have rows = %d elements" % (i, rows))
            if self.device is None:
                self.device = w.device
            if w.device != self.device or a.device != self.device or out.device != self.device:
                raise ValueError("every tensor of a table must be on one device")
            arr[i] = _Gemv(w.data_ptr(), a.data_ptr(), out.data_ptr(), rows, k, 1 if f32 else 0)
            self.outs.append(out)
        self._arr, self._n = arr, len(prods)
        self._keep = prods

    def __call__(self):
        """Launch every product (on the current stream); returns the outputs."""
        if self._n:
            with torch.cuda.device(self.device):
                _check(lib().f16wm_mat_vec_table(self._arr, self._n, _stream(self.device)))
        return self.outs


def mat_vec_table(prods) -> list:
    """Independent one-column products, each (w, a) or (w, a, out): W [rows, k]
    f16 times its own column a ([k] f16, or float32 rounded inside the launch),
    out [rows] f32, in as few launches as the library can (f16wm_mat_vec_table).
    Returns the outputs.  For repeated calls build a VecTable once."""
    return VecTable(prods)()


def _mm(fn, w, a, out, fn32=None):
    rows, k = _wk(w)
    if fn32 is not None and _act(a, "a"):
        fn = fn32
    else:
        _f16(a, "a")
    if a.dim() == 1:
        a = a.view(1, -1)
    if a.dim() != 2 or a.shape[1] != k:
        raise ValueError("a must be [n, k] with k = %d" % k)
    n = a.shape[0]
    if out is None:
        out = torch.empty((n, rows), dtype=torch.float32, device=w.device)
    _f32(out, "out")
    if out.numel() != n * rows:
        raise ValueError("out must have n*rows = %d elements" % (n * rows))
    with torch.cuda.device(w.device):
        _check(fn(w.data_ptr(), rows, k, a.data_ptr(), n, out.data_ptr(), _stream(w.device)))
    return out


def mat_mul(w: torch.Tensor, a: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Exact product in ggml's order for the shape: W [rows, k] x A [n, k] -> [n, rows] f32.
    A float32 `a` is rounded to f16 inside the same launch (equal to
    to_f16(a) first, bit for bit)."""
    return _mm(lib().f16wm_mat_mul, w, a, out, lib().f16wm_mat_mul_f32)


def mat_mul_mfma(w: torch.Tensor, a: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """The same product on the fp16 matrix cores (approximate, f32 accumulation)."""
    return _mm(lib().f16wm_mat_mul_mfma, w, a, out)


def _mm_multi(fn, ws, a, outs, fn32=None):
    ws = list(ws)
    if not 1 <= len(ws) <= MAX_MULTI:
        raise ValueError("1..%d matrices" % MAX_MULTI)
    k = None
    for w in ws:
        _, kk = _wk(w)
        if k is None:
            k = kk
        elif kk != k:
            raise ValueError("all matrices must share k")
    if fn32 is not None and _act(a, "a"):
        fn = fn32
    else:
        _f16(a, "a")
    if a.dim() == 1:
        a = a.view(1, -1)
    if a.dim() != 2 or a.shape[1] != k:
        raise ValueError("a must be [n, k] with k = %d" % k)
    n = a.shape[0]
    if outs is None:
        outs = [torch.empty((n, w.shape[0]), dtype=torch.float32, device=w.device) for w in ws]
    outs = list(outs)
    if len(outs) != len(ws):
        raise ValueError("one output per matrix")
    mats = (_Mat * len(ws))()
    for i, (w, o) in enumerate(zip(ws, outs)):
        _f32(o, "outs[%d]" % i)
        if o.numel() != n * w.shape[0]:
            raise ValueError("outs[%d] must have n*rows = %d elements" % (i, n * w.shape[0]))
        mats[i].w = w.data_ptr()
        mats[i].rows = w.shape[0]
        mats[i].out = o.data_ptr()
    dev = ws[0].device
    with torch.cuda.device(dev):
        _check(fn(mats, len(ws), k, a.data_ptr(), n, _stream(dev)))
    return outs


def mat_mul_multi(ws, a: torch.Tensor, outs=None) -> list:
    """Exact products of several matrices (same k) with one activation block
    [n, k]: one [n, rows_m] output each, each in its shape's order.  A float32
    block is rounded to f16 inside the launch (equal to to_f16 first)."""
    return _mm_multi(lib().f16wm_mat_mul_multi, ws, a, outs, lib().f16wm_mat_mul_multi_f32)


def mat_mul_mfma_multi(ws, a: torch.Tensor, outs=None) -> list:
    """The MFMA products of several matrices (same k) with one activation block, one launch."""
    return _mm_multi(lib().f16wm_mat_mul_mfma_multi, ws, a, outs)


# Which columns of a micro-batch leave the last layer (mat_mul_out).
OUT_NONE, OUT_LAST, OUT_ALL = 0, 1, 2


def mat_mul_out(w: torch.Tensor, a: torch.Tensor, mode: int, out: torch.Tensor | None = None):
    """The last layer's product over the columns that leave the model: mode
    OUT_NONE -> None, OUT_LAST -> [rows] (the last column alone: vec_dot),
    OUT_ALL -> [n, rows] (mat_mul)."""
    rows, k = _wk(w)
    _f16(a, "a")
    if a.dim() == 1:
        a = a.view(1, -1)
    if a.dim() != 2 or a.shape[1] != k:
        raise ValueError("a must be [n, k] with k = %d" % k)
    n = a.shape[0]
    if mode not in (OUT_NONE, OUT_LAST, OUT_ALL):
        raise ValueError("mode must be OUT_NONE, OUT_LAST or OUT_ALL")
    if mode == OUT_NONE:
        with torch.cuda.device(w.device):
            _check(lib().f16wm_mat_mul_out(w.data_ptr(), rows, k, a.data_ptr(), n, mode, None,
                                           _stream(w.device)))
        return None
    m = 1 if mode == OUT_LAST else n
    if out is None:
        out = torch.empty((rows,) if mode == OUT_LAST else (n, rows), dtype=torch.float32, device=w.device)
    _f32(out, "out")
    if out.numel() != m * rows:
        raise ValueError("out must have %d elements" % (m * rows))
    with torch.cuda.device(w.device):
        _check(lib().f16wm_mat_mul_out(w.data_ptr(), rows, k, a.data_ptr(), n, mode, out.data_ptr(),
                                       _stream(w.device)))
    return out


def kq(kc: torch.Tensor, q: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """vec_dot scores of queries q [n_head, d] against an f16 K cache kc
    [n_kv, n_kv_head, d] (grouped-query heads): [n_head, n_kv] f32."""
    _f16(kc, "kc")
    _f16(q, "q")
    if kc.dim() != 3 or q.dim() != 2 or q.shape[1] != kc.shape[2]:
        raise ValueError("kc must be [n_kv, n_kv_head, d] and q [n_head, d]")
    n_kv, n_kv_head, d = kc.shape
    n_head = q.shape[0]
    if out is None:
        out = torch.empty((n_head, n_kv), dtype=torch.float32, device=kc.device)
    _f32(out, "out")
    if out.numel() != n_head * n_kv:
        raise ValueError("out must have n_head*n_kv elements")
    with torch.cuda.device(kc.device):
        _check(lib().f16wm_kq(kc.data_ptr(), n_kv, n_kv_head, d, q.data_ptr(), n_head, out.data_ptr(),
                              _stream(kc.device)))
    return out


def _vecs(acc: torch.Tensor, f: torch.Tensor, fname: str):
    _f16(acc, "acc")
    if acc.dim() == 1:
        nvec, n = 1, acc.shape[0]
    elif acc.dim() == 2:
        nvec, n = acc.shape
    else:
        raise ValueError("acc must be [n] or [nvec, n]")
    _f32(f, fname)
    if f.numel() != nvec:
        raise ValueError("%s must have one value per vector (%d)" % (fname, nvec))
    return nvec, n


def mad(acc: torch.Tensor, v: torch.Tensor, w: torch.Tensor) -> torch.Tensor:
    """In place: acc[b] = f16(fma(v[b], w[b], acc[b])) for f16 acc, v [nvec, n]
    and f32 weights w [nvec] (all on the GPU).  Returns acc."""
    nvec, n = _vecs(acc, w, "w")
    _f16(v, "v")
    if v.numel() != acc.numel():
        raise ValueError("v must match acc")
    with torch.cuda.device(acc.device):
        _check(lib().f16wm_mad(acc.data_ptr(), v.data_ptr(), w.data_ptr(), nvec, n, _stream(acc.device)))
    return acc


def scale(acc: torch.Tensor, s: torch.Tensor) -> torch.Tensor:
    """In place: acc[b] = f16(acc[b] * s[b]) for f16 acc [nvec, n] and f32 s [nvec]."""
    nvec, n = _vecs(acc, s, "s")
    with torch.cuda.device(acc.device):
        _check(lib().f16wm_scale(acc.data_ptr(), s.data_ptr(), nvec, n, _stream(acc.device)))
    return acc
