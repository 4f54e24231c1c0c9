"""Host-side checks of the C-ABI library: it loads, exports every function the
header declares, and rejects bad arguments before any launch.  No kernel is
launched here; the GPU tests cover the compute.
"""
import ctypes
import os
import re

import pytest

import f16_weight_matrix_amd as f16wm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "f16wm.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(f16wm_[a-z0-9_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def L():
    return f16wm.lib()


def test_header_declares_the_boundary():
    assert _declared() == sorted([
        "f16wm_to_f16", "f16wm_widen", "f16wm_get_rows", "f16wm_mat_vec", "f16wm_mat_vec_multi",
        "f16wm_mat_vec_f32", "f16wm_mat_vec_multi_f32", "f16wm_mat_mul", "f16wm_mat_mul_mfma",
        "f16wm_mat_mul_multi", "f16wm_mat_mul_mfma_multi", "f16wm_takes_sgemm", "f16wm_last_error",
        "f16wm_version", "f16wm_mat_mul_out", "f16wm_kq", "f16wm_mad", "f16wm_scale",
        "f16wm_mat_mul_f32", "f16wm_mat_mul_multi_f32", "f16wm_mat_vec_table"])


def test_library_exports_every_declared_symbol(L):
    for name in _declared():
        assert hasattr(L, name), name


def test_exports_are_c_symbols():
    """extern "C": the dynamic symbol table holds the plain names."""
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", f16wm.LIB_PATH], capture_output=True,
                         text=True).stdout
    names = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in _declared():
        assert name in names, name


def test_version(L):
    assert "gfx950" in f16wm.version()


def test_takes_sgemm_rule(L):
    """The library's rule equals the page's n >= 2 && rows % 4 == 0 && k % 8 == 0
    over a grid of shapes; negative sizes give 0."""
    for rows in range(0, 20):
        for k in range(0, 40):
            for n in range(0, 5):
                want = n >= 2 and rows % 4 == 0 and k % 8 == 0
                assert f16wm.takes_sgemm(rows, k, n) is want, (rows, k, n)
    assert not f16wm.takes_sgemm(-4, 8, 2)
    assert not f16wm.takes_sgemm(4, -8, 2)
    assert not f16wm.takes_sgemm(4, 8, -2)


# Fake, never dereferenced device addresses: validation rejects before launch.
P = 1 << 40
STREAM = None


def _err(rc):
    assert rc == f16wm.F16WM_EINVAL, (rc, f16wm.last_error())
    return f16wm.last_error()


def test_mat_vec_rejects_bad_arguments(L):
    assert "negative" in _err(L.f16wm_mat_vec(P, -1, 8, P + 4096, P + 8192, STREAM))
    assert "negative" in _err(L.f16wm_mat_vec(P, 4, -8, P + 4096, P + 8192, STREAM))
    assert "null" in _err(L.f16wm_mat_vec(None, 4, 8, P + 4096, P + 8192, STREAM))
    assert "null" in _err(L.f16wm_mat_vec(P, 4, 8, None, P + 8192, STREAM))
    assert "null" in _err(L.f16wm_mat_vec(P, 4, 8, P + 4096, None, STREAM))
    assert "misaligned" in _err(L.f16wm_mat_vec(P + 1, 4, 8, P + 4096, P + 8192, STREAM))
    assert "misaligned" in _err(L.f16wm_mat_vec(P, 4, 8, P + 4096, P + 8194, STREAM))
    assert "too large" in _err(L.f16wm_mat_vec(P, 1 << 31, 1 << 31, P + 4096, P + 8192, STREAM))
    # out (4 rows x 4 bytes) overlapping w (4 x 8 x 2 bytes)
    assert "overlap" in _err(L.f16wm_mat_vec(P, 4, 8, P + 4096, P + 16, STREAM))
    assert "overlap" in _err(L.f16wm_mat_vec(P, 4, 8, P + 4096, P + 4096, STREAM))


def test_f32_activation_entry_points_reject_bad_arguments(L):
    assert "null" in _err(L.f16wm_mat_vec_f32(P, 4, 8, None, P + 8192, STREAM))
    assert "misaligned" in _err(L.f16wm_mat_vec_f32(P, 4, 8, P + 4098, P + 8192, STREAM))
    # out (4 floats) overlapping the f32 activation (8 floats = 32 bytes)
    assert "overlap" in _err(L.f16wm_mat_vec_f32(P, 4, 8, P + 4096, P + 4112, STREAM))
    Mat = f16wm._Mat
    mats = (Mat * 1)()
    mats[0].w, mats[0].rows, mats[0].out = P, 4, P + 4120
    assert "overlap" in _err(L.f16wm_mat_vec_multi_f32(mats, 1, 8, P + 4096, STREAM))
    assert L.f16wm_mat_vec_f32(P, 0, 8, P + 4096, P + 8192, STREAM) == 0


def test_widen_and_get_rows_reject_bad_arguments(L):
    assert "bad count" in _err(L.f16wm_widen(P, P + 4096, -1, STREAM))
    assert "misaligned" in _err(L.f16wm_widen(P, P + 4098, 4, STREAM))
    assert "overlap" in _err(L.f16wm_widen(P, P + 4, 4, STREAM))
    assert "negative" in _err(L.f16wm_get_rows(P, 4, 8, P + 4096, -1, P + 8192, STREAM))
    assert "null" in _err(L.f16wm_get_rows(P, 4, 8, None, 2, P + 8192, STREAM))
    assert "misaligned" in _err(L.f16wm_get_rows(P, 4, 8, P + 4100, 2, P + 8192, STREAM))
    assert "overlap" in _err(L.f16wm_get_rows(P, 4, 8, P + 4096, 2, P + 4100, STREAM))
    assert L.f16wm_get_rows(P, 4, 8, P + 4096, 0, P + 8192, STREAM) == 0


def test_mat_mul_rejects_bad_arguments(L):
    assert "negative" in _err(L.f16wm_mat_mul(P, 4, 8, P + 4096, -1, P + 8192, STREAM))
    assert "overlap" in _err(L.f16wm_mat_mul(P, 4, 8, P + 4096, 3, P + 4100, STREAM))
    assert "null" in _err(L.f16wm_mat_mul(P, 4, 8, None, 3, P + 8192, STREAM))
    assert "too large" in _err(L.f16wm_mat_mul(P, 1 << 21, 8, P, 1 << 21, P, STREAM))


def test_f32_activation_products_reject_bad_arguments(L):
    """f16wm_mat_mul_f32 / _multi_f32 check the f32 block as 4-byte elements:
    alignment, null, overlap with the output over n*k*4 bytes; an empty
    product returns 0 before any device call."""
    assert "misaligned" in _err(L.f16wm_mat_mul_f32(P, 4, 8, P + 4098, 3, P + 8192, STREAM))
    assert "null" in _err(L.f16wm_mat_mul_f32(P, 4, 8, None, 3, P + 8192, STREAM))
    # x spans 3 * 8 * 4 = 96 bytes from P + 4096: an output at P + 4160 overlaps it
    assert "overlap" in _err(L.f16wm_mat_mul_f32(P, 4, 8, P + 4096, 3, P + 4160, STREAM))
    assert L.f16wm_mat_mul_f32(P, 0, 8, P + 4096, 3, P + 8192, STREAM) == 0
    Mat = f16wm._Mat
    mats = (Mat * 1)()
    mats[0].w, mats[0].rows, mats[0].out = P, 4, P + (1 << 20)
    assert "count" in _err(L.f16wm_mat_mul_multi_f32(mats, 0, 8, P + (1 << 21), 3, STREAM))
    assert "misaligned" in _err(L.f16wm_mat_mul_multi_f32(mats, 1, 8, P + (1 << 21) + 2, 3, STREAM))


def test_grouped_products_reject_bad_arguments(L):
    Mat = f16wm._Mat
    mats = (Mat * 2)()
    mats[0].w, mats[0].rows, mats[0].out = P, 4, P + (1 << 20)
    mats[1].w, mats[1].rows, mats[1].out = P + 4096, 4, P + (1 << 20) + 16   # overlaps out[0] (n=3)
    assert "overlap" in _err(L.f16wm_mat_mul_multi(mats, 2, 8, P + (1 << 21), 3, STREAM))
    assert "count" in _err(L.f16wm_mat_mul_multi(mats, 0, 8, P + (1 << 21), 3, STREAM))
    assert "null" in _err(L.f16wm_mat_mul_mfma_multi(None, 2, 8, P + (1 << 21), 3, STREAM))
    mats[1].out = P + (1 << 20) + 4096
    rc = L.f16wm_mat_mul_mfma_multi(mats, 2, 12, P + (1 << 21), 3, STREAM)
    assert rc == f16wm.F16WM_EUNSUPPORTED
    mats[1].rows = 0
    mats[0].rows = 0
    assert L.f16wm_mat_mul_multi(mats, 2, 8, P + (1 << 21), 3, STREAM) == 0


def test_mat_mul_mfma_rejects_unsupported(L):
    rc = L.f16wm_mat_mul_mfma(P, 4, 12, P + 4096, 3, P + 8192, STREAM)
    assert rc == f16wm.F16WM_EUNSUPPORTED and "k % 8" in f16wm.last_error()
    rc = L.f16wm_mat_mul_mfma(P + 2, 4, 16, P + 4096, 3, P + 8192, STREAM)
    assert rc == f16wm.F16WM_EUNSUPPORTED


def test_to_f16_rejects_bad_arguments(L):
    assert "bad count" in _err(L.f16wm_to_f16(P, P + 4096, -1, STREAM))
    assert "null" in _err(L.f16wm_to_f16(None, P + 4096, 4, STREAM))
    assert "misaligned" in _err(L.f16wm_to_f16(P + 2, P + 4096, 4, STREAM))
    assert "overlap" in _err(L.f16wm_to_f16(P, P + 8, 4, STREAM))


def test_mat_vec_multi_rejects_bad_arguments(L):
    Mat = f16wm._Mat
    mats = (Mat * 2)()
    mats[0].w, mats[0].rows, mats[0].out = P, 4, P + (1 << 20)
    mats[1].w, mats[1].rows, mats[1].out = P + 4096, 4, P + (1 << 20) + 8   # overlaps out[0]
    assert "overlap" in _err(L.f16wm_mat_vec_multi(mats, 2, 8, P + (1 << 21), STREAM))
    assert "count" in _err(L.f16wm_mat_vec_multi(mats, 0, 8, P + (1 << 21), STREAM))
    assert "count" in _err(L.f16wm_mat_vec_multi(mats, 9, 8, P + (1 << 21), STREAM))
    assert "null" in _err(L.f16wm_mat_vec_multi(None, 2, 8, P + (1 << 21), STREAM))
    mats[1].out = P + (1 << 20) + 4096
    mats[1].rows = -1
    assert "negative" in _err(L.f16wm_mat_vec_multi(mats, 2, 8, P + (1 << 21), STREAM))


def _table(items):
    G = f16wm._Gemv
    arr = (G * max(1, len(items)))()
    for i, (w, a, out, rows, k, f32) in enumerate(items):
        arr[i] = G(w, a, out, rows, k, f32)
    return arr


def test_mat_vec_table_rejects_bad_arguments(L):
    """f16wm_mat_vec_table validates every product as f16wm_mat_vec does and
    refuses outputs that overlap another output, a weight or a column, all
    before any device call (the pointers here are never dereferenced)."""
    good = (P, P + 4096, P + 8192, 4, 8, 0)
    t = _table([good])
    assert "count" in _err(L.f16wm_mat_vec_table(t, -1, STREAM))
    assert "count" in _err(L.f16wm_mat_vec_table(t, f16wm.MAX_TABLE + 1, STREAM))
    assert "null table" in _err(L.f16wm_mat_vec_table(None, 2, STREAM))
    assert L.f16wm_mat_vec_table(None, 0, STREAM) == 0
    assert "a_f32" in _err(L.f16wm_mat_vec_table(_table([(P, P + 4096, P + 8192, 4, 8, 2)]), 1, STREAM))
    msg = _err(L.f16wm_mat_vec_table(_table([good, (P, P + 4096, P + 8192, -4, 8, 0)]), 2, STREAM))
    assert "[1]" in msg and "negative" in msg
    assert "null" in _err(L.f16wm_mat_vec_table(_table([(P, None, P + 8192, 4, 8, 0)]), 1, STREAM))
    assert "misaligned" in _err(L.f16wm_mat_vec_table(_table([(P, P + 4098, P + 8192, 4, 8, 1)]), 1, STREAM))
    # two outputs overlap: 4 floats at P + 8192 and at P + 8200
    two = [good, (P + 65536, P + 4096, P + 8200, 4, 8, 0)]
    assert "two outputs" in _err(L.f16wm_mat_vec_table(_table(two), 2, STREAM))
    # an output overlaps another product's weight (4 x 8 halves at P + 65536)
    cross = [good, (P + 65536, P + 4096, P + 12288, 4, 8, 0), (P + 16384, P + 4096, P + 65540, 1, 8, 0)]
    assert "weight or column" in _err(L.f16wm_mat_vec_table(_table(cross), 3, STREAM))
    # ... or another product's f32 column (8 floats at P + 4096)
    col = [(P, P + 4096, P + 8192, 4, 8, 1), (P + 65536, P + 12288, P + 4124, 1, 8, 0)]
    assert "weight or column" in _err(L.f16wm_mat_vec_table(_table(col), 2, STREAM))
    # shared weights and columns are fine, and so are empty products
    shared = [(P, P + 4096, P + 8192, 4, 8, 0), (P, P + 4096, P + 12288, 4, 8, 0), (P, P + 4096, P + 8192, 0, 8, 0)]
    assert L.f16wm_mat_vec_table(_table(shared[2:]), 1, STREAM) == 0
    import torch
    if not torch.cuda.is_available():
        rc = L.f16wm_mat_vec_table(_table(shared), 3, STREAM)
        assert rc == f16wm.F16WM_ENODEV, (rc, f16wm.last_error())


def test_next_rows_reject_bad_arguments(L):
    # the last layer's output columns
    assert "mode" in _err(L.f16wm_mat_mul_out(P, 4, 8, P + 4096, 3, 7, P + 8192, STREAM))
    assert "negative" in _err(L.f16wm_mat_mul_out(P, 4, 8, P + 4096, -1, 1, P + 8192, STREAM))
    assert "empty" in _err(L.f16wm_mat_mul_out(P, 4, 8, P + 4096, 0, 1, P + 8192, STREAM))
    assert L.f16wm_mat_mul_out(P, 4, 8, P + 4096, 3, 0, None, STREAM) == 0     # none: nothing to do
    assert "overlap" in _err(L.f16wm_mat_mul_out(P, 4, 8, P + 4096, 3, 1, P + 4, STREAM))
    # K-cache scores
    assert "multiple" in _err(L.f16wm_kq(P, 16, 3, 64, P + 65536, 8, P + (1 << 20), STREAM))
    assert "multiple" in _err(L.f16wm_kq(P, 16, 0, 64, P + 65536, 8, P + (1 << 20), STREAM))
    assert "negative" in _err(L.f16wm_kq(P, -1, 2, 64, P + 65536, 8, P + (1 << 20), STREAM))
    assert "null" in _err(L.f16wm_kq(P, 16, 2, 64, None, 8, P + (1 << 20), STREAM))
    assert "misaligned" in _err(L.f16wm_kq(P + 1, 16, 2, 64, P + 65536, 8, P + (1 << 20), STREAM))
    assert "overlap" in _err(L.f16wm_kq(P, 16, 2, 64, P + 65536, 8, P + 8, STREAM))
    assert L.f16wm_kq(P, 0, 2, 64, P + 65536, 8, P + (1 << 20), STREAM) == 0
    # mad / scale
    assert "bad size" in _err(L.f16wm_mad(P, P + 4096, P + 8192, -1, 8, STREAM))
    assert "null" in _err(L.f16wm_mad(P, None, P + 8192, 2, 8, STREAM))
    assert "overlap" in _err(L.f16wm_mad(P, P + 8, P + 8192, 2, 8, STREAM))
    assert "misaligned" in _err(L.f16wm_scale(P + 1, P + 8192, 2, 8, STREAM))
    assert "overlap" in _err(L.f16wm_scale(P, P + 4, 2, 8, STREAM))
    assert L.f16wm_scale(P, P + 8192, 0, 8, STREAM) == 0


def test_empty_products_are_no_ops(L):
    """rows = 0 or n = 0: nothing to do, success without touching a device."""
    assert L.f16wm_mat_vec(P, 0, 8, P + 4096, P + 8192, STREAM) == 0
    assert L.f16wm_mat_mul(P, 4, 8, P + 4096, 0, P + 8192, STREAM) == 0
    assert L.f16wm_mat_mul(P, 0, 8, P + 4096, 3, P + 8192, STREAM) == 0
    assert L.f16wm_mat_mul_mfma(P, 0, 8, P + 4096, 3, P + 8192, STREAM) == 0
    assert L.f16wm_to_f16(P, P + 4096, 0, STREAM) == 0
    assert f16wm.last_error() == ""


def test_no_device_is_reported_not_launched(L):
    """Valid arguments with no GPU present: F16WM_ENODEV, nothing launched."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    rc = L.f16wm_mat_vec(P, 4, 8, P + 4096, P + 8192, STREAM)
    assert rc == f16wm.F16WM_ENODEV, (rc, f16wm.last_error())
    assert "device" in f16wm.last_error()


def test_binding_rejects_cpu_tensors():
    import torch
    w = torch.zeros(4, 8, dtype=torch.float16)
    a = torch.zeros(8, dtype=torch.float16)
    with pytest.raises(ValueError):
        f16wm.mat_vec(w, a)
    with pytest.raises(TypeError):
        f16wm.mat_vec(w.float(), a)
