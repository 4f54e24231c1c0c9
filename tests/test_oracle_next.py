"""Pins of the oracle's next rows: the last layer's output columns, vec_dot over
an f16 K cache (scores), and the V-accumulator helpers mad and scale.

- mat_mul_out (bankML page "bankML/forward.rs", section "Why only the output
  rows leave the last layer"): the page's claim that the number of output rows
  changes the bits of an F16 product (one column takes vec_dot, all of them
  tinyBLAS when takes_sgemm holds), the column it selects (exact integer sums),
  and that "none" writes nothing.
- kq (f16 page, Technical usage vec_dot_u16): exact integer sums and one-hot
  queries pin the cache layout [n_kv][n_kv_head][d] and the grouped-query head
  mapping; an error bound against the exact fixed-point sum pins accuracy.
- mad / scale (f16 page, Technical usage): each element against the exact
  rational value rounded once to binary32 (round to nearest even, written here
  from the format) and then to binary16 by numpy's cast (itself pinned
  exhaustively against F16C).  mad's fused reading is "parity partly
  unpinned": the page names the helper, not its arithmetic.
"""
from fractions import Fraction
import math

import numpy as np
import pytest

F = np.float16


def f32_rne(x: Fraction) -> float:
    """The exact rational x rounded to binary32, nearest even (x != 0)."""
    sign = -1.0 if x < 0 else 1.0
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    assert Fraction(2) ** e <= a < Fraction(2) ** (e + 1)
    e = max(e, -126)                       # subnormals share the 2^-149 quantum
    q = Fraction(2) ** (e - 23)
    m = a / q
    fl = math.floor(m)
    r = m - fl
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = fl * q
    if v >= Fraction(2) ** 128:
        return sign * math.inf
    return sign * float(v)


def rand_f16(rng, shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(F)


# ---------------------------------------------------------------- mat_mul_out

def test_out_none_writes_nothing(orc):
    w = np.zeros((12, 64), np.uint16)
    a = np.zeros((5, 64), np.uint16)
    assert orc.mat_mul_out(w, a, orc.OUT_NONE) is None


@pytest.mark.parametrize("rows,k,n", [(12, 64, 5), (13, 64, 5), (12, 33, 3), (16, 1536, 4)])
def test_out_last_selects_the_last_column(orc, rows, k, n):
    # small integers: every order gives the exact integer sum
    rng = np.random.default_rng(rows * 1000 + k)
    w = rng.integers(-3, 4, (rows, k)).astype(F)
    a = rng.integers(-3, 4, (n, k)).astype(F)
    want = (w.astype(np.int64) @ a[-1].astype(np.int64)).astype(np.float32)
    got = orc.mat_mul_out(w.view(np.uint16), a.view(np.uint16), orc.OUT_LAST)
    assert got.shape == (rows,) and np.array_equal(got, want)
    full = orc.mat_mul_out(w.view(np.uint16), a.view(np.uint16), orc.OUT_ALL)
    assert full.shape == (n, rows)
    assert np.array_equal(full, (a.astype(np.int64) @ w.astype(np.int64).T).astype(np.float32))


def test_out_rows_change_the_bits_where_the_page_says(orc):
    # the page: one output row takes vec_dot, all rows take tinyBLAS (12 rows,
    # k % 8 == 0), so the last column's bits differ somewhere; with 13 rows
    # both are vec_dot and agree everywhere
    rng = np.random.default_rng(5)
    a = rand_f16(rng, (4, 576)).view(np.uint16)
    w12 = rand_f16(rng, (12, 576), 0.02).view(np.uint16)
    last = orc.mat_mul_out(w12, a, orc.OUT_LAST)
    full = orc.mat_mul_out(w12, a, orc.OUT_ALL)
    assert orc.takes_sgemm(12, 576, 4) and not orc.takes_sgemm(12, 576, 1)
    assert (last.view(np.uint32) != full[-1].view(np.uint32)).any()
    w13 = rand_f16(rng, (13, 576), 0.02).view(np.uint16)
    assert np.array_equal(orc.mat_mul_out(w13, a, orc.OUT_LAST).view(np.uint32),
                          orc.mat_mul_out(w13, a, orc.OUT_ALL)[-1].view(np.uint32))


# ---------------------------------------------------------------------- kq

@pytest.mark.parametrize("n_kv,n_kv_head,d,n_head", [(7, 2, 64, 8), (33, 3, 64, 9), (5, 1, 128, 3),
                                                     (9, 4, 72, 4), (4, 2, 8, 2), (3, 8, 128, 32)])
def test_kq_exact_integers_pin_layout_and_heads(orc, n_kv, n_kv_head, d, n_head):
    rng = np.random.default_rng(n_kv * 7 + d)
    kc = rng.integers(-4, 5, (n_kv, n_kv_head, d)).astype(F)
    q = rng.integers(-4, 5, (n_head, d)).astype(F)
    G = n_head // n_kv_head
    want = np.empty((n_head, n_kv), np.float32)
    for h_ in range(n_head):
        want[h_] = (kc[:, h_ // G, :].astype(np.int64) @ q[h_].astype(np.int64)).astype(np.float32)
    got = orc.kq(kc, q)
    assert np.array_equal(got, want)


def test_kq_one_hot_queries_pick_cache_elements(orc):
    rng = np.random.default_rng(11)
    n_kv, n_kv_head, d, n_head = 6, 2, 64, 6
    kc = rand_f16(rng, (n_kv, n_kv_head, d))
    for i in (0, 7, 31, 32, 63):
        q = np.zeros((n_head, d), F)
        q[:, i] = 1
        got = orc.kq(kc, q)
        for h_ in range(n_head):
            assert np.array_equal(got[h_], kc[:, h_ // 3, i].astype(np.float32))


def test_kq_within_the_vec_dot_error_bound(orc):
    rng = np.random.default_rng(12)
    kc = rand_f16(rng, (16, 2, 128))
    q = rand_f16(rng, (4, 128))
    got = orc.kq(kc, q)
    u = 2.0 ** -24
    m = 128 // 32 + 6
    gam = m * u / (1 - m * u)
    for h_ in range(4):
        for p in range(16):
            s, sa = orc.exact_dot(kc[p, h_ // 2].view(np.uint16), q[h_].view(np.uint16))
            assert abs(float(got[h_, p]) - s) <= gam * sa + 1e-45


# ---------------------------------------------------------------- mad / scale

def _exact_mad(acc16, v16, w32):
    out = np.empty(acc16.shape, F)
    for idx in np.ndindex(acc16.shape):
        a_, v_, w_ = float(acc16[idx]), float(v16[idx]), float(w32[idx[0]])
        ex = Fraction(v_) * Fraction(w_) + Fraction(a_)
        if ex == 0:
            prod_neg = math.copysign(1.0, v_) * math.copysign(1.0, w_) < 0
            r = -0.0 if (prod_neg and math.copysign(1.0, a_) < 0) else 0.0
        else:
            r = f32_rne(ex)
        out[idx] = np.float32(r).astype(F)
    return out


def _exact_scale(acc16, s32):
    out = np.empty(acc16.shape, F)
    for idx in np.ndindex(acc16.shape):
        a_, s_ = float(acc16[idx]), float(s32[idx[0]])
        ex = Fraction(a_) * Fraction(s_)
        r = math.copysign(0.0, a_ * s_) if ex == 0 else f32_rne(ex)
        out[idx] = np.float32(r).astype(F)
    return out


def test_mad_equals_the_exact_value_rounded_to_f32_then_f16(orc):
    rng = np.random.default_rng(21)
    nvec, n = 6, 67                       # odd length, as the page's check
    acc = rand_f16(rng, (nvec, n), 4.0)
    acc[0, :5] = [0.0, -0.0, 6.1e-5, -3e-8, 65504.0]
    v = rand_f16(rng, (nvec, n))
    v[1, :3] = [0.0, -0.0, 1e-7]
    w = (rng.standard_normal(nvec) * 3).astype(np.float32)
    w[2] = 0.0
    w[3] = np.float32(1.0000001)
    got = orc.mad(acc.view(np.uint16), v.view(np.uint16), w).view(F)
    want = _exact_mad(acc, v, w)
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


def test_mad_double_rounding_cases(orc):
    # values whose exact result lies just off an f16 tie: rounding the exact
    # sum straight to f16 and going through f32 first can differ; the
    # definition goes through f32 (the FMA result), then f16
    acc = np.array([[1.0, 1.0, -1.0, 2048.0]], F)
    v = np.array([[2.0 ** -11, 2.0 ** -11, 2.0 ** -11, 1.0]], F)
    w = np.array([1.0 + 2.0 ** -23], np.float32)
    got = orc.mad(acc.view(np.uint16), v.view(np.uint16), w).view(F)
    assert np.array_equal(got.view(np.uint16), _exact_mad(acc, v, w).view(np.uint16))


def test_mad_under_cancellation(orc):
    # acc close to -v*w: the result is a small residual whose f16 bits show
    # the product's low bits, which a separately rounded product would lose
    rng = np.random.default_rng(23)
    nvec, n = 8, 256
    v = rand_f16(rng, (nvec, n))
    w = (rng.standard_normal(nvec) * 3).astype(np.float32)
    acc = (-(v.astype(np.float32) * w[:, None])).astype(F)
    got = orc.mad(acc.view(np.uint16), v.view(np.uint16), w).view(F)
    assert np.array_equal(got.view(np.uint16), _exact_mad(acc, v, w).view(np.uint16))


def test_scale_equals_the_exact_product_rounded_to_f32_then_f16(orc):
    rng = np.random.default_rng(22)
    nvec, n = 5, 33
    acc = rand_f16(rng, (nvec, n), 8.0)
    acc[0, :4] = [0.0, -0.0, 6e-8, 65504.0]
    s = (rng.standard_normal(nvec)).astype(np.float32)
    s[1] = 1.0
    s[2] = 0.25
    got = orc.scale(acc.view(np.uint16), s).view(F)
    assert np.array_equal(got.view(np.uint16), _exact_scale(acc, s).view(np.uint16))
    assert np.array_equal(got[1].view(np.uint16), acc[1].view(np.uint16))      # s = 1
    assert np.array_equal(got[2].astype(np.float64) * 4, acc[2].astype(np.float64))   # 2^-2, no underflow here
