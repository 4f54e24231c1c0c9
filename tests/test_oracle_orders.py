"""Pins of the oracle's two reduction orders, its path choice and its products.

The bankML f16 page (Design notes) defines:
  vec_dot  -- four 8-lane f32 FMA accumulators over 32-element steps, reduced
              (a0+a2)+(a1+a3), low half + high half, two horizontal adds, the
              k % 32 tail added in double;
  sgemm    -- one 8-lane FMA chain, hsum ((l0+l4)+(l2+l6))+((l1+l5)+(l3+l7));
  takes_sgemm(rows, k, n) = n >= 2 and rows % 4 == 0 and k % 8 == 0.
The page prints no worked example, so each pin below is derived: exact integer
sums, one-hot rows, hand-built inputs whose value under each tree is worked out
by hand (cases A-E), invariance groups of each tree, textbook summation for
k < 32, an error bound against an exact fixed-point sum, and the point the
page makes in its Summary, that one row and column reduced in the two orders
need not agree bit for bit.  A dropped
or repeated term, a wrong sign or index, a transposed operand, a wrong tree
level or a tail summed in f32 each fails at least one of them.
"""
import numpy as np
import pytest

import synth

F = np.float16


def h(vals):
    """f16 bit patterns of exactly-representable values."""
    a = np.asarray(vals, dtype=np.float64)
    b = a.astype(F)
    assert np.array_equal(b.astype(np.float64), a), "value not exact in f16"
    return b.view(np.uint16)


def vec(k, entries):
    """Length-k f16 vector, zero except entries {index: value}."""
    v = np.zeros(k, dtype=np.float64)
    for i, x in entries.items():
        v[i] = x
    return h(v)


# ---------------------------------------------------------------- cases A-E
# Each case is built so the order's tree gives a value that a nearby wrong tree
# does not; the expected values are worked out in the comments (2^30 + 1 rounds
# to 2^30 in binary32).

def test_case_A_pairs_accumulators_0_2_and_1_3(orc):
    # products: +2^30 at element 0 (acc 0), -2^30 at 16 (acc 2), +1 at 8 (acc 1)
    # (a0+a2)+(a1+a3) = 0 + 1 = 1;  (a0+a1)+(a2+a3) would give 2^30 - 2^30 = 0
    x = vec(32, {0: 2 ** 15, 16: -(2 ** 15), 8: 1})
    y = vec(32, {0: 2 ** 15, 16: 2 ** 15, 8: 1})
    assert orc.vec_dot(x, y) == np.float32(1.0)


def test_case_B_low_plus_high_half(orc):
    # products +2^30 at lane 0, -2^30 at lane 4, +1 at lane 1 (all in acc 0)
    # u0 = s0 + s4 = 0, u1 = s1 + s5 = 1 -> 1;  adjacent-first would give 0
    x = vec(32, {0: 2 ** 15, 4: -(2 ** 15), 1: 1})
    y = vec(32, {0: 2 ** 15, 4: 2 ** 15, 1: 1})
    assert orc.vec_dot(x, y) == np.float32(1.0)


def test_case_C_hadd_pairing_vs_hsum(orc):
    # products +2^30, -2^30, +1 at lanes 0, 1, 2
    # vec_dot: (u0+u1)+(u2+u3) = 0 + 1 = 1
    # sgemm:   ((l0+l4)+(l2+l6)) + ((l1+l5)+(l3+l7)) = (2^30 + 1) - 2^30 = 0
    x = vec(32, {0: 2 ** 15, 1: -(2 ** 15), 2: 1})
    y = vec(32, {0: 2 ** 15, 1: 2 ** 15, 2: 1})
    assert orc.vec_dot(x, y) == np.float32(1.0)
    assert orc.sgemm_dot(x, y) == np.float32(0.0)


def test_case_D_tail_added_in_double(orc):
    # k = 63: product 1 at element 0, then 31 tail products of 2^-26.
    # double: 1 + 31*2^-26, rounded once to f32 -> 1 + 2^-21.
    # An f32 tail would stay at 1.0 (each 2^-26 is under half an ulp of 1).
    x = vec(63, {0: 1, **{i: 2.0 ** -13 for i in range(32, 63)}})
    y = vec(63, {0: 1, **{i: 2.0 ** -13 for i in range(32, 63)}})
    assert orc.vec_dot(x, y) == np.float32(1.0 + 2.0 ** -21)


def test_case_E_vector_part_rounded_to_f32_before_tail(orc):
    # k = 33: products 1 (element 0), 2^-24 (element 1), tail -1 (element 32).
    # f32 tree: 1 + 2^-24 is a tie -> 1.0; then 1.0 - 1 = +0.0.
    # A reduction kept in double would give 2^-24.
    x = vec(33, {0: 1, 1: 2.0 ** -12, 32: -1})
    y = vec(33, {0: 1, 1: 2.0 ** -12, 32: 1})
    r = orc.vec_dot(x, y)
    assert r == 0.0 and not np.signbit(r)


# ------------------------------------------------------ exact special cases

@pytest.mark.parametrize("k", list(range(1, 100)) + [127, 128, 129, 255, 511, 576, 1023, 1536, 1540])
def test_integer_inputs_sum_exactly(orc, k):
    """Small integers: every partial sum is an integer below 2^24, so every
    order gives the exact sum.  Catches dropped, repeated or misplaced terms."""
    rng = np.random.default_rng(k)
    x = rng.integers(-8, 9, size=k)
    y = rng.integers(-8, 9, size=k)
    exact = float(np.dot(x.astype(np.int64), y.astype(np.int64)))
    assert orc.vec_dot(h(x), h(y)) == np.float32(exact)
    if k % 8 == 0:
        assert orc.sgemm_dot(h(x), h(y)) == np.float32(exact)


@pytest.mark.parametrize("k", [1, 7, 8, 31, 32, 33, 64, 100, 576, 1540])
def test_one_hot(orc, k):
    """x = +-e_i picks out +-y_i exactly, for every position i (indexing and sign)."""
    y = synth.random_f16(1000 + k, (k,))
    yv = y.view(F).astype(np.float32)
    for i in range(k):
        for s in (1, -1):
            x = vec(k, {i: s})
            assert orc.vec_dot(x, y) == s * yv[i]
            if k % 8 == 0:
                assert orc.sgemm_dot(x, y) == s * yv[i]


# -------------------------------------------------------- tree invariances

def _perm_vec_dot(k, groups):
    """Permutation of element indices that swaps, inside every 32-element step,
    the given (j, l) positions (j = accumulator, l = lane)."""
    p = np.arange(k)
    for t in range(k // 32):
        for (a, b) in groups:
            ia, ib = 32 * t + a, 32 * t + b
            p[ia], p[ib] = ib, ia
    return p


def _perm_sgemm(k, lanes):
    p = np.arange(k)
    for t in range(k // 8):
        for (a, b) in lanes:
            p[8 * t + a], p[8 * t + b] = 8 * t + b, 8 * t + a
    return p


def _acc_swap(ja, jb):
    return [(8 * ja + l, 8 * jb + l) for l in range(8)]


def _lane_swap(pairs):
    return [(8 * j + a, 8 * j + b) for j in range(4) for (a, b) in pairs]


VD_INVARIANT = {
    "acc0<->acc2": _acc_swap(0, 2),
    "acc1<->acc3": _acc_swap(1, 3),
    "lane l<->l+4": _lane_swap([(0, 4), (1, 5), (2, 6), (3, 7)]),
    "lanes 0<->1,4<->5": _lane_swap([(0, 1), (4, 5)]),
}
VD_NOT_INVARIANT = {
    "acc0<->acc1": _acc_swap(0, 1),
    "lanes 0<->2,4<->6": _lane_swap([(0, 2), (4, 6)]),
}
SG_INVARIANT = {
    "lane l<->l+4": [(0, 4), (1, 5), (2, 6), (3, 7)],
    "lanes 0<->2,4<->6": [(0, 2), (4, 6)],
}
SG_NOT_INVARIANT = {
    "lanes 0<->1,4<->5": [(0, 1), (4, 5)],
}


def _trials(k=576, n=60):
    for s in range(n):
        yield synth.random_f16((7, s), (k,)), synth.random_f16((8, s), (k,))


def test_vec_dot_tree_invariances(orc):
    """Permutations the (a0+a2)+(a1+a3) / low+high / hadd tree cannot see leave
    the bits unchanged; the ones it can see change them on some inputs."""
    k = 576
    for name, g in VD_INVARIANT.items():
        p = _perm_vec_dot(k, g)
        for x, y in _trials(k):
            assert orc.vec_dot(x[p], y[p]) == orc.vec_dot(x, y), name
    for name, g in VD_NOT_INVARIANT.items():
        p = _perm_vec_dot(k, g)
        diff = sum(orc.vec_dot(x[p], y[p]) != orc.vec_dot(x, y) for x, y in _trials(k))
        assert diff >= 1, name


def test_sgemm_tree_invariances(orc):
    k = 576
    for name, g in SG_INVARIANT.items():
        p = _perm_sgemm(k, g)
        for x, y in _trials(k):
            assert orc.sgemm_dot(x[p], y[p]) == orc.sgemm_dot(x, y), name
    for name, g in SG_NOT_INVARIANT.items():
        p = _perm_sgemm(k, g)
        diff = sum(orc.sgemm_dot(x[p], y[p]) != orc.sgemm_dot(x, y) for x, y in _trials(k))
        assert diff >= 1, name


def test_chain_order_matters_within_a_lane(orc):
    """Each chain adds in ascending step order: reversing the steps of one
    chain changes the result on some inputs, reversing nothing does not."""
    k = 576
    diff_vd = diff_sg = 0
    for x, y in _trials(k):
        # reverse the step order of all chains at once (whole 32-blocks / 8-blocks)
        pv = np.concatenate([np.arange(32 * t, 32 * t + 32) for t in reversed(range(k // 32))])
        ps = np.concatenate([np.arange(8 * t, 8 * t + 8) for t in reversed(range(k // 8))])
        diff_vd += orc.vec_dot(x[pv], y[pv]) != orc.vec_dot(x, y)
        diff_sg += orc.sgemm_dot(x[ps], y[ps]) != orc.sgemm_dot(x, y)
    assert diff_vd >= 1 and diff_sg >= 1


def test_sign_and_power_of_two_scaling(orc):
    for x, y in _trials(576, 20):
        nx = (x ^ np.uint16(0x8000))
        assert orc.vec_dot(nx, y) == -orc.vec_dot(x, y)
        assert orc.sgemm_dot(nx, y) == -orc.sgemm_dot(x, y)
        y2 = (y.view(F).astype(np.float32) * 4).astype(F).view(np.uint16)  # exact: |y| small
        assert orc.vec_dot(x, y2) == 4 * orc.vec_dot(x, y)
        assert orc.sgemm_dot(x, y2) == 4 * orc.sgemm_dot(x, y)


# ------------------------------------------------------------ closed forms

@pytest.mark.parametrize("k", range(1, 32))
def test_short_rows_are_a_double_sum(orc, k):
    """k < 32: no 32-element step, so vec_dot is the textbook left-to-right
    binary64 sum of the exact products, rounded once to f32."""
    for s in range(5):
        x = synth.random_f16((k, s, 1), (k,))
        y = synth.random_f16((k, s, 2), (k,))
        xs = x.view(F).astype(np.float64)
        ys = y.view(F).astype(np.float64)
        d = 0.0
        for i in range(k):
            d = d + float(xs[i]) * float(ys[i])   # each product exact in binary64
        assert orc.vec_dot(x, y) == np.float32(d)


# --------------------------------------------------- error against exact sum

U = 2.0 ** -24


def _gamma(m):
    return m * U / (1 - m * U)


@pytest.mark.parametrize("k", [8, 32, 40, 63, 64, 576, 1536, 1540, 4096, 14336])
def test_within_error_bound_of_exact_sum(orc, k):
    """Recursive summation bound: |computed - exact| <= gamma_m * sum|x_i y_i|,
    m = longest chain + tree depth + final rounding (u = 2^-24).  The exact
    sum comes from a fixed-point sum of the products (integers times 2^-48)."""
    for s in range(10):
        x = synth.random_f16((k, s, 3), (k,), 0.02)
        y = synth.random_f16((k, s, 4), (k,))
        ex, sa = orc.exact_dot(x, y)
        vd = float(orc.vec_dot(x, y))
        assert abs(vd - ex) <= _gamma(k // 32 + 6) * sa + 64 * 2.0 ** -53 * sa
        if k % 8 == 0:
            sg = float(orc.sgemm_dot(x, y))
            assert abs(sg - ex) <= _gamma(k // 8 + 3) * sa


def test_exact_dot_against_fraction_arithmetic(orc):
    """The fixed-point exact sum itself, against Python's exact rationals."""
    from fractions import Fraction
    for s in range(20):
        k = 1 + 37 * s
        x = synth.random_f16((s, 5), (k,), 3.0)
        y = synth.random_f16((s, 6), (k,), 300.0)
        xs = x.view(F).astype(np.float64)
        ys = y.view(F).astype(np.float64)
        exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(xs, ys))
        got, _ = orc.exact_dot(x, y)
        assert got == float(exact)


# ----------------------------------------------------------- path choice

def test_takes_sgemm_truth_table(orc):
    """n >= 2 and rows % 4 == 0 and k % 8 == 0 (f16 page, Technical usage)."""
    table = {
        (12, 1536, 2): True, (13, 1536, 2): False, (12, 1540, 2): False,
        (12, 1536, 1): False, (12, 8, 6): True, (12, 31, 3): False, (12, 33, 3): False,
        (16, 576, 512): True, (576, 576, 3): True, (576, 576, 1): False,
        (4, 8, 2): True, (0, 8, 2): True, (4, 0, 2): True, (2, 8, 2): False,
        (49152, 576, 512): True, (128256, 4096, 512): True,
    }
    for (r, k, n), want in table.items():
        assert orc.takes_sgemm(r, k, n) is want, (r, k, n)


def test_the_two_reductions_differ(orc):
    """f16 page, Summary: the vec_dot and tinyBLAS reductions of one row and
    one column are not bit-interchangeable, which is why the shape rule that
    picks between them needs its own check.  Here most elements of the 576x576
    weight times 3 f16-rounded N(0,1) columns come out differently in the two
    orders, while staying within rounding distance of each other."""
    w, a = synth.c1()
    a16 = orc.to_f16(a)
    vd = np.array([[orc.vec_dot(w[r], a16[c]) for r in range(576)] for c in range(3)])
    sg = np.array([[orc.sgemm_dot(w[r], a16[c]) for r in range(576)] for c in range(3)])
    ndiff = int(np.count_nonzero(vd != sg))
    assert ndiff > 0
    # both still agree closely (same exact sum, different rounding order)
    assert np.max(np.abs(vd - sg)) < 1e-5


# --------------------------------------------------------------- products

def test_mat_mul_layout_out_c_rows_plus_r(orc):
    """W = identity rows, so element (r, c) is A[c][r] exactly under either
    order: checks out[c*rows + r] (not its transpose) for both paths."""
    for (rows, n) in [(16, 3), (13, 3), (16, 1)]:
        k = 16
        w = h(np.eye(rows, k))
        a = synth.random_f16((rows, n), (n, k))
        out = orc.mat_mul(w, a)
        assert out.shape == (n, rows)
        want = a.view(F).astype(np.float32)[:, :rows]
        assert np.array_equal(out, want)


def test_mat_mul_dispatch_per_shape(orc):
    """Each element equals the order its full shape picks."""
    for rows, k, n in [(12, 1536, 2), (13, 1536, 2), (12, 1540, 3), (12, 8, 6), (13, 31, 4),
                       (12, 33, 5), (12, 1536, 1), (16, 64, 3)]:
        w = synth.random_f16((rows, k, 1), (rows, k), 0.02)
        a = synth.random_f16((rows, k, 2), (n, k))
        out = orc.mat_mul(w, a)
        f = orc.sgemm_dot if orc.takes_sgemm(rows, k, n) else orc.vec_dot
        want = np.array([[f(w[r], a[c]) for r in range(rows)] for c in range(n)], dtype=np.float32)
        assert np.array_equal(out.view(np.uint32), want.view(np.uint32))


def test_threads_do_not_change_bits(orc):
    w, a = synth.c1()
    a16 = orc.to_f16(a)
    ref = orc.mat_mul(w, a16, threads=1)
    for t in (2, 3, 7, 16):
        assert np.array_equal(orc.mat_mul(w, a16, threads=t).view(np.uint32), ref.view(np.uint32))
    mv = orc.mat_vec(w, a16[0], threads=5)
    assert np.array_equal(mv.view(np.uint32), orc.mat_mul(w, a16[:1], threads=1)[0].view(np.uint32))


def test_mat_mul_at_matches_full(orc):
    rows, k, n = 24, 200, 3
    w = synth.random_f16((9, 1), (rows, k), 0.02)
    a = synth.random_f16((9, 2), (n, k))
    full = orc.mat_mul(w, a)
    rr, cc = np.meshgrid(np.arange(rows), np.arange(n))
    got = orc.mat_mul_at(w, a, rr.ravel(), cc.ravel())
    assert np.array_equal(got, full.ravel())


def test_degenerate_sizes(orc):
    """k = 0 gives +0.0 under both orders; empty products are empty."""
    z = np.zeros(0, dtype=np.uint16)
    r = orc.vec_dot(z, z)
    assert r == 0.0 and not np.signbit(r)
    r = orc.sgemm_dot(z, z)
    assert r == 0.0 and not np.signbit(r)
    assert orc.mat_mul(np.zeros((0, 8), np.uint16), np.zeros((2, 8), np.uint16)).shape == (2, 0)
    assert orc.mat_mul(np.zeros((4, 8), np.uint16), np.zeros((0, 8), np.uint16)).shape == (0, 4)


def test_fp64_reference_close_to_exact(orc):
    w = synth.random_f16((3, 1), (8, 4096), 0.02)
    a = synth.random_f16((3, 2), (2, 4096))
    rr = np.repeat(np.arange(8), 2)
    cc = np.tile(np.arange(2), 8)
    ref, scale = orc.fp64_at(w, a, rr, cc)
    for i in range(rr.size):
        ex, sa = orc.exact_dot(w[rr[i]], a[cc[i]])
        assert abs(ref[i] - ex) <= 4096 * 2.0 ** -53 * sa
        assert scale[i] == pytest.approx(sa, rel=1e-12)
