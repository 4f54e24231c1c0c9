"""GPU parity: the HIP library through its C ABI against the oracle, element by
element, on the same seeded inputs.

Exact paths (to_f16, vec_dot, tinyBLAS) must be bit-identical to the oracle
(NaN compared as "is NaN").  The MFMA fast path must stay within
max |y - ref| / sum_i |w_i a_i| <= 2e-3 of the binary64 reference.
Every exact product is checked completely, the full-size ones included
(every n = 1 product of both decode steps, every n = 512 product of the
135M layer 0 and of the 8B set, the oracle running on the host's cores).  The
MFMA path is checked on samples: at least 16 elements in every 64 x 64 block
of the output (every tile of every launch shape is a union of such blocks),
against the 2e-3 gate, a bound derived from f32 accumulation, and the plain
relative error on elements that are not near zero.
"""
import concurrent.futures as cf
import os

import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import f16_weight_matrix_amd as f16wm  # noqa: E402
from mfma_gate import f32_accumulation_bound, mfma_check, tile_samples  # noqa: E402

DEV = torch.device("cuda:0")


def host_threads() -> int:
    """Oracle threads: the cores this process may run on, at most 16 (one
    GPU's share of a shared host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


HOST_T = host_threads()


def say(*a):
    print(*a, flush=True)


def up16(x: np.ndarray, offset: int = 0) -> torch.Tensor:
    """uint16 numpy -> float16 GPU tensor (optionally at an element offset
    inside a larger allocation, to test misaligned pointers)."""
    flat = torch.from_numpy(np.ascontiguousarray(x).view(np.int16).reshape(-1)).to(DEV)
    if offset:
        buf = torch.empty(flat.numel() + offset, dtype=torch.int16, device=DEV)
        buf[offset:] = flat
        flat = buf[offset:]
    return flat.view(torch.float16).view(x.shape)


def up32(x: np.ndarray, offset: int = 0) -> torch.Tensor:
    flat = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32).reshape(-1)).to(DEV)
    if offset:
        buf = torch.empty(flat.numel() + offset, dtype=torch.float32, device=DEV)
        buf[offset:] = flat
        flat = buf[offset:]
    return flat.view(x.shape)


def f32_column(seed, k):
    """N(0,1) f32 values with the rounding's edge cases mixed in."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(k).astype(np.float32)
    specials = np.array([np.inf, -np.inf, np.nan, 65520.0, 65519.99, 2 ** -25, 1e-7, -0.0, 7e4,
                         1 + 2 ** -11], dtype=np.float32)
    idx = rng.choice(k, size=min(k // 8, specials.size), replace=False)
    x[idx] = specials[:idx.size]
    return x


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint32)


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what: str):
    got = np.ascontiguousarray(got, dtype=np.float32)
    want = np.ascontiguousarray(want, dtype=np.float32)
    assert got.shape == want.shape, what
    gn, wn = np.isnan(got), np.isnan(want)
    same = (got.view(np.uint32) == want.view(np.uint32)) | (gn & wn)
    if not same.all():
        idx = np.argwhere(~same)
        i = tuple(idx[0])
        raise AssertionError("%s: %d of %d elements differ; first at %s: got %r (0x%08x) want %r (0x%08x)"
                             % (what, len(idx), got.size, i, float(got[i]), got.view(np.uint32)[i],
                                float(want[i]), want.view(np.uint32)[i]))


@pytest.fixture(scope="module")
def orc():
    import oracle
    return oracle.default()


# ------------------------------------------------------------------ to_f16

def test_to_f16_matches_oracle(orc):
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(100003).astype(np.float32),
        (rng.standard_normal(5000) * 1e-6).astype(np.float32),     # f16 subnormal range
        (rng.standard_normal(5000) * 7e4).astype(np.float32),      # overflow range
        np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 65504, 65519.99, 65520, 2 ** -25, -(2 ** -25),
                  2 ** -24, 1 + 2 ** -11], dtype=np.float32),
        np.array([0x7F800001, 0xFFC00001, 0x7FBFFFFF, 0x00000001], dtype=np.uint32).view(np.float32),
    ])
    want = orc.to_f16(x)
    for off in (0, 1, 3):           # 16-byte aligned, and not
        xs = up32(np.concatenate([np.zeros(off, np.float32), x]))[off:]
        got = f16wm.to_f16(xs)
        g = got.cpu().numpy().view(np.uint16)
        assert np.array_equal(g, want), "offset %d: %d differ" % (off, int((g != want).sum()))


def test_to_f16_exhaustive(orc):
    """All 2^32 binary32 bit patterns, bit-exact against the oracle."""
    chunk = 1 << 27
    nthreads = min(16, os.cpu_count() or 1)
    pool = cf.ThreadPoolExecutor(nthreads)
    bad = 0
    for c in range((1 << 32) // chunk):
        lo = c * chunk
        xg = torch.arange(lo, lo + chunk, dtype=torch.int64, device=DEV).to(torch.int32).view(torch.float32)
        got = f16wm.to_f16(xg).cpu().numpy().view(np.uint16)
        xh = np.arange(lo, lo + chunk, dtype=np.uint64).astype(np.uint32).view(np.float32)
        parts = np.array_split(np.arange(chunk), nthreads)
        want = np.empty(chunk, dtype=np.uint16)

        def run(ix):
            want[ix[0]:ix[-1] + 1] = orc.to_f16(xh[ix[0]:ix[-1] + 1])
        list(pool.map(run, parts))
        nb = int(np.count_nonzero(got != want))
        bad += nb
        if c % 8 == 0 or nb:
            say("to_f16 exhaustive chunk %d/32: %d mismatches" % (c, nb))
        del xg
    pool.shutdown()
    assert bad == 0


# ------------------------------------------------- widening of every f16

def test_every_f16_value_widens_exactly(orc):
    """Every one of the 2^16 f16 patterns goes through each kernel's widening:
    each activation column holds one pattern next to zeros and the weight
    rows are one-hot on it, so the product is widen(pattern) (exactly; NaN as
    NaN).  Bit-exact against the oracle, and equal to the oracle's widen on
    every non-NaN pattern."""
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    wid = orc.widen(pats)
    for rows, k, what in [(4, 8, "tinyBLAS"), (3, 32, "vec_dot fallback (n columns)"),
                          (4, 33, "vec_dot, double tail")]:
        w = np.zeros((rows, k), dtype=np.uint16)
        w[:, 0] = 0x3C00                                   # 1.0
        if k == 33:
            w[:, 0], w[:, 32] = 0, 0x3C00                   # the pattern sits in the tail
        a = np.zeros((pats.size, k), dtype=np.uint16)
        a[:, 32 if k == 33 else 0] = pats
        got = f16wm.mat_mul(up16(w), up16(a)).cpu().numpy()      # n = 65536 columns
        assert_bits_equal(got, orc.mat_mul(w, a), "widen via " + what)
        ok = ~np.isnan(wid) & (pats != 0x8000)             # -0 * 1 + (+0) = +0
        assert np.array_equal(got[ok, 0].view(np.uint32), wid[ok].view(np.uint32)), what
    # one column at a time through the GEMV kernel
    w = np.zeros((4, 64), dtype=np.uint16)
    w[np.arange(4), np.arange(4) * 9] = 0x3C00
    for c0 in range(0, 1 << 16, 64 * 97):
        col = pats[c0:c0 + 64].copy()
        got = f16wm.mat_vec(up16(w), up16(col)).cpu().numpy()
        assert_bits_equal(got, orc.mat_vec(w, col), "widen via vec_dot GEMV at %d" % c0)


def test_widen_entry_point_all_patterns(orc):
    """f16wm_widen on all 2^16 patterns (aligned and not), against the oracle."""
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    want = orc.widen(pats)
    for off in (0, 1, 5):
        got = f16wm.widen(up16(pats, off)).cpu().numpy()
        assert_bits_equal(got, want, "widen offset %d" % off)


@pytest.mark.parametrize("rows,k", [(49152, 576), (128256, 4096), (13, 31), (100, 1000)])
def test_get_rows(orc, rows, k):
    """Embedding lookup (get_rows / dequantize_row): selected rows widened
    exactly; first, last and repeated ids; an out-of-range id gives NaN."""
    w = synth.random_f16((81, rows, k), (rows, k), 0.02) if rows * k < 10 ** 8 else \
        synth.weight(synth.CFG_8B, 0, "logits", rows, k)
    rng = np.random.default_rng(82)
    ids = np.concatenate([[0, rows - 1, 0], rng.integers(0, rows, 509)]).astype(np.int64)
    got = f16wm.get_rows(up16(w), torch.from_numpy(ids).to(DEV)).cpu().numpy()
    assert_bits_equal(got, orc.widen(w[ids]), "get_rows %dx%d" % (rows, k))
    bad = torch.tensor([rows, -1, 2 if rows > 2 else 0], dtype=torch.int64, device=DEV)
    g2 = f16wm.get_rows(up16(w), bad).cpu().numpy()
    assert np.isnan(g2[:2]).all()
    assert_bits_equal(g2[2], orc.widen(w[int(bad[2])]), "get_rows valid id after bad ones")


# --------------------------------------------------------------- C1: 576

def test_576_parity_both_orders(orc):
    """576x576 weight, seed 0: n = 1 (vec_dot) and n = 3 (tinyBLAS), bit-exact,
    with the activation rounded on the GPU."""
    w, a = synth.c1()
    a16_want = orc.to_f16(a)
    wd = up16(w)
    a16 = f16wm.to_f16(up32(a))
    assert np.array_equal(a16.cpu().numpy().view(np.uint16), a16_want)
    mv = f16wm.mat_vec(wd, a16[0])
    assert_bits_equal(mv.cpu().numpy(), orc.mat_vec(w, a16_want[0]), "576 n=1")
    mm = f16wm.mat_mul(wd, a16)
    want3 = orc.mat_mul(w, a16_want)
    assert_bits_equal(mm.cpu().numpy(), want3, "576 n=3")
    # the two orders differ on the GPU exactly where they differ in the oracle
    per_col = torch.stack([f16wm.mat_vec(wd, a16[c]) for c in range(3)]).cpu().numpy()
    want_vd = np.stack([orc.mat_vec(w, a16_want[c]) for c in range(3)])
    assert_bits_equal(per_col, want_vd, "576 vec_dot per column")
    ndiff = int(np.count_nonzero(per_col.view(np.uint32) != mm.cpu().numpy().view(np.uint32)))
    say("576x576 n=3: %d of 1728 elements differ between the two orders" % ndiff)
    assert ndiff == int(np.count_nonzero(want_vd.view(np.uint32) != want3.view(np.uint32))) > 0


# ------------------------------------------------ both sides of takes_sgemm

def _sweep_case(orc, rows, k, n, seed, woff=0, aoff=0):
    w = synth.random_f16((seed, rows, k, 1), (rows, k), 0.02)
    a = synth.random_f16((seed, rows, k, 2), (n, k))
    got = f16wm.mat_mul(up16(w, woff), up16(a, aoff))
    return got, orc.mat_mul(w, a)


def test_tail_and_fallback_sweep(orc):
    """rows 12 and 13 (both sides of rows % 4), every k from 1 to 1,540
    (every k % 8 and k % 32), n = 1..6: every element bit-exact."""
    torch.cuda.synchronize()
    fails = []
    for rows in (12, 13):
        for k in range(1, 1541):
            for n in range(1, 7):
                got, want = _sweep_case(orc, rows, k, n, 11)
                g = got.cpu().numpy()
                if not np.array_equal(g.view(np.uint32), want.view(np.uint32)):
                    fails.append((rows, k, n))
        say("sweep rows=%d done, %d failing shapes so far" % (rows, len(fails)))
    assert not fails, fails[:20]


@pytest.mark.parametrize("rows,k,n", [(13, 1540, 2), (12, 1536, 2), (13, 1540, 6), (12, 1536, 6),
                                      (12, 8, 3), (13, 31, 4), (12, 33, 5), (576, 576, 3),
                                      (1000, 1000, 5), (100, 4096, 65), (260, 200, 130)])
@pytest.mark.parametrize("woff,aoff", [(0, 0), (1, 0), (0, 3), (4, 4)])
def test_shapes_and_alignment(orc, rows, k, n, woff, aoff):
    """Ragged tiles and misaligned (2-byte) pointers take other kernels; the
    bits stay the same."""
    got, want = _sweep_case(orc, rows, k, n, 12, woff, aoff)
    assert_bits_equal(got.cpu().numpy(), want, "mat_mul %dx%d n=%d offs=%d,%d" % (rows, k, n, woff, aoff))
    got1 = f16wm.mat_vec(up16(synth.random_f16((12, rows, k, 1), (rows, k), 0.02), woff),
                         up16(synth.random_f16((12, rows, k, 2), (n, k)), aoff)[0])
    assert_bits_equal(got1.cpu().numpy(), orc.mat_mul(synth.random_f16((12, rows, k, 1), (rows, k), 0.02),
                                                      synth.random_f16((12, rows, k, 2), (n, k))[:1])[0],
                      "mat_vec %dx%d" % (rows, k))


def test_gemv_past_the_32_bit_offset_limit(orc):
    """A row so long (k = 2^26 + 40: 134 MB per row) that 16 rows of it pass the
    2^31-byte offsets of the staged kernels: the launch falls back to the
    one-lane-per-chain kernel, through f16wm_mat_vec and through a table;
    every element against the oracle, the 8-element tail included."""
    k = (1 << 26) + 40
    w = synth.random_f16((86, 1), (3, k), 0.02)
    a = synth.random_f16((86, 2), (k,))
    want = orc.mat_vec(w, a, threads=HOST_T)
    wd, ad = up16(w), up16(a)
    assert_bits_equal(f16wm.mat_vec(wd, ad).cpu().numpy(), want, "mat_vec k=2^26+40")
    outs = f16wm.mat_vec_table([(wd, ad), (wd[:1], ad)])
    assert_bits_equal(outs[0].cpu().numpy(), want, "table k=2^26+40")
    assert_bits_equal(outs[1].cpu().numpy(), want[:1], "table k=2^26+40, one row")


def test_random_shapes_every_exact_kernel(orc):
    """120 seeded random products (rows 1-700, k 1-3000, n 1-300, f16 or f32
    activations, aligned or not): every kernel class of the exact orders on
    shapes nobody picked, every element against the oracle."""
    rng = np.random.default_rng(2024)
    for case in range(120):
        rows = int(rng.integers(1, 700))
        k = int(rng.choice([int(rng.integers(1, 3000)), 8 * int(rng.integers(1, 375))]))
        n = int(rng.choice([1, 2, 3, int(rng.integers(1, 300))]))
        if rng.random() < 0.5:
            rows = max(4, rows // 4 * 4)                 # takes_sgemm more often
        f32 = bool(rng.random() < 0.3)
        woff, aoff = (0, 0) if rng.random() < 0.7 else (int(rng.integers(0, 8)), int(rng.integers(0, 8)))
        w = synth.random_f16((87, case, 1), (rows, k), 0.02)
        if f32:
            x = rng.standard_normal((n, k)).astype(np.float32)
            a16 = orc.to_f16(x)
            got = f16wm.mat_mul(up16(w, woff), up32(x, aoff)).cpu().numpy()
        else:
            a16 = synth.random_f16((87, case, 2), (n, k))
            got = f16wm.mat_mul(up16(w, woff), up16(a16, aoff)).cpu().numpy()
        assert_bits_equal(got, orc.mat_mul(w, a16, threads=HOST_T),
                          "random case %d: rows=%d k=%d n=%d f32=%s offs=%d,%d" % (case, rows, k, n, f32, woff, aoff))
    say("120 random exact products bit-exact")


# ------------------------------------------------------------ grouped GEMV

@pytest.mark.parametrize("shapes", [
    [(576, 576), (192, 576), (192, 576)],
    [(1536, 576), (1536, 576)],
    [(4096, 4096), (1024, 4096), (1024, 4096)],
    [(1, 96), (63, 96), (64, 96), (65, 96), (7, 96), (200, 96), (3, 96), (129, 96)],
    [(5, 33), (7, 33)],
    [(4097, 1000), (33, 1000), (100, 1000)],
    [(17, 576), (40, 576), (3, 576)],
    [(5000, 4104)],
])
def test_mat_vec_multi(orc, shapes):
    """Grouped GEMVs, including row tiles that straddle two matrices and
    k % 32 tails for the 16-lane kernel (4096 rows or more), and ragged
    groups for the short-row kernel (k <= 576)."""
    k = shapes[0][1]
    ws = [synth.random_f16((21, i, r, k), (r, k), 0.02) for i, (r, _) in enumerate(shapes)]
    a = synth.random_f16((22, k), (k,))
    outs = f16wm.mat_vec_multi([up16(w) for w in ws], up16(a))
    for i, (w, o) in enumerate(zip(ws, outs)):
        assert_bits_equal(o.cpu().numpy(), orc.mat_vec(w, a), "multi matrix %d %s" % (i, shapes[i]))


# ------------------------------------------- f32 activations, rounded inside

@pytest.mark.parametrize("rows,k,off", [(576, 576, 0), (13, 1540, 0), (1000, 4104, 0), (100, 96, 1),
                                        (64, 33, 3), (4096, 14336, 0), (70000, 64, 0), (5, 8, 2),
                                        (4099, 1000, 0), (6001, 16376, 0)])
def test_f32_activation_equals_to_f16_then_product(orc, rows, k, off):
    """mat_vec with an f32 column equals to_f16 then mat_vec, bit for bit
    (edge values of the rounding included; aligned and misaligned columns)."""
    w = synth.random_f16((71, rows, k), (rows, k), 0.02)
    x = f32_column((72, rows, k), k)
    want = orc.mat_vec(w, orc.to_f16(x))
    got = f16wm.mat_vec(up16(w), up32(x, off))
    assert_bits_equal(got.cpu().numpy(), want, "mat_vec f32 %dx%d off=%d" % (rows, k, off))


@pytest.mark.parametrize("shapes", [
    [(4096, 4096), (1024, 4096), (1024, 4096)],
    [(14336, 4096), (14336, 4096)],
    [(3, 40), (64, 40), (65, 40)],
])
def test_f32_activation_multi(orc, shapes):
    k = shapes[0][1]
    ws = [synth.random_f16((73, i, r, k), (r, k), 0.02) for i, (r, _) in enumerate(shapes)]
    x = f32_column((74, k), k)
    x16 = orc.to_f16(x)
    outs = f16wm.mat_vec_multi([up16(w) for w in ws], up32(x))
    for i, (w, o) in enumerate(zip(ws, outs)):
        assert_bits_equal(o.cpu().numpy(), orc.mat_vec(w, x16), "multi f32 matrix %d" % i)


# Exact tinyBLAS-order kernels by launch size: a launch of at most 1024
# 32 x 32 output tiles runs one tile per block (tinyblas_lanes); a larger one
# runs 64 x 64 blocks (tinyblas_mfma) with buffer loads when the operands are
# 16-byte aligned and guarded loads otherwise.  k % 64 != 0 leaves a partial
# last stage, whose chunks past k read zero.
@pytest.mark.parametrize("rows,k,n,off", [
    (576, 576, 512, 0),     # 288 tiles: tinyblas_lanes
    (2048, 1024, 512, 0),   # exactly 1024 tiles: still tinyblas_lanes
    (2080, 1024, 512, 0),   # 1040 tiles: 64 x 64 blocks, f32 block through buffer loads
    (2080, 1000, 512, 0),   # 1040 tiles, k % 64 = 40: a partial last stage
    (2080, 1000, 500, 0),   # ragged last column block too
    (2080, 1000, 512, 1),   # misaligned f32 block: guarded loads
    (576, 1536, 7, 1),      # misaligned f32 block, few tiles: guarded loads
    (12, 1536, 5, 0),       # one ragged tile
    (13, 1540, 3, 0),       # vec_dot order (rows % 4 != 0), k tail
    (12, 33, 4, 1),         # vec_dot order (k % 8 != 0), misaligned
])
def test_f32_activation_products(orc, rows, k, n, off):
    """mat_mul with an f32 block equals the oracle (to_f16, then the shape's
    order) on every element, and equals to_f16 then mat_mul on the GPU bit
    for bit (NaN payloads included), in every kernel class.  Each column
    carries the rounding's edge values."""
    w = synth.random_f16((75, rows, k), (rows, k), 0.02)
    x = np.stack([f32_column((76, rows, k, c), k) for c in range(n)])
    W, X = up16(w), up32(x, off)
    got = f16wm.mat_mul(W, X)
    ref = f16wm.mat_mul(W, f16wm.to_f16(X))
    assert np.array_equal(bits(got), bits(ref)), "f32 block vs to_f16 then mat_mul"
    want = orc.mat_mul(w, orc.to_f16(x), threads=HOST_T)
    assert_bits_equal(got.cpu().numpy(), want, "mat_mul f32 %dx%d n=%d off=%d" % (rows, k, n, off))


@pytest.mark.parametrize("rows,k,n,woff,aoff", [
    (2048, 1024, 512, 0, 0), (2080, 1024, 512, 0, 0), (2080, 1000, 512, 0, 0), (2080, 1000, 500, 0, 0),
    (2080, 1000, 512, 1, 0), (2080, 1000, 512, 0, 3), (14336, 4096, 96, 0, 0)])
def test_many_tile_exact_products(orc, rows, k, n, woff, aoff):
    """f16 activation blocks on both sides of the 1024-tile switch, with a
    partial last k stage, ragged column blocks, and misaligned operands
    (guarded loads), every element against the oracle."""
    w = synth.random_f16((79, rows, k), (rows, k), 0.02)
    a = synth.random_f16((80, n, k), (n, k))
    got = f16wm.mat_mul(up16(w, woff), up16(a, aoff)).cpu().numpy()
    assert_bits_equal(got, orc.mat_mul(w, a, threads=HOST_T), "mat_mul %dx%d n=%d offs=%d,%d"
                      % (rows, k, n, woff, aoff))


@pytest.mark.parametrize("shapes,n", [
    ([(576, 576), (192, 576), (192, 576)], 512),
    ([(4096, 512), (1024, 512)], 512),                # 2560 tiles: 64 x 64 blocks, f32 block
    ([(4096, 1000), (1024, 1000), (1024, 1000)], 512),  # partial last stage in a grouped launch
    ([(12, 100), (13, 100), (16, 100)], 5),
])
def test_f32_activation_grouped_products(orc, shapes, n):
    """Grouped exact products with an f32 block: every element against the
    oracle, and bit-equal to to_f16 then the f16 grouped product."""
    k = shapes[0][1]
    ws = [synth.random_f16((77, i, r, k), (r, k), 0.02) for i, (r, _) in enumerate(shapes)]
    x = np.stack([f32_column((78, c, k), k) for c in range(n)])
    x16 = orc.to_f16(x)
    Ws, X = [up16(w) for w in ws], up32(x)
    got = f16wm.mat_mul_multi(Ws, X)
    ref = f16wm.mat_mul_multi(Ws, f16wm.to_f16(X))
    for i in range(len(ws)):
        assert np.array_equal(bits(got[i]), bits(ref[i])), "matrix %d" % i
        assert_bits_equal(got[i].cpu().numpy(), orc.mat_mul(ws[i], x16, threads=HOST_T),
                          "grouped f32 matrix %d %s n=%d" % (i, shapes[i], n))


# ------------------------------------------------------ grouped products

@pytest.mark.parametrize("shapes,n", [
    ([(576, 576), (192, 576), (192, 576)], 512),      # 135M Q/K/V, one prefill micro-batch
    ([(1536, 576), (1536, 576)], 512),                # 135M gate/up
    ([(12, 100), (13, 100), (16, 100)], 5),           # mixed orders: 13 rows falls back to vec_dot
    ([(4, 40), (100, 40)], 1),                        # one column: vec_dot
    ([(1000, 64), (0, 64), (24, 64)], 70),            # an empty matrix in the group
])
def test_grouped_exact_products(orc, shapes, n):
    k = shapes[0][1]
    ws = [synth.random_f16((91, i, r, k), (r, k), 0.02) for i, (r, _) in enumerate(shapes)]
    a = synth.random_f16((92, k, n), (n, k))
    outs = f16wm.mat_mul_multi([up16(w) for w in ws], up16(a))
    for i, (w, o) in enumerate(zip(ws, outs)):
        assert_bits_equal(o.cpu().numpy(), orc.mat_mul(w, a), "grouped exact matrix %d %s n=%d" % (i, shapes[i], n))


@pytest.mark.parametrize("shapes,n", [
    ([(4096, 4096), (1024, 4096), (1024, 4096)], 512),
    ([(576, 576), (192, 576), (192, 576)], 512),
    ([(200, 40), (13, 40)], 77),
])
def test_grouped_mfma_products(orc, shapes, n):
    k = shapes[0][1]
    ws = [synth.random_f16((93, i, r, k), (r, k), 0.02) for i, (r, _) in enumerate(shapes)]
    a = synth.random_f16((94, k, n), (n, k))
    outs = f16wm.mat_mul_mfma_multi([up16(w) for w in ws], up16(a))
    for i, (w, o) in enumerate(zip(ws, outs)):
        rr, cc = tile_samples(w.shape[0], n, 3 + i)
        mfma_check(orc, w, a, o.cpu().numpy(), rr, cc, "grouped mfma matrix %d %s" % (i, shapes[i]))


# ---------------------------------------------------------- edge cases

def test_degenerate_sizes(orc):
    w = torch.empty((8, 0), dtype=torch.float16, device=DEV)
    a = torch.empty((3, 0), dtype=torch.float16, device=DEV)
    out = torch.full((3, 8), 7.0, device=DEV)
    f16wm.mat_mul(w, a, out)                                   # k = 0: +0.0 everywhere
    assert (bits(out) == 0).all()
    out1 = torch.full((8,), 7.0, device=DEV)
    f16wm.mat_vec(w, a[0], out1)
    assert (bits(out1) == 0).all()
    outm = torch.full((3, 8), 7.0, device=DEV)
    f16wm.mat_mul_mfma(w, a, outm)
    assert (bits(outm) == 0).all()
    # rows = 0 / n = 0: no-ops
    f16wm.mat_mul(torch.empty((0, 16), dtype=torch.float16, device=DEV),
                  torch.zeros((2, 16), dtype=torch.float16, device=DEV))
    f16wm.mat_mul(torch.zeros((4, 16), dtype=torch.float16, device=DEV),
                  torch.empty((0, 16), dtype=torch.float16, device=DEV))
    f16wm.to_f16(torch.empty(0, device=DEV))
    # the same through the f32-block entry points (tinyBLAS order for 8 rows,
    # vec_dot order for 13)
    x = torch.empty((3, 0), dtype=torch.float32, device=DEV)
    for r in (8, 13):
        outf = torch.full((3, r), 7.0, device=DEV)
        f16wm.mat_mul(torch.empty((r, 0), dtype=torch.float16, device=DEV), x, outf)
        assert (bits(outf) == 0).all(), r
    f16wm.mat_mul(torch.empty((0, 16), dtype=torch.float16, device=DEV),
                  torch.zeros((2, 16), dtype=torch.float32, device=DEV))
    f16wm.mat_mul(torch.zeros((4, 16), dtype=torch.float16, device=DEV),
                  torch.empty((0, 16), dtype=torch.float32, device=DEV))


def test_inf_and_nan_propagate_like_the_oracle(orc):
    rows, k, n = 16, 100, 3
    w = synth.random_f16(31, (rows, k), 0.02)
    a = synth.random_f16(32, (n, k))
    w[2, 5] = 0x7C00      # +inf
    w[3, 40] = 0xFC00     # -inf
    w[4, 99] = 0x7E00     # NaN (in the double tail of vec_dot)
    a[1, 7] = 0x7C00
    for nn in (1, 2, 3):
        got = f16wm.mat_mul(up16(w), up16(a[:nn]))
        assert_bits_equal(got.cpu().numpy(), orc.mat_mul(w, a[:nn]), "inf/nan n=%d" % nn)
    w2 = synth.random_f16(33, (16, 96), 0.02)
    w2[1, 3] = 0x7C00
    w2[1, 4] = 0xFC00      # inf - inf = NaN inside a chain
    got = f16wm.mat_mul(up16(w2), up16(a[:, :96]))
    assert_bits_equal(got.cpu().numpy(), orc.mat_mul(w2, a[:, :96]), "inf-inf")


def test_large_magnitudes_and_cancellation(orc):
    """Values near the f16 range limits and heavy cancellation (products up to
    2^32) exercise every rounding in the trees."""
    rng = np.random.default_rng(44)
    for k in (64, 96, 1024, 1027):
        mag = np.exp2(rng.integers(-24, 16, size=(24, k))).astype(np.float32)
        sgn = rng.choice([-1.0, 1.0], size=(24, k)).astype(np.float32)
        w = (mag * sgn).astype(np.float16).view(np.uint16)
        a = (np.exp2(rng.integers(-24, 16, size=(4, k))) * rng.choice([-1.0, 1.0], size=(4, k))).astype(
            np.float16).view(np.uint16)
        for nn in (1, 4):
            got = f16wm.mat_mul(up16(w), up16(a[:nn]))
            assert_bits_equal(got.cpu().numpy(), orc.mat_mul(w, a[:nn]), "magnitudes k=%d n=%d" % (k, nn))


@pytest.mark.parametrize("rows,k,n", [(136, 264, 133), (1064, 264, 1000)])
def test_tinyblas_order_special_values(orc, rows, k, n):
    """The tinyBLAS order (computed one chain step per fp32 MFMA) on rows and
    columns made of signed zeros, subnormals, the f16 extremes, infinities
    and NaNs, over several output tiles with ragged edges; also an unaligned
    activation pointer (the guarded-load kernel).  136 x 133 (25 32 x 32
    tiles) runs one tile per block; 1064 x 1000 (1088 tiles) runs the 64 x 64
    blocks, with ragged last row and column blocks."""
    rng = np.random.default_rng(45)
    w = synth.random_f16(61, (rows, k), 0.02)
    a = synth.random_f16(62, (n, k))
    w[0, :] = 0x8000                                    # -0 row
    w[1, :] = rng.integers(1, 0x400, k)                 # positive subnormals
    w[2, :] = rng.integers(0x8001, 0x8400, k)           # negative subnormals
    w[3, ::2], w[3, 1::2] = 0x7BFF, 0xFBFF              # +-65504: cancellation at 2^32 scale
    w[70, 9] = 0x7C00                                   # +inf in the second row tile
    w[71, 17] = 0x7E00                                  # NaN
    w[72, 3], w[72, 11] = 0x7C00, 0xFC00                # inf and -inf in one row: NaN
    w[rows - 1, k - 1] = 0xFC00                         # -inf in the last row, last step
    a[0, :] = 0x8000                                    # -0 column
    a[1, :] = rng.integers(1, 0x400, k)                 # subnormal column
    a[2, 5] = 0x7C00                                    # inf meets finite and zero weights
    a[n - 3, ::3] = 0x7BFF                              # a column in the ragged last tile
    assert f16wm.takes_sgemm(rows, k, n)
    want = orc.mat_mul(w, a, threads=HOST_T)
    got = f16wm.mat_mul(up16(w), up16(a))
    assert_bits_equal(got.cpu().numpy(), want, "tinyBLAS specials")
    got = f16wm.mat_mul(up16(w), up16(a, offset=1))
    assert_bits_equal(got.cpu().numpy(), want, "tinyBLAS specials, unaligned activation")


def _f16(v) -> int:
    """The f16 bit pattern of a value that f16 holds exactly."""
    h = np.array([v], dtype=np.float16)
    assert float(h[0]) == v or (np.isnan(v) and np.isnan(h[0]))
    return int(h.view(np.uint16)[0])


# One chain step of the tinyBLAS order is acc = fma(w, a, acc): with f16
# operands the product is exact in binary32, so the step is the binary32 sum
# acc + w*a rounded to nearest, ties to even.  The exact GEMM kernels compute
# it as one rank-1 update of v_mfma_f32_32x32x1_2b_f32.  Each case below is
# (chain lane, [(step, w, a), ...], expected element) for a k = 64 row and
# column (eight steps per chain lane, every other element zero), so the
# element's other seven lanes are +0 and the hsum adds only exact zeros.
_STEP_CASES = [
    # name, lane, steps, expected f32 value
    ("tie to even (down)", 0, [(0, 1.0, 1.0), (1, 2.0 ** -12, 2.0 ** -12)], 1.0),
    ("tie to even (up)", 3, [(0, 1.0, 1.0), (1, 2.0 ** -12, 2.0 ** -11), (2, 2.0 ** -12, 2.0 ** -12)],
     1.0 + 2.0 ** -22),
    ("above the tie", 5, [(0, 1.0, 1.0), (1, 2.0 ** -12 * (1 + 2.0 ** -6), 2.0 ** -12)], 1.0 + 2.0 ** -23),
    ("below the tie", 7, [(0, 1.0, 1.0), (1, 2.0 ** -12 * (1 - 2.0 ** -11), 2.0 ** -12)], 1.0),
    ("negative tie to even", 4, [(0, 1.0, 1.0), (3, -(2.0 ** -12), 2.0 ** -13)], 1.0),
    ("exact cancellation gives +0", 1, [(0, 1.0, 1.0), (5, -1.0, 1.0)], 0.0),
    ("cancellation at 2^32", 6, [(0, 65504.0, 65504.0), (1, -65504.0, 65504.0), (7, 1.0, 1.0)], 1.0),
    ("absorbed below half an ulp", 2, [(0, 65504.0, 65504.0), (1, 2.0 ** -14, 2.0 ** -14)],
     65504.0 * 65504.0),
    ("+inf then finite", 0, [(0, np.inf, 1.0), (4, -3.0, 2.0)], np.inf),
    ("+inf plus -inf", 5, [(2, np.inf, 1.0), (6, -np.inf, 1.0)], np.nan),
    ("NaN operand", 3, [(1, np.nan, 1.0), (2, 1.0, 1.0)], np.nan),
]


def _step_case_operands(k=64):
    rows = []
    for name, lane, steps, want in _STEP_CASES:
        wv = np.zeros(k, np.uint16)
        av = np.zeros(k, np.uint16)
        for t, x, y in steps:
            wv[8 * t + lane] = _f16(x)
            av[8 * t + lane] = _f16(y)
        rows.append((name, wv, av, want))
    # -0 products onto +0 accumulators in all eight lanes: every step adds
    # -0 to +0, which is +0, so the element is +0 (a -0 in all eight lanes
    # would survive the hsum)
    rows.append(("-0 products onto +0", np.full(k, 0x8000, np.uint16), np.full(k, _f16(1.5), np.uint16), 0.0))
    return rows


@pytest.mark.parametrize("rows,n,f32act,aoff", [(64, 40, False, 0), (1064, 1000, False, 0),
                                                (1064, 1000, True, 0), (1064, 1000, False, 1)])
def test_fp32_mfma_chain_step_rounding(orc, rows, n, f32act, aoff):
    """The rounding of one chain step on the fp32 matrix cores: ties to even
    in both directions, just above and below a tie, a negative tie, exact
    cancellation to +0, -0 products onto +0 accumulators, absorption at
    2^32, infinities and NaN.  Each case sits at a (row, column) pair spread
    over the output tiles (the first, the middle and the ragged last ones)
    in a background of random values; its element must equal the value the
    IEEE definition gives (worked out above, independent of the oracle) and
    the whole product must equal the oracle bit for bit.  64 x 40 runs one
    tile per block, 1064 x 1000 the 64 x 64 blocks (f16 or f32 activation
    block, aligned or guarded loads)."""
    k = 64
    w = synth.random_f16((95, rows, k), (rows, k), 0.02)
    a = synth.random_f16((96, n, k), (n, k))
    cases = _step_case_operands(k)
    pos_r = np.linspace(0, rows - 1, len(cases)).astype(np.int64)
    pos_c = np.linspace(n - 1, 0, len(cases)).astype(np.int64)
    for (name, wv, av, _), r, c in zip(cases, pos_r, pos_c):
        w[r] = wv
        a[c] = av
    if f32act:
        got = f16wm.mat_mul(up16(w), up32(orc.widen(a), aoff)).cpu().numpy()
    else:
        got = f16wm.mat_mul(up16(w), up16(a, aoff)).cpu().numpy()
    for (name, _, _, want), r, c in zip(cases, pos_r, pos_c):
        g = got[c, r]
        if np.isnan(want):
            assert np.isnan(g), (name, g)
        else:
            assert np.float32(g).view(np.uint32) == np.float32(want).view(np.uint32), \
                "%s at (%d, %d): got %r, IEEE gives %r" % (name, r, c, float(g), want)
    assert_bits_equal(got, orc.mat_mul(w, a, threads=HOST_T), "chain-step cases %dx%d n=%d" % (rows, k, n))


def test_repeatable_bits():
    w = up16(synth.random_f16(51, (1000, 4096), 0.02))
    a = up16(synth.random_f16(52, (7, 4096)))
    r1 = bits(f16wm.mat_mul(w, a))
    r2 = bits(f16wm.mat_mul(w, a))
    assert np.array_equal(r1, r2)
    v1 = bits(f16wm.mat_vec(w, a[0]))
    assert np.array_equal(v1, bits(f16wm.mat_vec(w, a[0])))


def test_mfma_bits_do_not_depend_on_the_launch():
    """Every fp16 MFMA kernel adds an element's 16-deep k slices in the same
    order, so the tile shape a launch picks (256 x 256 for the grouped gate
    and up, 128 x 128 with two or four LDS buffers, 128 x 64, a ragged last
    tile) changes no bit, and a repeated launch gives the same bits."""
    k, n = 512, 512
    g = up16(synth.random_f16((61, 14336, k), (14336, k), 0.02))
    u = up16(synth.random_f16((62, 14336, k), (14336, k), 0.02))
    a = up16(synth.random_f16((63, n, k), (n, k)))
    grouped = f16wm.mat_mul_mfma_multi([g, u], a)
    gb = bits(grouped[0])
    assert np.array_equal(bits(f16wm.mat_mul_mfma_multi([g, u], a)[0]), gb), "repeated grouped launch"
    assert np.array_equal(bits(f16wm.mat_mul_mfma(g, a)), gb), "gate alone"
    assert np.array_equal(bits(f16wm.mat_mul_mfma(u, a)), bits(grouped[1])), "up alone"
    for rows in (6144, 4100, 4096):
        got = bits(f16wm.mat_mul_mfma(g[:rows].contiguous(), a))
        assert np.array_equal(got, gb[:, :rows]), "first %d rows alone" % rows


def test_binding_reports_library_errors():
    w = torch.zeros((4, 12), dtype=torch.float16, device=DEV)
    a = torch.zeros((3, 12), dtype=torch.float16, device=DEV)
    with pytest.raises(f16wm.F16WMError) as e:
        f16wm.mat_mul_mfma(w, a)
    assert e.value.code == f16wm.F16WM_EUNSUPPORTED


# ------------------------------------------------------------ MFMA path

@pytest.mark.parametrize("rows,k,n", [(128, 32, 128), (200, 40, 130), (576, 576, 512), (1, 8, 1),
                                      (1000, 4104, 77), (49152, 576, 16), (4100, 1000, 300)])
def test_mfma_small_shapes(orc, rows, k, n):
    w = synth.random_f16((61, rows, k), (rows, k), 0.02)
    a = synth.random_f16((62, rows, k), (n, k))
    got = f16wm.mat_mul_mfma(up16(w), up16(a)).cpu().numpy()
    rr, cc = tile_samples(rows, n, 1)
    e, rel = mfma_check(orc, w, a, got, rr, cc, "mfma %dx%d n=%d" % (rows, k, n))
    say("mfma %dx%d n=%d: %d samples, max err/sum|wa| = %.3g (bound %.3g), max rel = %.3g"
        % (rows, k, n, rr.size, e, f32_accumulation_bound(k), rel))


def test_random_shapes_mfma(orc):
    """40 seeded random MFMA products (rows 1-3000, k a multiple of 8 up to
    5000 -- k % 64 != 0 takes the generic kernel --, n 1-600), each sampled in
    every 64 x 64 output block against the acceptance check."""
    rng = np.random.default_rng(2025)
    for case in range(40):
        rows = int(rng.integers(1, 3000))
        k = 8 * int(rng.integers(1, 625))
        n = int(rng.integers(1, 600))
        w = synth.random_f16((88, case, 1), (rows, k), 0.02)
        a = synth.random_f16((88, case, 2), (n, k))
        got = f16wm.mat_mul_mfma(up16(w), up16(a)).cpu().numpy()
        rr, cc = tile_samples(rows, n, 100 + case, per=4)
        mfma_check(orc, w, a, got, rr, cc, "random mfma case %d: rows=%d k=%d n=%d" % (case, rows, k, n))
    say("40 random MFMA products within the bounds")


# ----------------------------------------------- full-size model shapes

def test_smollm2_135m_decode_step_all_matrices(orc):
    """Every product of a 135M-shaped decode step (30 distinct layers + the tied
    49152x576 logits), launched as the decode step launches them, bit-exact."""
    S = synth.SMOLLM2_135M
    for layer in range(synth.SMOLLM2_135M_LAYERS):
        ws = {m: synth.weight(synth.CFG_135M, layer, m, *S[m]) for m in S}
        acts = synth.activation(synth.CFG_135M, layer, 0, 4, 1536)
        a_attn = orc.to_f16(acts[0, :576])
        a_o = orc.to_f16(acts[1, :576])
        a_ffn = orc.to_f16(acts[2, :576])
        a_down = orc.to_f16(acts[3, :1536])
        g = {m: up16(ws[m]) for m in ws}
        q, kk, v = f16wm.mat_vec_multi([g["q"], g["k"], g["v"]], up16(a_attn))
        o = f16wm.mat_vec(g["o"], up16(a_o))
        gate, upp = f16wm.mat_vec_multi([g["gate"], g["up"]], up16(a_ffn))
        down = f16wm.mat_vec(g["down"], up16(a_down))
        for name, got, w, x in [("q", q, ws["q"], a_attn), ("k", kk, ws["k"], a_attn), ("v", v, ws["v"], a_attn),
                                ("o", o, ws["o"], a_o), ("gate", gate, ws["gate"], a_ffn),
                                ("up", upp, ws["up"], a_ffn), ("down", down, ws["down"], a_down)]:
            assert_bits_equal(got.cpu().numpy(), orc.mat_vec(w, x), "135M layer %d %s" % (layer, name))
        if layer % 10 == 0:
            say("135M decode layer %d ok" % layer)
    wl = synth.weight(synth.CFG_135M, 0, "logits", *synth.SMOLLM2_135M_LOGITS)
    al = orc.to_f16(synth.activation(synth.CFG_135M, 30, 0, 1, 576)[0])
    got = f16wm.mat_vec(up16(wl), up16(al))
    assert_bits_equal(got.cpu().numpy(), orc.mat_vec(wl, al), "135M logits")


def test_smollm2_135m_prefill_512(orc):
    """n = 512 micro-batch on the 135M matrices (tinyBLAS order): layer 0 and
    the tied 49152x576 logits, every element bit-exact; the MFMA product
    sampled in every 64 x 64 output block."""
    S = dict(synth.SMOLLM2_135M)
    S["logits"] = synth.SMOLLM2_135M_LOGITS
    acts = synth.activation(synth.CFG_135M_PREFILL, 0, 0, synth.PREFILL_N, 1536)
    for i, (m, (rows, k)) in enumerate(S.items()):
        w = synth.weight(synth.CFG_135M, 0, m, rows, k)
        a16 = orc.to_f16(acts[:, :k])
        got = f16wm.mat_mul(up16(w), up16(a16)).cpu().numpy()
        assert_bits_equal(got, orc.mat_mul(w, a16, threads=HOST_T), "135M prefill layer 0 %s" % m)
        gm = f16wm.mat_mul_mfma(up16(w), up16(a16)).cpu().numpy()
        rr, cc = tile_samples(rows, synth.PREFILL_N, 30 + i)
        e, rel = mfma_check(orc, w, a16, gm, rr, cc, "135M prefill mfma %s" % m)
        say("135M prefill %s: exact ok (%d elements); mfma err %.3g rel %.3g over %d samples"
            % (m, got.size, e, rel, rr.size))


def test_llama3_8b_decode_gemv_all_matrices(orc):
    """The 8B-shaped GEMV set at full size, launched as the benchmark launches
    it (Q/K/V and gate/up grouped), every element bit-exact."""
    S = synth.LLAMA3_8B
    ws = {m: synth.weight(synth.CFG_8B, 0, m, *S[m]) for m in S}
    ws["logits"] = synth.weight(synth.CFG_8B, 0, "logits", *synth.LLAMA3_8B_LOGITS)
    acts = synth.activation(synth.CFG_8B, 0, 0, 5, 14336)
    x = {"attn": orc.to_f16(acts[0, :4096]), "o": orc.to_f16(acts[1, :4096]),
         "ffn": orc.to_f16(acts[2, :4096]), "down": orc.to_f16(acts[3, :14336]),
         "logits": orc.to_f16(acts[4, :4096])}
    g = {m: up16(w) for m, w in ws.items()}
    q, kk, v = f16wm.mat_vec_multi([g["q"], g["k"], g["v"]], up16(x["attn"]))
    gate, upp = f16wm.mat_vec_multi([g["gate"], g["up"]], up16(x["ffn"]))
    res = {"q": (q, "attn"), "k": (kk, "attn"), "v": (v, "attn"), "gate": (gate, "ffn"), "up": (upp, "ffn"),
           "o": (f16wm.mat_vec(g["o"], up16(x["o"])), "o"),
           "down": (f16wm.mat_vec(g["down"], up16(x["down"])), "down"),
           "logits": (f16wm.mat_vec(g["logits"], up16(x["logits"])), "logits")}
    for m, (got, src) in res.items():
        assert_bits_equal(got.cpu().numpy(), orc.mat_vec(ws[m], x[src]), "8B gemv %s" % m)
        say("8B gemv %s ok" % m)


_8B_ALL = dict(synth.LLAMA3_8B, logits=synth.LLAMA3_8B_LOGITS)


@pytest.mark.parametrize("m", list(_8B_ALL))
def test_llama3_8b_prefill_512(orc, m):
    """n = 512 on each 8B matrix: the exact order on EVERY element against the
    oracle (all 7.6e11 flops of the set, the oracle on the host's cores), and
    the MFMA product sampled in every 64 x 64 output block."""
    rows, k = _8B_ALL[m]
    i = list(_8B_ALL).index(m)
    acts = synth.activation(synth.CFG_8B_PREFILL, 0, 0, synth.PREFILL_N, 14336)
    w = synth.weight(synth.CFG_8B, 0, m, rows, k)
    a16 = orc.to_f16(acts[:, :k])
    del acts
    wd, ad = up16(w), up16(a16)
    got = f16wm.mat_mul(wd, ad).cpu().numpy()
    gm = f16wm.mat_mul_mfma(wd, ad).cpu().numpy()
    del wd, ad
    say("8B prefill %s: %dx%d n=512 on the GPU; oracle on %d threads" % (m, rows, k, HOST_T))
    assert_bits_equal(got, orc.mat_mul(w, a16, threads=HOST_T), "8B prefill %s" % m)
    rr, cc = tile_samples(rows, synth.PREFILL_N, 10 + i)
    e, rel = mfma_check(orc, w, a16, gm, rr, cc, "8B prefill mfma %s" % m)
    say("8B prefill %s: exact ok (%d elements); mfma err %.3g (bound %.3g) rel %.3g over %d samples"
        % (m, got.size, e, f32_accumulation_bound(k), rel, rr.size))


@pytest.mark.parametrize("group", [("q", "k", "v"), ("gate", "up")])
def test_llama3_8b_grouped_prefill_as_bench(orc, group):
    """The grouped n = 512 launches the benchmark times (Q/K/V in one launch,
    gate/up in one launch, sharing one rounded activation block), exact
    order on every element against the oracle, and the MFMA product sampled
    in every 64 x 64 output block."""
    S = synth.LLAMA3_8B
    k = S[group[0]][1]
    acts = synth.activation(synth.CFG_8B_PREFILL, 0, 0, synth.PREFILL_N, 14336)
    x = np.ascontiguousarray(acts[:, :k])
    del acts
    a16 = orc.to_f16(x)
    ws = {m: synth.weight(synth.CFG_8B, 0, m, *S[m]) for m in group}
    wd = [up16(ws[m]) for m in group]
    ad = f16wm.to_f16(up32(x))                       # rounded on the GPU, as the bench does
    assert np.array_equal(ad.view(torch.int16).cpu().numpy().view(np.uint16), a16)
    exact = [o.cpu().numpy() for o in f16wm.mat_mul_multi(wd, ad)]
    mfma = [o.cpu().numpy() for o in f16wm.mat_mul_mfma_multi(wd, ad)]
    del wd, ad
    for i, m in enumerate(group):
        assert_bits_equal(exact[i], orc.mat_mul(ws[m], a16, threads=HOST_T), "8B grouped prefill %s" % m)
        rr, cc = tile_samples(S[m][0], synth.PREFILL_N, 40 + i)
        e, rel = mfma_check(orc, ws[m], a16, mfma[i], rr, cc, "8B grouped mfma %s" % m)
        say("8B grouped %s: exact ok; mfma err %.3g rel %.3g" % (m, e, rel))


# ------------------------------------------- decode sequences as HIP graphs

def _replay_and_check(graph, outs, wants, what, eager=None, replays=3):
    """Replays `graph` several times, with the outputs poisoned before each
    replay and eager library work (and a synchronisation) between replays;
    every output of every replay must equal the oracle bit for bit."""
    for rep in range(replays):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, wnt) in enumerate(zip(outs, wants)):
            assert_bits_equal(o.cpu().numpy(), wnt, "%s replay %d output %d" % (what, rep, i))
        if eager is not None:
            eager()
            torch.cuda.synchronize()
    say("%s: %d replays bit-exact (%d outputs each)" % (what, replays, len(outs)))


def test_smollm2_135m_decode_step_as_graph(orc):
    """The 135M-shaped decode step as the benchmark runs it: 30 layers x
    {Q/K/V grouped, O, gate/up grouped, down} + the tied 49152x576 logits,
    121 launches taking f32 columns (rounded inside each launch), captured
    once as a HIP graph and replayed; every one of the 211 outputs against
    the oracle on every replay."""
    S = synth.SMOLLM2_135M
    L = synth.SMOLLM2_135M_LAYERS
    groups = [("qkv", ["q", "k", "v"], 576), ("o", ["o"], 576), ("gateup", ["gate", "up"], 576),
              ("down", ["down"], 1536)]
    W, X, O, want = {}, {}, {}, {}
    for l in range(L):
        acts = synth.activation(synth.CFG_135M, l, 0, 4, 1536)
        for gi, (g, mats, k) in enumerate(groups):
            x = np.ascontiguousarray(acts[gi, :k])
            X[(l, g)] = up32(x)
            x16 = orc.to_f16(x)
            for m in mats:
                w = synth.weight(synth.CFG_135M, l, m, *S[m])
                W[(l, m)] = up16(w)
                O[(l, m)] = torch.empty(S[m][0], dtype=torch.float32, device=DEV)
                want[(l, m)] = orc.mat_vec(w, x16, threads=HOST_T)
    wl = synth.weight(synth.CFG_135M, 0, "logits", *synth.SMOLLM2_135M_LOGITS)
    xl = np.ascontiguousarray(synth.activation(synth.CFG_135M, L, 0, 1, 576)[0])
    W["logits"], X["logits"] = up16(wl), up32(xl)
    O["logits"] = torch.empty(wl.shape[0], dtype=torch.float32, device=DEV)
    want["logits"] = orc.mat_vec(wl, orc.to_f16(xl), threads=HOST_T)

    def step():
        for l in range(L):
            for g, mats, _ in groups:
                if len(mats) > 1:
                    f16wm.mat_vec_multi([W[(l, m)] for m in mats], X[(l, g)], [O[(l, m)] for m in mats])
                else:
                    f16wm.mat_vec(W[(l, mats[0])], X[(l, g)], O[(l, mats[0])])
        f16wm.mat_vec(W["logits"], X["logits"], O["logits"])

    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    keys = list(want)
    _replay_and_check(graph, [O[key] for key in keys], [want[key] for key in keys], "135M decode step graph",
                      eager=step)
    del graph

    # the same 211 products as one table (f16wm_mat_vec_table): eagerly, then
    # captured and replayed
    src = {"q": "qkv", "k": "qkv", "v": "qkv", "o": "o", "gate": "gateup", "up": "gateup", "down": "down"}
    T = {key: torch.empty_like(o) for key, o in O.items()}
    table = f16wm.VecTable([(W[(l, m)], X[(l, src[m])], T[(l, m)]) for l in range(L) for m in S] +
                           [(W["logits"], X["logits"], T["logits"])])
    for o in T.values():
        o.fill_(float("nan"))
    table()
    torch.cuda.synchronize()
    for key in keys:
        assert_bits_equal(T[key].cpu().numpy(), want[key], "135M decode table %s" % (key,))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        table()
    torch.cuda.synchronize()
    _replay_and_check(graph, [T[key] for key in keys], [want[key] for key in keys], "135M decode step table graph",
                      eager=step)
    del graph


def test_llama3_8b_decode_set_as_graph(orc):
    """The 8B-shaped decode set as the benchmark runs it (Q/K/V grouped, O,
    gate/up grouped, down, logits; f32 columns rounded inside each launch),
    captured once as a HIP graph and replayed; all eight outputs against the
    oracle on every replay."""
    S = dict(synth.LLAMA3_8B, logits=synth.LLAMA3_8B_LOGITS)
    acts = synth.activation(synth.CFG_8B, 0, 0, 5, 14336)
    dec_k = {"attn": 4096, "o": 4096, "ffn": 4096, "down": 14336, "logits": 4096}
    X = {g: up32(np.ascontiguousarray(acts[i, :dec_k[g]])) for i, g in enumerate(dec_k)}
    x16 = {g: orc.to_f16(acts[i, :dec_k[g]]) for i, g in enumerate(dec_k)}
    src = {"q": "attn", "k": "attn", "v": "attn", "o": "o", "gate": "ffn", "up": "ffn", "down": "down",
           "logits": "logits"}
    W, O, want = {}, {}, {}
    for m, (rows, k) in S.items():
        w = synth.weight(synth.CFG_8B, 0, m, rows, k)
        W[m] = up16(w)
        O[m] = torch.empty(rows, dtype=torch.float32, device=DEV)
        want[m] = orc.mat_vec(w, x16[src[m]], threads=HOST_T)
        del w

    def step():
        f16wm.mat_vec_multi([W["q"], W["k"], W["v"]], X["attn"], [O["q"], O["k"], O["v"]])
        f16wm.mat_vec(W["o"], X["o"], O["o"])
        f16wm.mat_vec_multi([W["gate"], W["up"]], X["ffn"], [O["gate"], O["up"]])
        f16wm.mat_vec(W["down"], X["down"], O["down"])
        f16wm.mat_vec(W["logits"], X["logits"], O["logits"])

    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    _replay_and_check(graph, [O[m] for m in S], [want[m] for m in S], "8B decode set graph", eager=step)
    del graph

    # the eight products as one table launch, eagerly and as a graph
    T = {m: torch.empty_like(O[m]) for m in S}
    table = f16wm.VecTable([(W[m], X[src[m]], T[m]) for m in S])
    for o in T.values():
        o.fill_(float("nan"))
    table()
    torch.cuda.synchronize()
    for m in S:
        assert_bits_equal(T[m].cpu().numpy(), want[m], "8B decode table %s" % m)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        table()
    torch.cuda.synchronize()
    _replay_and_check(graph, [T[m] for m in S], [want[m] for m in S], "8B decode set table graph", eager=step)
    del graph


def _table_case(orc, seed, rows, k, f32, off=0):
    """A product's weight and column (host and device; f32 columns also
    rounded by the oracle)."""
    w = synth.random_f16((seed, rows, k, 1), (rows, k), 0.02)
    if f32:
        x = f32_column((seed, rows, k, 2), k)
        return w, x, orc.to_f16(x), up16(w), up32(x, off)
    a = synth.random_f16((seed, rows, k, 2), (k,))
    return w, a, a, up16(w), up16(a, off)


def test_mat_vec_table_every_kernel_class(orc):
    """One f16wm_mat_vec_table call over 230 products of every kind: short
    rows (k <= 576, registers) and staged rows (k up to 16384 with the whole
    column in LDS, and k = 16392 without), f16 and f32 columns (the rounding's
    edge values included), k % 32 tails, rows that leave a ragged last tile,
    empty matrices, k = 0, a shared column and a shared weight, more than 96
    products of one class (several launches), and misaligned or k % 8 != 0
    products that fall back to their own launches.  Every element against the
    oracle."""
    rng = np.random.default_rng(97)
    shapes = []
    for i in range(110):                     # > 96 products of the short-row f16 class
        shapes.append((int(rng.integers(1, 70)), int(rng.choice([8, 32, 40, 544, 576])), False, 0))
    for i in range(40):                      # short rows, f32 columns
        shapes.append((int(rng.integers(1, 300)), int(rng.choice([64, 200, 576])), True, 0))
    for i in range(40):                      # staged rows
        shapes.append((int(rng.integers(1, 400)), int(rng.choice([584, 640, 1000, 1536, 4096, 4104])), bool(i % 2), 0))
    shapes += [(4096, 14336, False, 0), (1000, 14336, True, 0), (33, 16384, False, 0), (17, 16392, True, 0),
               (70, 16392, False, 0), (0, 576, False, 0), (5, 0, False, 0), (16, 33, False, 0), (9, 100, True, 1),
               (40, 1000, False, 1), (3, 31, True, 0)]
    prods, wants = [], []
    for i, (rows, k, f32, off) in enumerate(shapes):
        w, x, x16, wd, xd = _table_case(orc, 2000 + i, rows, k, f32, off)
        prods.append((wd, xd))
        wants.append(orc.mat_vec(w, x16, threads=HOST_T) if rows else np.zeros(0, np.float32))
    # a shared column (product 0's) and a shared weight (product 1's)
    w0, _, x16_0, _, _ = _table_case(orc, 2000, *shapes[0][:3])
    prods.append((up16(w0), prods[0][1]))
    wants.append(orc.mat_vec(w0, x16_0, threads=HOST_T))
    w1, _, _, _, _ = _table_case(orc, 2001, *shapes[1][:3])
    a_new = synth.random_f16(3000, (shapes[1][1],))
    prods.append((prods[1][0], up16(a_new)))
    wants.append(orc.mat_vec(w1, a_new, threads=HOST_T))
    say("mat_vec_table: %d products" % len(prods))
    outs = f16wm.mat_vec_table(prods)
    for i, (o, wnt) in enumerate(zip(outs, wants)):
        assert_bits_equal(o.cpu().numpy(), wnt, "table product %d %s" % (i, shapes[i] if i < len(shapes) else "shared"))


# ------------------------------------------------------------- next rows

def _with_specials(h: np.ndarray, seed: int) -> np.ndarray:
    """f16 bit patterns with infinities, a NaN, subnormals, signed zeros and
    extremes planted at a few seeded positions."""
    out = h.copy().reshape(-1)
    sp = np.array([np.inf, -np.inf, np.nan, 6e-8, -6e-8, 0.0, -0.0, 65504.0, -65504.0, 6.1e-5],
                  dtype=np.float16).view(np.uint16)
    rng = np.random.default_rng(seed)
    idx = rng.choice(out.size, size=min(out.size // 16, sp.size), replace=False)
    out[idx] = sp[:idx.size]
    return out.reshape(h.shape)


@pytest.mark.parametrize("rows,k,n", [(12, 576, 4), (13, 576, 4), (12, 33, 3), (576, 576, 512),
                                      (4096, 4096, 7), (100, 1000, 1)])
def test_mat_mul_out_modes(orc, rows, k, n):
    """The last layer's output columns (forward page, why only the output rows
    leave the last layer): the last column alone in the vec_dot order, all
    columns in the shape's order, none computes nothing."""
    say("mat_mul_out rows=%d k=%d n=%d" % (rows, k, n))
    w = synth.random_f16(rows * 31 + k, (rows, k), 0.02)
    a = synth.random_f16(n * 17 + k, (n, k))
    wd, ad = up16(w), up16(a)
    assert f16wm.mat_mul_out(wd, ad, f16wm.OUT_NONE) is None
    last = f16wm.mat_mul_out(wd, ad, f16wm.OUT_LAST).cpu().numpy()
    assert_bits_equal(last, orc.mat_mul_out(w, a, orc.OUT_LAST), "last column")
    full = f16wm.mat_mul_out(wd, ad, f16wm.OUT_ALL).cpu().numpy()
    assert_bits_equal(full, orc.mat_mul_out(w, a, orc.OUT_ALL), "all columns")
    if orc.takes_sgemm(rows, k, n):
        # the page's point: the one-row product has different bits
        assert (last.view(np.uint32) != full[-1].view(np.uint32)).any()


@pytest.mark.parametrize("n_kv,n_kv_head,d,n_head,qoff", [
    (7, 2, 64, 8, 0), (33, 3, 64, 9, 0), (5, 1, 128, 3, 0), (9, 4, 72, 4, 0), (100, 2, 40, 6, 0),
    (17, 2, 30, 4, 0), (5, 1, 64, 100, 0), (33, 3, 30, 27, 0), (50, 2, 64, 4, 1), (1, 1, 8, 1, 0),
    (2000, 3, 64, 9, 0), (4096, 8, 128, 32, 0), (765, 2, 64, 4, 0), (48007, 8, 128, 24, 0),
    (40, 128, 128, 128, 0), (300, 1, 64, 512, 0), (1000, 3, 128, 12, 0), (3, 1, 128, 513, 0),
    (2500, 4, 128, 8, 0), (3000, 2, 128, 16, 0), (999, 5, 64, 10, 0)])
def test_kq_scores_match_the_oracle(orc, n_kv, n_kv_head, d, n_head, qoff):
    """vec_dot_u16 over an f16 K cache [n_kv][n_kv_head][d] with grouped-query
    heads: every score bit for bit; d % 8 != 0 or an unaligned query takes the
    lane-per-chain kernel, d % 32 != 0 exercises the binary64 tail, more query
    heads per KV head than a block holds splits them over blocks.  For the
    LDS kernel (d of 64 or 128): a grid of 6 tiles, blocks with 3 tiles
    each, query heads that leave threads idle, one position per 32 KB tile,
    512 query heads, rows that do not divide the tile; 513 heads fall back.
    Query heads per KV head divisible by 4, by 2 only, or odd: a K row read
    shared by a quad of lanes, a pair, or read by each lane."""
    say("kq n_kv=%d n_kv_head=%d d=%d n_head=%d qoff=%d" % (n_kv, n_kv_head, d, n_head, qoff))
    kc = _with_specials(synth.random_f16(n_kv + d, (n_kv, n_kv_head, d)), 1)
    q = synth.random_f16(n_head + d, (n_head, d))
    got = f16wm.kq(up16(kc), up16(q, qoff)).cpu().numpy()
    assert_bits_equal(got, orc.kq(kc, q), "kq")


def test_kq_8b_shaped_long_cache(orc):
    """An 8B-shaped layer cache at 32768 positions (8 KV heads x 128, 32 query
    heads): all 1,048,576 scores bit for bit."""
    n_kv, n_kv_head, d, n_head = 32768, 8, 128, 32
    kc = synth.random_f16(77, (n_kv, n_kv_head, d))
    q = synth.random_f16(78, (n_head, d))
    got = f16wm.kq(up16(kc), up16(q)).cpu().numpy()
    assert_bits_equal(got, orc.kq(kc, q), "kq 8B 32k")


@pytest.mark.parametrize("nvec,n,off", [(6, 67, 0), (32, 128, 0), (32, 128, 1), (1, 8, 0), (1000, 64, 0),
                                        (3, 5, 0), (4096, 128, 0)])
def test_mad_and_scale_match_the_oracle(orc, nvec, n, off):
    """The f16 V-accumulator updates, every element bit for bit (infinities,
    NaN, subnormals, signed zeros, overflow past 65504 included); n % 8 != 0
    or an unaligned accumulator takes the one-element kernel."""
    say("mad/scale nvec=%d n=%d off=%d" % (nvec, n, off))
    acc = _with_specials(synth.random_f16(nvec + n, (nvec, n), 4.0), 2)
    v = _with_specials(synth.random_f16(nvec * 3 + n, (nvec, n)), 3)
    rng = np.random.default_rng(nvec * 7 + n)
    w = (rng.standard_normal(nvec) * 3).astype(np.float32)
    s = (rng.standard_normal(nvec) * 2).astype(np.float32)
    if nvec > 2:
        w[1], s[1] = 0.0, 1.0
        w[2], s[2] = 3e4, 1e5          # overflow to infinity in f16
    ad = up16(acc, off)
    f16wm.mad(ad, up16(v), up32(w))
    want = orc.mad(acc, v, w)
    assert_f16_equal(ad.view(torch.int16).cpu().numpy().view(np.uint16), want, "mad")
    f16wm.scale(ad, up32(s))
    want = orc.scale(want, s)
    assert_f16_equal(ad.view(torch.int16).cpu().numpy().view(np.uint16), want, "scale")


def test_mad_and_scale_round_to_f32_before_f16(orc):
    """Results whose f32 value is an exact f16 tie while the exact value is
    not: rounding once, straight to f16, gives the other neighbour.  (A
    compiler fusion of the multiply or FMA with the f16 conversion into one
    mixed-precision instruction did exactly that.)"""
    acc = np.array([[0x39b2] * 8], np.uint16)                       # 0.712
    s = np.array([-0.5759602], np.float32)
    v = np.array([[0x3c01] * 8], np.uint16)                         # 1 + 2^-10
    w = np.array([np.float32(1) + np.float32(2.0 ** -23)], np.float32)
    want_s = orc.scale(acc, s)
    assert want_s[0, 0] == 0xb690                                   # the tie rounded to even
    ad = up16(acc)
    f16wm.scale(ad, up32(s))
    assert_f16_equal(ad.view(torch.int16).cpu().numpy().view(np.uint16), want_s, "scale tie")
    for a0 in (0x3c00, 0xbc00, 0x6800, 0x1400):
        acc2 = np.array([[a0] * 8], np.uint16)
        ad = up16(acc2)
        f16wm.mad(ad, up16(v), up32(w))
        assert_f16_equal(ad.view(torch.int16).cpu().numpy().view(np.uint16), orc.mad(acc2, v, w), "mad")


def assert_f16_equal(got: np.ndarray, want: np.ndarray, what: str):
    """f16 bit patterns equal, NaN compared as "is NaN" (payload propagation
    through an f32 NaN is the hardware's)."""
    got, want = np.asarray(got, np.uint16), np.asarray(want, np.uint16)
    assert got.shape == want.shape, what
    isnan = lambda b: ((b & 0x7c00) == 0x7c00) & ((b & 0x03ff) != 0)  # noqa: E731
    same = (got == want) | (isnan(got) & isnan(want))
    if not same.all():
        i = tuple(np.argwhere(~same)[0])
        raise AssertionError("%s: %d of %d differ; first at %s: got 0x%04x want 0x%04x"
                             % (what, int((~same).sum()), got.size, i, got[i], want[i]))
