"""The acceptance check of the fp16 matrix-core (MFMA) product, shared by the
GPU parity tests and the CPU test that shows it catches plausible mistakes.

The MFMA path is approximate (its summation order is the matrix core's), so
it is judged against the binary64 reference of the oracle on sampled elements:
at least 16 in every 64 x 64 block of the output, against (1) the gate
max |y - ref| / sum|w a| <= 2e-3, (2) an error bound derived from f32
accumulation, element by element, and (3) the plain relative error on
elements that are not near zero.
"""
import numpy as np

MFMA_TOL = 2e-3


def tile_samples(rows, n, seed, per=16, blk=64):
    """`per` seeded random elements in every blk x blk block of a rows x n
    output, ragged edge blocks included (every tile shape the MFMA kernels
    use, 256 x 256 down to 128 x 64, is a union of 64 x 64 blocks).
    Returns (row indices, column indices)."""
    rng = np.random.default_rng(seed)
    r0, c0 = np.meshgrid(np.arange(0, rows, blk), np.arange(0, n, blk), indexing="ij")
    r0, c0 = r0.ravel(), c0.ravel()
    hr, hc = np.minimum(blk, rows - r0), np.minimum(blk, n - c0)
    rr = r0[:, None] + (rng.random((r0.size, per)) * hr[:, None]).astype(np.int64)
    cc = c0[:, None] + (rng.random((c0.size, per)) * hc[:, None]).astype(np.int64)
    return rr.ravel(), cc.ravel()


def f32_accumulation_bound(k: int) -> float:
    """Relative bound (times sum |w a|) on an fp16 MFMA product with f32
    accumulation over k, and on the binary64 reference's own error.  Every
    f16 x f16 product is exact; one v_mfma_f32_32x32x16_f16 adds 16 of them to
    the f32 accumulator, so with any internal order of at least f32 precision
    each product passes through at most ceil(k/16) + 15 roundings of unit
    2^-24: recursive summation gives |y - exact| <= gamma_m * sum|w a| with
    m = ceil(k/16) + 16 (one spare) and gamma_m = m u / (1 - m u).  The
    binary64 reference adds at most k * 2^-53 * sum|w a|."""
    m = -(-k // 16) + 16
    u = 2.0 ** -24
    return m * u / (1 - m * u) + k * 2.0 ** -53


def mfma_check(orc, w, a, got, rr, cc, what):
    """The MFMA product at the sampled elements against the binary64
    reference: (1) the gate max |y - ref| / sum|w a| <= 2e-3; (2) the f32
    accumulation bound above, element by element; (3) the plain relative
    error |y - ref| / |ref| <= 2e-3 on elements with |ref| >= 1e-2 rms(ref).
    Returns (max gate ratio, max relative error)."""
    ref, scale = orc.fp64_at(w, a, rr, cc)
    y = got[cc, rr].astype(np.float64)
    d = np.abs(y - ref)
    err = d / np.maximum(scale, 1e-300)
    gate = float(err.max())
    assert gate <= MFMA_TOL, "%s: max |y-ref|/sum|wa| = %.3g" % (what, gate)
    bound = f32_accumulation_bound(w.shape[1]) * scale
    bad = d > bound
    if bad.any():
        i = int(np.argmax(bad))
        raise AssertionError("%s: %d of %d sampled elements exceed the f32 accumulation bound; first (r=%d, c=%d): "
                             "|y-ref| = %.3g > %.3g" % (what, int(bad.sum()), d.size, rr[i], cc[i], d[i], bound[i]))
    rms = np.sqrt(np.mean(ref ** 2))
    big = np.abs(ref) >= 1e-2 * rms
    rel = float((d[big] / np.abs(ref[big])).max()) if big.any() else 0.0
    assert rel <= MFMA_TOL, "%s: max relative error %.3g on |ref| >= 1e-2 rms" % (what, rel)
    return gate, rel
