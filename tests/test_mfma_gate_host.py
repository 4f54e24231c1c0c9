"""The MFMA acceptance check (tests/mfma_gate.py) catches plausible mistakes.

On the CPU: the product of seeded f16 operands is accumulated the way a
matrix core with f32 accumulators could do it (each 16 products summed
exactly and rounded once to binary32, then added to a binary32 accumulator),
which the check must accept; then the same result with one planted mistake —
one 64-deep k stage left out of one element, one element's sign flipped, the
output transposed, the last k stage repeated in one element — which it must
reject.  The binary64 reference is the oracle's (itself pinned to the exact
fixed-point sum in test_oracle_orders.py).
"""
import numpy as np
import pytest

import synth
from mfma_gate import f32_accumulation_bound, mfma_check, tile_samples


def emulated_f32_product(w, a):
    """out[c, r]: 16-deep exact partial sums rounded to f32, accumulated in f32."""
    wf = w.view(np.float16).astype(np.float64)
    af = a.view(np.float16).astype(np.float64)
    k = w.shape[1]
    acc = np.zeros((a.shape[0], w.shape[0]), np.float32)
    for k0 in range(0, k, 16):
        part = af[:, k0:k0 + 16] @ wf[:, k0:k0 + 16].T     # exact: f16 x f16 products, 16 terms
        acc = (acc + part.astype(np.float32)).astype(np.float32)
    return acc


@pytest.fixture(scope="module")
def case():
    rows, k, n = 192, 2048, 128
    w = synth.random_f16((5, 1), (rows, k), 0.02)
    a = synth.random_f16((5, 2), (n, k))
    return w, a, emulated_f32_product(w, a)


def test_bound_scales_with_k():
    assert f32_accumulation_bound(16) < f32_accumulation_bound(4096) < f32_accumulation_bound(14336) < 1e-4


def test_an_f32_accumulated_product_passes(orc, case):
    w, a, got = case
    rr, cc = tile_samples(w.shape[0], a.shape[0], 1)
    assert rr.size == 16 * 3 * 2                   # 16 per 64 x 64 block, 3 x 2 blocks
    gate, rel = mfma_check(orc, w, a, got, rr, cc, "emulated")
    assert gate < 1e-6 and rel < 1e-3


def _planted(orc, w, a, got, what):
    rr, cc = tile_samples(w.shape[0], a.shape[0], 1)
    with pytest.raises(AssertionError):
        mfma_check(orc, w, a, got, rr, cc, what)


def test_a_dropped_k_stage_is_caught(orc, case):
    """One element loses its products 1024..1087 (a 64-deep stage)."""
    w, a, got = case
    rr, cc = tile_samples(w.shape[0], a.shape[0], 1)
    r, c = int(rr[40]), int(cc[40])                 # a sampled element
    bad = got.copy()
    wf = w[r, 1024:1088].view(np.float16).astype(np.float64)
    af = a[c, 1024:1088].view(np.float16).astype(np.float64)
    bad[c, r] = np.float32(bad[c, r] - np.dot(wf, af))
    _planted(orc, w, a, bad, "dropped stage")


def test_a_repeated_k_stage_is_caught(orc, case):
    w, a, got = case
    rr, cc = tile_samples(w.shape[0], a.shape[0], 1)
    r, c = int(rr[7]), int(cc[7])
    bad = got.copy()
    wf = w[r, -64:].view(np.float16).astype(np.float64)
    af = a[c, -64:].view(np.float16).astype(np.float64)
    bad[c, r] = np.float32(bad[c, r] + np.dot(wf, af))
    _planted(orc, w, a, bad, "repeated stage")


def test_a_sign_slip_and_a_transposed_output_are_caught(orc, case):
    w, a, got = case
    rr, cc = tile_samples(w.shape[0], a.shape[0], 1)
    bad = got.copy()
    bad[cc[3], rr[3]] = -bad[cc[3], rr[3]]
    _planted(orc, w, a, bad, "sign")
    # transposed: rows and columns of the output swapped (square block)
    sq = got[:128, :128].T.copy()
    w2 = w[:128]
    rr2, cc2 = tile_samples(128, 128, 2)
    with pytest.raises(AssertionError):
        mfma_check(orc, w2, a, sq, rr2, cc2, "transposed")
