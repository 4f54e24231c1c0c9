"""Pins of the oracle's f16 conversions to things other than itself.

to_f16 (bankML f16 page, Design notes "Activation": round to nearest even, as
F16C vcvtps2ph with immediate 0 does) is checked on every one of the 2^32
binary32 bit patterns against (1) the host's own F16C instruction and (2)
numpy's float32 -> float16 cast (non-NaN inputs).  widen (Technical usage:
"exact") is checked on all 2^16 binary16 patterns against numpy's float16 ->
float32 cast and the host's vcvtph2ps.
"""
import concurrent.futures as cf
import ctypes
import os
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def _has_f16c():
    try:
        with open("/proc/cpuinfo") as f:
            txt = f.read()
    except OSError:
        return False
    return " f16c" in txt and " avx" in txt


@pytest.fixture(scope="module")
def f16c(tmp_path_factory):
    if not _has_f16c():
        pytest.skip("host CPU has no F16C")
    out = str(tmp_path_factory.mktemp("f16c") / "libf16c.so")
    subprocess.check_call(["gcc", "-O2", "-mavx", "-mf16c", "-fPIC", "-shared",
                           os.path.join(HERE, "helpers", "f16c_cvt.c"), "-o", out])
    L = ctypes.CDLL(out)
    L.f16c_to_f16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
    L.f16c_widen.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
    return L


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


CHUNK = 1 << 25


def _check_chunk(orc, f16c, c):
    bits = np.arange(c * CHUNK, (c + 1) * CHUNK, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    got = orc.to_f16(x)
    hw = np.empty_like(got)
    f16c.f16c_to_f16(_p(x), _p(hw), x.size)
    bad_hw = int(np.count_nonzero(got != hw))
    nan = np.isnan(x)
    with np.errstate(over="ignore", invalid="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    bad_np = int(np.count_nonzero((got != ref) & ~nan))
    # NaN: quiet NaN, sign kept, top ten payload bits kept
    xb = bits[nan]
    want = ((xb >> 16) & 0x8000) | 0x7E00 | ((xb & 0x7FFFFF) >> 13)
    bad_nan = int(np.count_nonzero(got[nan] != want.astype(np.uint16)))
    return bad_hw, bad_np, bad_nan


@pytest.mark.slow
def test_to_f16_exhaustive_vs_f16c_and_numpy(orc, f16c):
    """All 2^32 binary32 inputs: the oracle equals F16C vcvtps2ph(imm=0) bit for
    bit (NaNs included) and numpy's cast on every non-NaN input."""
    nchunks = (1 << 32) // CHUNK
    tot = np.zeros(3, dtype=np.int64)
    with cf.ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        for r in ex.map(lambda c: _check_chunk(orc, f16c, c), range(nchunks)):
            tot += r
    assert tot.tolist() == [0, 0, 0]


def test_to_f16_special_values(orc):
    """Boundary values worked out from the binary16 format."""
    cases = [
        (0.0, 0x0000), (-0.0, 0x8000), (1.0, 0x3C00), (-2.0, 0xC000),
        (65504.0, 0x7BFF),                 # largest finite f16
        (65519.99, 0x7BFF),                # below the midpoint to 2^16
        (65520.0, 0x7C00),                 # the midpoint rounds to even = overflow
        (float("inf"), 0x7C00), (float("-inf"), 0xFC00),
        (2.0 ** -14, 0x0400),              # smallest normal
        (2.0 ** -24, 0x0001),              # smallest subnormal
        (2.0 ** -25, 0x0000),              # tie between 0 and 2^-24 -> even (0)
        (-(2.0 ** -25), 0x8000),
        (1.5 * 2.0 ** -25, 0x0001),        # above the tie
        (1.0 + 2.0 ** -11, 0x3C00),        # tie between 1 and 1+2^-10 -> even (1)
        (1.0 + 3 * 2.0 ** -11, 0x3C02),    # tie between 1+2^-10 and 1+2^-9 -> even
        (2.0 ** -14 - 2.0 ** -25, 0x0400), # tie between 1023*2^-24 and 2^-14 -> even (1024)
    ]
    x = np.array([c[0] for c in cases], dtype=np.float32)
    got = orc.to_f16(x)
    assert [hex(v) for v in got.tolist()] == [hex(c[1]) for c in cases]


def test_widen_exhaustive(orc, request):
    """All 2^16 binary16 patterns widen exactly (numpy's cast; F16C too)."""
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.widen(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(got.view(np.uint32)[~nan], ref.view(np.uint32)[~nan])
    assert np.isnan(got[nan]).all()
    # the NaN results keep the sign and carry the payload in the top bits, quiet
    gb = got.view(np.uint32)[nan]
    hb = h[nan].astype(np.uint32)
    assert np.array_equal(gb, ((hb & 0x8000) << 16) | 0x7FC00000 | ((hb & 0x3FF) << 13))
    if _has_f16c():
        hw = np.empty_like(got)
        f16c = request.getfixturevalue("f16c")
        f16c.f16c_widen(_p(h), _p(hw), h.size)
        assert np.array_equal(got.view(np.uint32)[~nan], hw.view(np.uint32)[~nan])


def test_round_trip(orc):
    """to_f16(widen(h)) == h for every non-NaN f16."""
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ok = ~np.isnan(h.view(np.float16))
    assert np.array_equal(orc.to_f16(orc.widen(h))[ok], h[ok])
