"""Pins for the oracle's NF4 codec (oracle.nf4), against facts fixed by the
mathematics rather than by the oracle itself."""
import math

import numpy as np
import pytest

from oracle import nf4


def _phi(x):
    """Standard normal CDF from the C library's erf (independent of scipy)."""
    return 0.5 * (1.0 + math.erf(x / math.sqrt(2.0)))


def _phi_inv(p):
    lo, hi = -10.0, 10.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if _phi(mid) < p:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def test_codebook_invariants():
    c = nf4.codebook()
    assert c.dtype == np.float32 and c.shape == (16,)
    assert np.all(np.diff(c) > 0)
    assert c[0] == -1.0 and c[15] == 1.0 and c[7] == 0.0
    assert np.sum(c < 0) == 7 and np.sum(c > 0) == 8


def test_codebook_is_normal_quantiles():
    # c_i * z_top must land on the evenly spaced probabilities of the
    # construction: 9 points from 1-delta to 1/2 for the positive half and
    # 8 for the negative half (delta = (1/32 + 1/30)/2).
    delta = 0.5 * (1 / 32 + 1 / 30)
    z_top = _phi_inv(1 - delta)
    c = nf4.codebook_f64()
    pos = sorted(c[c > 0])
    neg = sorted(-c[c < 0])
    want_pos = sorted(np.linspace(1 - delta, 0.5, 9)[:-1])
    want_neg = sorted(np.linspace(1 - delta, 0.5, 8)[:-1])
    for ci, p in zip(pos, want_pos):
        assert abs(_phi(ci * z_top) - p) < 1e-9
    for ci, p in zip(neg, want_neg):
        assert abs(_phi(ci * z_top) - p) < 1e-9
    # float32 values are the nearest float32 of the float64 levels
    assert np.array_equal(nf4.codebook(), c.astype(np.float32))


def test_midpoint_rule_equals_argmin_bruteforce():
    rng = np.random.default_rng(123)
    x = rng.uniform(-1, 1, 200000).astype(np.float32)
    c64 = nf4.codebook().astype(np.float64)
    mids = nf4.midpoints()
    code_mid = (x[:, None] > mids[None, :]).sum(1)
    dist = np.abs(x.astype(np.float64)[:, None] - c64[None, :])
    code_arg = dist.argmin(1)
    # exclude exact float32 ties with a midpoint (handled by the tie rule)
    tie = np.isin(x, mids)
    assert np.array_equal(code_mid[~tie], code_arg[~tie])


def test_pack_layout_by_hand():
    assert list(nf4.pack([1, 2, 3])) == [0x21, 0x03]
    assert list(nf4.unpack(np.array([0x21, 0x03], np.uint8), 3)) == [1, 2, 3]


def test_quantize_known_block():
    # one block of 64: element 0 is the max (-> code 15), a ties-at-midpoint
    # element goes to the lower code, exact levels map to their own code
    c = nf4.codebook()
    mids = nf4.midpoints()
    w = np.zeros(64, np.float32)
    w[0] = 1.0
    w[1] = mids[9]               # exactly between c_9 and c_10 -> 9
    w[2] = c[3]                  # a level -> 3
    w[3] = -1.0                  # -> 0
    w[4] = -0.0                  # -> 7
    codes, absmax = nf4.quantize(w)
    got = nf4.unpack(codes, 64)
    assert absmax[0] == 1.0
    assert list(got[:5]) == [15, 9, 3, 0, 7]
    assert np.all(got[5:] == 7)


def test_zero_block_and_partial_tail():
    w = np.zeros(64 + 64 + 5, np.float32)
    w[64:128] = np.linspace(-2, 3, 64, dtype=np.float32)
    w[128:] = [0.5, -0.25, 0, 0.125, 0.5]
    codes, absmax = nf4.quantize(w)
    assert codes.size == (w.size + 1) // 2 and absmax.size == 3
    assert absmax[0] == 0 and np.all(nf4.unpack(codes, w.size)[:64] == 7)
    assert absmax[1] == np.float32(3.0) and absmax[2] == np.float32(0.5)
    # odd length pads a zero high nibble
    assert codes[-1] >> 4 == 0
    d = nf4.dequantize(codes, absmax, w.size)
    assert np.all(d[:64] == 0)
    assert d[127] == 3.0 and d[128] == 0.5


def test_round_trip_exact():
    rng = np.random.default_rng(7)
    nblk = 300
    codes = rng.integers(0, 16, nblk * 64).astype(np.uint8)
    # every block holds one element at +-1 so that its absmax is recovered
    codes[::64] = rng.choice([0, 15], nblk)
    absmax = (rng.uniform(0.01, 0.2, nblk)).astype(np.float32)
    packed = nf4.pack(codes)
    w = nf4.dequantize(packed, absmax, codes.size)
    packed2, absmax2 = nf4.quantize(w)
    assert np.array_equal(packed2, packed)
    assert np.array_equal(absmax2.view(np.uint32), absmax.view(np.uint32))


def test_requantize_is_idempotent_on_weights():
    rng = np.random.default_rng(11)
    w = (rng.standard_normal(64 * 500, dtype=np.float32) * np.float32(0.02))
    p1, a1 = nf4.quantize(w)
    w1 = nf4.dequantize(p1, a1, w.size)
    p2, a2 = nf4.quantize(w1)
    assert np.array_equal(p1, p2) and np.array_equal(a1, a2)
    # error bound: half the widest gap between levels, times absmax
    gap = np.max(np.diff(nf4.codebook().astype(np.float64))) / 2
    err = np.abs(w1.astype(np.float64) - w)
    assert np.all(err <= gap * np.repeat(a1, 64) + 1e-12)


def test_non_finite_rejected():
    w = np.zeros(64, np.float32)
    w[3] = np.nan
    with pytest.raises(ValueError):
        nf4.quantize(w)
    w[3] = np.inf
    with pytest.raises(ValueError):
        nf4.quantize(w)


def test_thresholds_are_float64_midpoints_rounded():
    # For float32 x near each midpoint (but not equal to the float32
    # threshold) the code must be the nearest float64 level: no float32
    # value lies strictly between the float64 midpoint and its rounding.
    c64 = nf4.codebook_f64()
    mids = nf4.midpoints()
    xs = []
    for j in range(15):
        m64 = (c64[j] + c64[j + 1]) / 2
        x = np.float32(m64)
        for _ in range(16):
            x = np.nextafter(x, np.float32(-2))
        for _ in range(33):
            xs.append(x)
            x = np.nextafter(x, np.float32(2))
    xs = np.array(xs, np.float32)
    xs = xs[~np.isin(xs, mids)]
    code = (xs[:, None] > mids[None, :]).sum(1)
    near = np.abs(xs.astype(np.float64)[:, None] - c64[None, :]).argmin(1)
    assert np.array_equal(code, near)
