"""Pins for the oracle's group quantizer (CPU only).

Each check fixes the oracle against something other than itself: brute-force
nearest-grid search in exact rational arithmetic, the round-trip bound, exact
grid points, the round-half-even tie rule, and the centering relation
s_sym / s_asym = gamma = 2M/R (gist.science summary, Methodology 1).
"""
from fractions import Fraction

import numpy as np
import pytest

import slq_synth as S

BITS = [2, 3, 4, 5, 6, 7, 8]


def _groups(bits, seed):
    """A mix of group shapes: skewed, outliers, one-signed, all-zero, tiny."""
    g = np.random.Generator(np.random.PCG64(seed))
    rows = [
        S.skewed_weights(1, 128, seed)[0],
        g.uniform(0.01, 0.2, 128).astype(np.float32),        # all positive
        -g.uniform(0.01, 0.2, 128).astype(np.float32),       # all negative
        np.zeros(128, np.float32),                            # degenerate
        (g.standard_normal(128) * 1e-3).astype(np.float32),
        (g.standard_normal(128) * 40.0 + 5.0).astype(np.float32),
    ]
    return np.stack(rows)


@pytest.mark.parametrize("bits", BITS)
def test_codes_are_nearest_grid_points(orc, bits):
    W = _groups(bits, 11 + bits)
    q, s, z = orc.quantize(W, bits)
    maxq = (1 << bits) - 1
    assert q.max() <= maxq and z.max() <= maxq
    for r in range(W.shape[0]):
        sr = Fraction(float(s[r, 0]))
        zr = int(z[r, 0])
        for i in range(0, 128, 7):
            w = Fraction(float(W[r, i]))
            dist = [abs(w - (c - zr) * sr) for c in range(maxq + 1)]
            best = min(dist)
            # fl32(w/s) may move a value within one ulp of a half-integer
            assert dist[int(q[r, i])] <= best + sr * Fraction(1, 1 << 20), (r, i)


@pytest.mark.parametrize("bits", BITS)
def test_grid_covers_range_including_zero(orc, bits):
    """Reading R1: the grid spans [min(0, min w), max(0, max w)]."""
    W = _groups(bits, 21 + bits)
    q, s, z = orc.quantize(W, bits)
    maxq = (1 << bits) - 1
    for r in range(W.shape[0]):
        lo = min(0.0, float(W[r].min()))
        hi = max(0.0, float(W[r].max()))
        if hi == lo:
            assert s[r, 0] == 1.0 and z[r, 0] == 0   # reading R2
            continue
        sr = float(s[r, 0])
        assert abs(-int(z[r, 0]) * sr - lo) <= 0.5 * sr * (1 + 1e-6)
        assert abs((maxq - int(z[r, 0])) * sr - hi) <= 0.5 * sr * (1 + 1e-6)
        # scale equals range / (2^b - 1) up to one fp32 rounding
        assert abs(sr - (hi - lo) / maxq) <= 2 ** -23 * sr * 2


@pytest.mark.parametrize("bits", BITS)
def test_round_trip_error_at_most_half_scale(orc, bits):
    W = S.skewed_weights(64, 512, 5 + bits, row_offset_std=0.005)
    q, s, z = orc.quantize(W, bits)
    wh = orc.dequantize(q, s, z)
    srep = np.repeat(s, 128, axis=1)
    err = np.abs(W.astype(np.float64) - wh)
    assert (err <= srep * (0.5 + 2 ** -12)).all()
    assert (err / srep).max() > 0.45   # the bound is reached, not vacuous


@pytest.mark.parametrize("bits", BITS)
def test_values_on_grid_reproduce_codes(orc, bits):
    maxq = (1 << bits) - 1
    g = np.random.Generator(np.random.PCG64(bits))
    s0 = np.float32(2.0 ** -6)
    z0 = int(g.integers(1, maxq))
    codes = g.integers(0, maxq + 1, size=128)
    codes[3], codes[77] = 0, maxq
    W = ((codes - z0).astype(np.float32) * s0)[None, :]
    q, s, z = orc.quantize(W, bits)
    assert s[0, 0] == s0 and z[0, 0] == z0
    assert (q[0] == codes).all()


def test_ties_round_half_to_even(orc):
    # 4-bit group with lo = 0, hi = 15/16: s = 1/16 exactly, z = 0
    w = np.full(128, 0.25, np.float32)
    w[0], w[1] = 0.0, 15 / 16
    w[2] = 2.5 / 16   # tie between 2 and 3 -> 2
    w[3] = 3.5 / 16   # tie between 3 and 4 -> 4
    w[4] = 0.5 / 16   # tie between 0 and 1 -> 0
    q, s, z = orc.quantize(w[None, :], 4)
    assert s[0, 0] == np.float32(1 / 16) and z[0, 0] == 0
    assert list(q[0, :5]) == [0, 15, 2, 4, 0]


@pytest.mark.parametrize("bits", [3, 4, 8])
def test_symmetric_grid_and_centering_ratio(orc, bits):
    """s_sym / s_asym = 2M/R = gamma; equal grids when lo = -hi."""
    maxq = (1 << bits) - 1
    g = np.random.Generator(np.random.PCG64(99))
    W = g.uniform(-0.3, 0.5, size=(16, 128)).astype(np.float32)
    _, sa, za = orc.quantize(W, bits)
    qs, ss, zs = orc.quantize(W, bits, symmetric=True)
    assert (zs == (1 << (bits - 1))).all()
    for r in range(16):
        M = float(np.abs(W[r]).max())
        R = float(W[r].max()) - float(W[r].min())
        assert abs(float(ss[r, 0]) / float(sa[r, 0]) - 2 * M / R) < 1e-5
        assert abs(float(ss[r, 0]) - 2 * M / maxq) <= 2 ** -22 * float(ss[r, 0])
    # symmetric group: lo = -hi -> identical scale bits
    Wsym = g.uniform(-0.2, 0.2, size=(4, 128)).astype(np.float32)
    Wsym[:, 0], Wsym[:, 1] = -0.25, 0.25
    _, sa2, _ = orc.quantize(Wsym, bits)
    _, ss2, _ = orc.quantize(Wsym, bits, symmetric=True)
    assert (sa2.view(np.uint32) == ss2.view(np.uint32)).all()
    # symmetric round trip also within s/2
    wh = orc.dequantize(qs, ss, zs)
    assert (np.abs(W - wh) <= np.repeat(ss, 128, axis=1) * (0.5 + 2 ** -12)).all()


def test_groups_are_independent_along_k(orc):
    """A change in one group moves only that group's scale, zero and codes."""
    W = S.skewed_weights(4, 1024, 3)
    q, s, z = orc.quantize(W, 5)
    W2 = W.copy()
    W2[2, 384:512] *= 3.0
    q2, s2, z2 = orc.quantize(W2, 5)
    diff = (s != s2)
    assert diff[2, 3] and diff.sum() == 1
    mask = np.ones_like(q, bool)
    mask[2, 384:512] = False
    assert (q[mask] == q2[mask]).all()
