"""Pins of the oracle's compact group metadata (SLQ README, Search: the
bit-width map adds 0.156 bits per parameter of scale and zero point, 20 bits
per 128-group; Evaluation: Uniform-4 at 4.16 bpp).

Readings: binary16 scale rounded up from the fp32 scale; the zero point and
codes computed with the stored scale; 4-bit zero points for b <= 4 (nibble i,
low nibble first), bytes above."""
import numpy as np
import pytest

import oracle
import slq_synth as S


def f16_np(bits):
    return float(np.array([bits], np.uint16).view(np.float16)[0])


def test_binary16_value_and_round_up_exhaustive():
    """Every positive finite binary16 value (numpy's float16 as the second
    implementation): the value decodes alike, rounds up to itself, the next
    fp32 above it rounds to the next binary16 value, the one below to itself."""
    for b in range(1, 0x7C00):
        v = f16_np(b)
        assert oracle.f16_value(b) == v
        f = np.float32(v)
        assert oracle.f16_round_up(f) == b
        up = np.nextafter(f, np.float32(np.inf))
        assert oracle.f16_round_up(up) == (b + 1 if b < 0x7BFF else 0x7BFF)
        dn = np.nextafter(f, np.float32(0))
        if dn > 0:
            assert oracle.f16_round_up(dn) == b


def test_round_up_random_and_saturation():
    g = np.random.default_rng(1)
    for s in np.exp(g.uniform(np.log(1e-9), np.log(6e4), 4000)).astype(np.float32):
        b = oracle.f16_round_up(s)
        assert f16_np(b) >= s and (b == 1 or f16_np(b - 1) < s)
    assert oracle.f16_round_up(np.float32(1e6)) == 0x7BFF


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 8])
def test_compact_grid_bound(bits):
    W = S.skewed_weights(24, 1024, 40 + bits)
    W[3] = 0.0
    q, s16, z = oracle.quantize_compact(W, bits)
    _, s32, _ = oracle.quantize(W, bits)
    sv = np.vectorize(oracle.f16_value)(s16).astype(np.float64)
    assert np.all(sv >= s32) and np.all(sv <= s32 * (1 + 2.0 ** -10))
    assert q.max() <= 2 ** bits - 1 and z.max() <= 2 ** bits - 1
    zp = oracle.pack_zeros(z, bits)
    wh = oracle.dequantize_compact(q, s16, zp, bits)
    err = np.abs(W.astype(np.float64) - wh)
    bound = np.repeat(sv, 128, axis=1) * (0.5 + 2.0 ** -12)
    assert np.all(err <= bound)
    assert np.all(wh[3] == 0.0)


def test_representable_scale_matches_fp32_metadata():
    """A group whose fp32 scale is a binary16 value gives the same codes and
    zero point under both layouts."""
    g = np.random.default_rng(2)
    bits, maxq = 4, 15
    W = (g.integers(0, maxq + 1, (8, 256)) - 5).astype(np.float32) * np.float32(2.0 ** -6)
    W[:, 0] = -5 * 2.0 ** -6
    W[:, 1] = 10 * 2.0 ** -6     # range = 15 * 2^-6, s = 2^-6
    q1, s32, z1 = oracle.quantize(W, bits)
    q2, s16, z2 = oracle.quantize_compact(W, bits)
    assert np.all(s32 == 2.0 ** -6)
    assert np.array_equal(q1, q2) and np.array_equal(z1, z2)
    assert np.all(np.vectorize(oracle.f16_value)(s16) == s32)


def test_metadata_bits_match_the_readme_map():
    """16-bit scale + 4-bit zero point = 20 bits per 128-group: the README's
    "2:2.156 ... 4:4.156" and Uniform-4 at 4.16 bpp; 24 bits above 4 bits."""
    for b in (2, 3, 4):
        bpp = oracle.bits_per_param(b, 16 + oracle.compact_zero_bits(b))
        assert bpp == b + 0.15625 and round(bpp, 3) == round(b + 0.156, 3)
    assert round(oracle.bits_per_param(4, 16 + oracle.compact_zero_bits(4)), 2) == 4.16
    for b in (5, 6, 7, 8):
        assert oracle.bits_per_param(b, 16 + oracle.compact_zero_bits(b)) == b + 0.1875


def test_zero_point_layout_golden():
    assert list(oracle.pack_zeros(np.array([3, 10, 7], np.uint8), 4)) == [0xA3, 0x07]
    assert list(oracle.pack_zeros(np.array([1, 2, 3, 0], np.uint8), 2)) == [0x21, 0x03]
    assert list(oracle.pack_zeros(np.array([200, 17, 5], np.uint8), 8)) == [200, 17, 5]


def test_dequantize_compact_by_hand():
    q = np.array([[0, 5, 15, 7] * 32], np.uint8)
    s16 = np.array([0x2E66], np.uint16)    # binary16 0.1 rounded to 0.0999755859375
    zp = oracle.pack_zeros(np.array([5], np.uint8), 4)
    wh = oracle.dequantize_compact(q, s16, zp, 4)
    s = np.float32(f16_np(0x2E66))
    ref = ((q.astype(np.int32) - 5).astype(np.float32) * s)
    assert np.array_equal(wh, ref)
