"""Pins for the oracle's weight-only matmul y = x . W_hat^T (CPU only).

Exact rational brute force on tiny shapes, numpy's float64 matmul, one-hot
activations, zero rows and row invariants; shapes are non-square so a
transposed operand cannot pass.
"""
from fractions import Fraction

import numpy as np

import slq_synth as S


def test_brute_force_exact_rational(orc):
    m, k, n = 3, 128, 5
    x = S.activations_bf16(m, k, 1)
    W = S.skewed_weights(n, k, 2)
    q, s, z = orc.quantize(W, 4)
    wh = orc.dequantize(q, s, z)
    y, bound = orc.gemm(x, wh)
    assert y.shape == (m, n)
    xf = S.bf16_bits_to_f32(x)
    for i in range(m):
        for c in range(n):
            exact = sum(Fraction(float(xf[i, j])) * Fraction(float(wh[c, j])) for j in range(k))
            babs = sum(abs(Fraction(float(xf[i, j])) * Fraction(float(wh[c, j]))) for j in range(k))
            assert abs(y[i, c] - float(exact)) <= 1e-12 * float(babs)
            assert abs(bound[i, c] - float(babs)) <= 1e-12 * float(babs)


def test_matches_numpy_float64_matmul(orc):
    m, k, n = 7, 384, 33
    x = S.activations_bf16(m, k, 3)
    W = S.skewed_weights(n, k, 4, row_offset_std=0.005)
    q, s, z = orc.quantize(W, 3)
    wh = orc.dequantize(q, s, z)
    y, bound = orc.gemm(x, wh)
    xf = S.bf16_bits_to_f32(x).astype(np.float64)
    ref = xf @ wh.astype(np.float64).T
    assert np.allclose(y, ref, rtol=0, atol=1e-12 * bound.max())
    assert np.allclose(bound, np.abs(xf) @ np.abs(wh.astype(np.float64)).T, rtol=1e-13)
    assert (bound >= np.abs(y)).all()


def test_one_hot_and_zero_rows(orc):
    k, n = 256, 9
    W = S.skewed_weights(n, k, 5)
    W[4] = 0.0
    q, s, z = orc.quantize(W, 6)
    wh = orc.dequantize(q, s, z)
    assert (wh[4] == 0).all()
    x = np.zeros((k, k), np.uint16)
    x[np.arange(k), np.arange(k)] = 0x3F80   # bf16 1.0
    y, _ = orc.gemm(x, wh)
    assert (y == wh.T.astype(np.float64)).all()
    xr = S.activations_bf16(2, k, 6)
    xr[1] = xr[0]
    y2, b2 = orc.gemm(xr, wh)
    assert (y2[:, 4] == 0).all() and (b2[:, 4] == 0).all()
    assert (y2[0] == y2[1]).all()


def test_pairs_match_full(orc):
    m, k, n = 4, 256, 6
    x = S.activations_bf16(m, k, 7)
    W = S.skewed_weights(n, k, 8)
    q, s, z = orc.quantize(W, 5)
    wh = orc.dequantize(q, s, z)
    y, b = orc.gemm(x, wh)
    xi = np.array([0, 3, 2, 1], np.int64)
    wi = np.array([5, 0, 2, 4], np.int64)
    yp, bp = orc.gemm_pairs(x, wh, xi, wi)
    assert (yp == y[xi, wi]).all() and (bp == b[xi, wi]).all()
