"""Pins of the oracle's fp32 GPTQ column pass with lazy 128-column blocks
(oracle.c, oracle_gptq_columns; the published GPTQ algorithm, Frantar et al.,
ICLR 2023, Algorithm 1, named by the SLQ README, Pipeline paragraph, as the
code-choice step).  It is pinned against the fp64 column-by-column pass
(oracle/gptq.py, itself pinned in test_oracle_gptq.py): exactly, on inputs
where every fp32 operation of either form is exact, and by agreement and
layer loss on correlated Hessians; a diagonal factor reduces it to the plain
quantizer."""
import numpy as np
import pytest

import oracle
import slq_synth as S
from oracle import gptq as G


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_diagonal_factor_is_round_to_nearest(bits):
    """A diagonal U moves nothing, so the codes, scales and zero points are
    the plain quantizer's, bit for bit."""
    W = S.skewed_weights(10, 384, 40 + bits)
    U = np.diag(np.linspace(0.5, 2.0, 384)).astype(np.float32)
    q, s, z = oracle.gptq_columns(W, U, bits)
    q0, s0, z0 = oracle.quantize(W, bits)
    assert np.array_equal(q, q0) and np.array_equal(s.view(np.uint32), s0.view(np.uint32))
    assert np.array_equal(z, z0)


def exact_case(bits, n=32, k=256, seed=5):
    """Weights on a grid of s/4 with s = 2^-bits fixed in every group by two
    columns that sit on the group's ends and never move (p = 0: lo = -z s,
    p = 1: hi = (maxq - z) s); a sparse factor with U_ii in {1/2, 1, 2} and
    couplings i -> i + 64 inside a group and i -> i + 128 into the next group,
    each in {+-1/4, +-1/2}.  Every product and sum of either column pass is
    then exact in fp32 (at most three levels of moves, 20 significant bits)."""
    g = np.random.Generator(np.random.PCG64(seed))
    maxq = 2 ** bits - 1
    s = 2.0 ** -bits
    z = 2 ** (bits - 2) if bits > 2 else 1
    lo, hi = -z * s, (maxq - z) * s
    steps = g.integers(round(4 * lo / s) + 4, round(4 * hi / s) - 3, size=(n, k))
    W = (steps * (s / 4)).astype(np.float32)
    sent = np.zeros(k, bool)
    for g0 in range(0, k, 128):
        W[:, g0] = lo
        W[:, g0 + 1] = hi
        sent[g0:g0 + 2] = True
    U = np.zeros((k, k), np.float32)
    U[np.arange(k), np.arange(k)] = g.choice([0.5, 1.0, 2.0], size=k)
    U[sent, sent] = 1.0
    vals = np.array([-0.5, -0.25, 0.25, 0.5], np.float32)
    for i in range(k):
        if sent[i]:
            continue
        if i % 128 < 64 and not sent[i + 64]:
            U[i, i + 64] = g.choice(vals)
        if i + 128 < k and not sent[i + 128]:
            U[i, i + 128] = g.choice(vals)
    assert np.all(np.abs(W) <= max(abs(lo), abs(hi)))
    return W, U


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_exact_inputs_agree_with_the_fp64_pass(bits):
    """With exact arithmetic the lazy blocks (later columns moved once per
    block) and the immediate updates reach the same codes, scales and zero
    points, so every step and index of the fp32 pass is that of the
    algorithm."""
    W, U = exact_case(bits)
    q, s, z = oracle.gptq_columns(W, U, bits)
    q64, s64, z64 = G.gptq_columns64(W, U, bits)
    assert np.array_equal(s, s64) and np.array_equal(z, z64)
    assert np.array_equal(q, q64), (q != q64).sum()
    # the moves did change codes against round-to-nearest
    q0, _, _ = oracle.quantize(W, bits)
    assert (q != q0).sum() > 20


@pytest.mark.parametrize("bits", [3, 4, 8])
def test_agrees_with_the_fp64_pass_on_correlated_hessians(bits):
    """fp32 weights, fused updates and lazy blocks change only codes whose
    pre-rounding value sits near a rounding boundary: almost every code equals
    the fp64 pass's and the layer loss matches."""
    k = 512
    H = S.gptq_hessian(k, 60 + bits)
    W = S.skewed_weights(24, k, 61 + bits)
    q, s, z, U = G.gptq32(W, H, bits)
    qr, sr, zr, Ur = G.gptq(W, H, bits)
    assert np.array_equal(U, Ur)
    agree = (q == qr).mean()
    l32 = G.proxy_loss(W, oracle.dequantize(q, s, z), H)
    l64 = G.proxy_loss(W, oracle.dequantize(qr, sr, zr), H)
    assert agree >= 0.995, agree
    assert abs(l32 - l64) <= 0.01 * l64, (l32, l64)


def test_dead_inputs_are_zero_columns():
    k = 256
    H = S.gptq_hessian(k, 70)
    H[9, :] = 0.0
    H[:, 9] = 0.0
    W = S.skewed_weights(6, k, 71)
    q, s, z, _ = G.gptq32(W, H, 4)
    assert np.all(oracle.dequantize(q, s, z)[:, 9] == 0.0)
