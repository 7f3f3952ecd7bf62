"""Pins of the GPTQ oracle (published algorithm: Frantar et al., ICLR 2023,
Algorithm 1 with the Cholesky form; named by the SLQ README, Pipeline, as the
code-choice step).  The pages do not define it, so these pin it by properties
that any correct implementation has."""
import numpy as np
import pytest

import oracle
import slq_synth as S
from oracle import gptq as G


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_identity_hessian_is_round_to_nearest(bits):
    """With H = c I the inverse factor is diagonal, so no error is propagated
    and every code, scale and zero point is the plain quantizer's."""
    W = S.skewed_weights(12, 384, 3 + bits)
    q, s, z, U = G.gptq(W, 5.0 * np.eye(384), bits)
    q0, s0, z0 = oracle.quantize(W, bits)
    assert np.array_equal(q, q0) and np.array_equal(s, s0) and np.array_equal(z, z0)
    assert np.allclose(U, np.diag(np.diag(U)))


def test_factor_and_first_update_are_the_closed_form():
    """U^T U = H^-1, and quantizing column 0 moves column j by
    -delta * Hinv[0, j] / Hinv[0, 0] (the optimal-brain-surgeon update)."""
    H = S.gptq_hessian(96, 7)
    W = S.skewed_weights(5, 96, 8)
    Hp, Wp = G.prepare_hessian(H, W)
    U = G.upper_inverse_factor(Hp)
    Hinv = np.linalg.inv(Hp)
    assert np.allclose(U.T @ U, Hinv, rtol=1e-10, atol=1e-12 * np.abs(Hinv).max())
    assert np.allclose(U, np.triu(U))
    delta = 0.37
    upd_chol = delta / U[0, 0] * U[0, 1:]
    upd_obs = delta * Hinv[0, 1:] / Hinv[0, 0]
    np.testing.assert_allclose(upd_chol, upd_obs, rtol=1e-10, atol=1e-14)


@pytest.mark.parametrize("bits", [3, 4])
def test_beats_round_to_nearest_on_correlated_hessians(bits):
    k = 256
    H = S.gptq_hessian(k, 11)
    W = S.skewed_weights(16, k, 12 + bits)
    q, s, z, _ = G.gptq(W, H, bits)
    wh = oracle.dequantize(q, s, z)
    q0, s0, z0 = oracle.quantize(W, bits)
    wh0 = oracle.dequantize(q0, s0, z0)
    l_gptq, l_rtn = G.proxy_loss(W, wh, H), G.proxy_loss(W, wh0, H)
    assert l_gptq < 0.8 * l_rtn, (l_gptq, l_rtn)
    assert q.max() <= 2 ** bits - 1


def test_dead_inputs():
    k = 128
    H = S.gptq_hessian(k, 3)
    H[5, :] = 0.0
    H[:, 5] = 0.0
    W = S.skewed_weights(4, k, 2)
    q, s, z, _ = G.gptq(W, H, 4)
    wh = oracle.dequantize(q, s, z)
    assert np.all(wh[:, 5] == 0.0)


def obs_sequence(W, H, bits, group=128):
    """The same greedy column order by explicit inverse downdates instead of
    the Cholesky rows: after quantizing column i with error d, the remaining
    columns move by -d * Hinv[i, j] / Hinv[i, i], and Hinv loses row and column
    i (its Schur complement): Hinv -= Hinv[:, i] Hinv[i, :] / Hinv[i, i]."""
    Hp, Wp = G.prepare_hessian(H, W)
    Hinv = np.linalg.inv(Hp)
    n, k = Wp.shape
    q = np.zeros((n, k), np.int64)
    maxq = 2 ** bits - 1
    for i in range(k):
        if i % group == 0:
            params = [G.group_params(Wp[r, i:i + group].astype(np.float32), bits) for r in range(n)]
        s = np.array([p[0] for p in params], np.float32)
        z = np.array([p[1] for p in params], np.int64)
        qi = np.clip(np.rint(Wp[:, i].astype(np.float32) / s) + z, 0, maxq).astype(np.int64)
        q[:, i] = qi
        d = Wp[:, i] - ((qi - z).astype(np.float32) * s).astype(np.float64)
        Wp[:, i + 1:] -= np.outer(d / Hinv[i, i], Hinv[i, i + 1:])
        Hinv = Hinv - np.outer(Hinv[:, i], Hinv[i, :]) / Hinv[i, i]
    return q


@pytest.mark.parametrize("bits", [3, 4])
def test_matches_explicit_inverse_sequence(bits):
    """Codes equal to the explicit-inverse formulation (two groups, so the
    second group's parameters come from weights the first group moved)."""
    H = S.gptq_hessian(256, 21 + bits)
    W = S.skewed_weights(6, 256, 30 + bits)
    q, _, _, _ = G.gptq(W, H, bits)
    q_ref = obs_sequence(W, H, bits)
    assert (q != q_ref).mean() <= 0.002, (q != q_ref).mean()
