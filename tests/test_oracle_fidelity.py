"""Pins for the oracle's EAR / KL reductions and row log-sum-exp (CPU only).

Closed forms, invariants (identity, symmetry, shift), the total-variation
identity EAR = 1 - TV, Pinsker's inequality, and scipy's logsumexp / entropy
as library routines.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp, softmax
from scipy.stats import entropy

import slq_synth as S

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_worked_values.json")))


def test_identical_distributions(orc):
    a, _ = S.fidelity_logits(4, 5000, 0.0, 1)
    ear, kl, means = orc.ear_kl(a, a)
    assert np.allclose(ear, 1.0, atol=1e-12) and np.allclose(kl, 0.0, atol=1e-15)
    assert abs(means[0] - 1.0) < 1e-12 and abs(means[1]) < 1e-15


def test_two_token_closed_form(orc):
    a = np.array([[0.0, 0.0]], np.float32)
    b = np.array([[math.log(3.0), 0.0]], np.float32)
    ear, kl, _ = orc.ear_kl(a, b)
    # p = (1/2, 1/2), q = (3/4, 1/4)
    b0 = float(b[0, 0])   # ln 3 rounded to fp32
    q0 = math.exp(b0) / (math.exp(b0) + 1.0)
    assert abs(ear[0] - (0.5 + (1 - q0))) < 1e-15
    assert abs(ear[0] - 0.75) < 1e-7
    assert abs(kl[0] - 0.5 * math.log(4.0 / 3.0)) < 1e-7
    assert abs(0.5 * math.log(4.0 / 3.0) - 0.1438410362) < 1e-10


def test_against_library_routines_and_identities(orc):
    g = np.random.Generator(np.random.PCG64(5))
    a = (g.standard_normal((6, 300)) * 2).astype(np.float32)
    b = (a + g.standard_normal((6, 300)) * 0.3).astype(np.float32)
    ear, kl, means = orc.ear_kl(a, b)
    p = softmax(a.astype(np.float64), axis=1)
    q = softmax(b.astype(np.float64), axis=1)
    assert np.allclose(ear, np.minimum(p, q).sum(1), atol=1e-13)
    assert np.allclose(ear, 1 - 0.5 * np.abs(p - q).sum(1), atol=1e-13)
    assert np.allclose(kl, entropy(p, q, axis=1), atol=1e-13)
    assert ((1 - ear) <= np.sqrt(kl / 2) + 1e-15).all() and (ear <= 1 + 1e-15).all()
    assert abs(means[0] - ear.mean()) < 1e-15 and abs(means[1] - kl.mean()) < 1e-15
    ear2, kl2, _ = orc.ear_kl(b, a)
    assert np.allclose(ear, ear2, atol=1e-14)          # EAR is symmetric
    assert not np.allclose(kl, kl2, atol=1e-6)         # KL is not
    assert np.allclose(orc.row_lse(a), logsumexp(a.astype(np.float64), axis=1), atol=1e-12)


def test_shift_invariance(orc):
    g = np.random.Generator(np.random.PCG64(6))
    # multiples of 2^-10 in +-16 stay exact after adding 1000 in fp32
    a = (np.round(g.standard_normal((3, 2000)) * 3 * 1024) / 1024).astype(np.float32)
    b = (np.round((a + g.standard_normal((3, 2000)) * 0.1) * 1024) / 1024).astype(np.float32)
    e0, k0, _ = orc.ear_kl(a, b)
    e1, k1, _ = orc.ear_kl(a + np.float32(1000.0), b - np.float32(1000.0))
    assert np.allclose(e0, e1, atol=1e-12) and np.allclose(k0, k1, atol=1e-12)


def test_disjoint_support_gives_zero_ear(orc):
    a = np.array([[50.0, -50.0, -50.0]], np.float32)
    b = np.array([[-50.0, -50.0, 50.0]], np.float32)
    ear, kl, _ = orc.ear_kl(a, b)
    assert ear[0] < 1e-30 and kl[0] > 99.0


@pytest.mark.parametrize("sigma", [0.01, 0.05])
def test_small_noise_asymptotics(orc, sigma):
    """First order in sigma, with i.i.d. noise n_v and its p-mean nbar:
    1 - EAR ~ E sum_v p_v |n_v - nbar| / 2, where n_v - nbar has variance
    sigma^2 (1 - 2 p_v + sum p^2), and KL ~ sigma^2 (1 - sum p^2) / 2."""
    a, b = S.fidelity_logits(16, 20000, sigma, 7)
    ear, kl, _ = orc.ear_kl(a, b)
    p = softmax(a.astype(np.float64), axis=1)
    sp2 = (p ** 2).sum(1, keepdims=True)
    tau = sigma * np.sqrt(1 - 2 * p + sp2)
    want_tv = 0.5 * (p * tau * math.sqrt(2 / math.pi)).sum(1)
    want_kl = 0.5 * sigma ** 2 * (1 - sp2[:, 0])
    assert abs((1 - ear).mean() / want_tv.mean() - 1) < 0.1
    assert abs(kl.mean() / want_kl.mean() - 1) < 0.1


def test_ear_interpretation_from_pages(orc):
    """The pages read EAR 0.99 as 99% agreement: EAR is the probability that
    the two models emit the same token under the best coupling, i.e. 1 - TV.
    Two distributions that agree on 99% of their mass (q moves 1% of p's mass
    from token 0 to token 1; and a 4-token case) give EAR = 0.99 to rounding,
    and the same agreement computed by coupling (the mass both put on each
    token) matches, within the fp32 rounding of the logits."""
    v = GOLDEN["ear_interpretation"]
    cases = [(np.array([0.5, 0.5]), np.array([0.49, 0.51])),
             (np.array([0.4, 0.3, 0.2, 0.1]), np.array([0.39, 0.3, 0.2, 0.11]))]
    for p, q in cases:
        a = np.log(p)[None, :]
        b = np.log(q)[None, :]
        ear, kl, _ = orc.ear_kl(a, b)
        agreement = np.minimum(p, q).sum()          # coupled mass on equal tokens
        assert abs(agreement - v["agreement"]) < 1e-12
        # the logits are fp32: log p rounds at ~6e-8 relative
        assert abs(ear[0] - v["ear"]) < 1e-7, (ear[0], v["ear"])
        assert abs(ear[0] - (1 - 0.5 * np.abs(p - q).sum())) < 1e-7
