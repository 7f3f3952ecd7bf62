"""Pins of the oracle's top-K EAR / top-K KL (gist.science summary,
Methodology 2: EAR summed over the top-K tokens of each position; SLQ README,
Evaluation: top-K KL), at a temperature.

Readings: the top-K set is the K largest reference probabilities (= largest
reference logits), ties to the lower token index; no renormalization over the
set; temperature T divides both logit rows before the softmax."""
import numpy as np
import pytest

import oracle
import slq_synth as S


def brute(a, b, k, T):
    """numpy reference: library sort for the selection, library softmax."""
    a64, b64 = a.astype(np.float64) / T, b.astype(np.float64) / T
    ear, kl = [], []
    for r in range(a.shape[0]):
        lp = a64[r] - np.logaddexp.reduce(a64[r])
        lq = b64[r] - np.logaddexp.reduce(b64[r])
        order = np.lexsort((np.arange(a.shape[1]), -a[r].astype(np.float64)))[:k]
        p, q = np.exp(lp[order]), np.exp(lq[order])
        ear.append(np.minimum(p, q).sum())
        kl.append((p * (lp[order] - lq[order])).sum())
    return np.array(ear), np.array(kl)


def test_full_vocab_is_the_full_ear_kl():
    a, b = S.fidelity_logits(6, 3000, 0.05, 11)
    e1, k1, m1 = oracle.ear_kl_topk(a, b, 3000, 1.0)
    e0, k0, m0 = oracle.ear_kl(a, b)
    np.testing.assert_allclose(e1, e0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(k1, k0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(m1, m0, rtol=0, atol=1e-12)


@pytest.mark.parametrize("k", [1, 3, 10, 37])
@pytest.mark.parametrize("T", [0.5, 1.0, 2.0])
def test_brute_force_small(k, T):
    rng = np.random.default_rng(100 + k)
    a = rng.normal(0, 3, (5, 61)).astype(np.float32)
    a[:, 7] = a[:, 3]                      # exact ties inside the top set
    b = (a + rng.normal(0, 0.3, a.shape)).astype(np.float32)
    e, kl, m = oracle.ear_kl_topk(a, b, k, T)
    eb, kb = brute(a, b, k, T)
    np.testing.assert_allclose(e, eb, rtol=0, atol=1e-13)
    np.testing.assert_allclose(kl, kb, rtol=0, atol=1e-13)
    assert abs(m[0] - eb.mean()) < 1e-13 and abs(m[1] - kb.mean()) < 1e-13


def test_identical_models():
    """q = p: KL is exactly 0 and EAR is the top-K probability mass of p."""
    a, _ = S.fidelity_logits(4, 2000, 0.1, 5)
    for k in (1, 10, 2000):
        e, kl, _ = oracle.ear_kl_topk(a, a, k, 1.0)
        assert np.all(kl == 0.0)
        srt = np.sort(a.astype(np.float64), axis=1)[:, ::-1]
        lse = np.logaddexp.reduce(a.astype(np.float64), axis=1)
        mass = np.exp(srt[:, :k] - lse[:, None]).sum(axis=1)
        np.testing.assert_allclose(e, mass, rtol=1e-13)
    e, _, _ = oracle.ear_kl_topk(a, a, 2000, 1.0)
    np.testing.assert_allclose(e, 1.0, rtol=0, atol=1e-12)


def test_ties_take_the_lower_index():
    """Equal logits: the set is the first K tokens; p = 1/V on each."""
    V, k = 50, 7
    a = np.zeros((1, V), np.float32)
    b = np.linspace(-1, 1, V, dtype=np.float32)[None, :]
    e, kl, _ = oracle.ear_kl_topk(a, b, k, 1.0)
    q = np.exp(b[0].astype(np.float64) - np.logaddexp.reduce(b[0].astype(np.float64)))
    p = 1.0 / V
    assert abs(e[0] - np.minimum(p, q[:k]).sum()) < 1e-15
    assert abs(kl[0] - (p * (np.log(p) - np.log(q[:k]))).sum()) < 1e-15


def test_two_token_closed_form_with_temperature():
    """V = 2, K = 1: p0 = 1 / (1 + exp(-x/T)), q0 = 1 / (1 + exp(-y/T))."""
    for x, y, T in ((1.5, 1.0, 1.0), (2.0, 3.0, 0.5), (0.25, -0.5, 3.0)):
        a = np.array([[x, 0.0]], np.float32)
        b = np.array([[y, 0.0]], np.float32)
        e, kl, _ = oracle.ear_kl_topk(a, b, 1, T)
        p0 = 1.0 / (1.0 + np.exp(-np.float64(np.float32(x)) / T))
        q0 = 1.0 / (1.0 + np.exp(-np.float64(np.float32(y)) / T))
        assert abs(e[0] - min(p0, q0)) < 1e-15
        assert abs(kl[0] - p0 * (np.log(p0) - np.log(q0))) < 1e-14


def test_shift_invariance():
    """Adding a constant to a row of logits changes neither distribution (logits
    on a 1/256 grid, so the fp32 shifts below are exact)."""
    a, b = S.fidelity_logits(3, 1000, 0.05, 8)
    a = (np.round(a * 256) / 256).astype(np.float32)
    b = (np.round(b * 256) / 256).astype(np.float32)
    e0, k0, _ = oracle.ear_kl_topk(a, b, 10, 1.0)
    e1, k1, _ = oracle.ear_kl_topk(a + np.float32(64.0), b - np.float32(32.0), 10, 1.0)
    np.testing.assert_allclose(e1, e0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(k1, k0, rtol=0, atol=1e-12)


def test_ear_grows_with_k():
    a, b = S.fidelity_logits(4, 1500, 0.2, 9)
    prev = np.zeros(4)
    for k in (1, 2, 5, 10, 100, 1500):
        e, _, _ = oracle.ear_kl_topk(a, b, k, 1.0)
        assert np.all(e >= prev - 1e-15)
        prev = e
