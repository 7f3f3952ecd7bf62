"""GPU parity of top-K EAR / top-K KL at a temperature against the fp64 oracle
within 1e-5 absolute (gist.science summary, Methodology 2; README, Evaluation).

The top-K set is the K largest reference logits with ties to the lower index;
the selection is integer work on the raw logits, so sets with exact ties are
part of the cases and any wrong pick shows as a difference far above 1e-5."""
import numpy as np
import pytest
import torch

import oracle
import slq_synth as S
import weight_only_mixed_amd as slq
from tests.gpu_util import FID_TOL, gpu, say

pytestmark = pytest.mark.gpu


def check(a, b, k, T, what):
    ear, kl, means = slq.slq_ear_kl_topk(gpu(a), gpu(b), k, T)
    torch.cuda.synchronize()
    e_ref, k_ref, m_ref = oracle.ear_kl_topk(a, b, k, T)
    ear, kl, means = ear.cpu().numpy(), kl.cpu().numpy(), means.cpu().numpy()
    de, dk = np.abs(ear - e_ref).max(), np.abs(kl - k_ref).max()
    dm = np.abs(means - m_ref).max()
    say(f"{what} K={k} T={T}: max|dEAR|={de:.2e} max|dKL|={dk:.2e} means {means} vs {m_ref}")
    assert de <= FID_TOL and dk <= FID_TOL and dm <= FID_TOL, (what, k, T)
    return ear, kl, means


@pytest.mark.parametrize("rows,vocab", [(1, 64), (3, 1000), (5, 1003), (7, 4099), (64, 20000)])
@pytest.mark.parametrize("k", [1, 10, 16, 17, 64])
def test_small_shapes(rows, vocab, k):
    a, b = S.fidelity_logits(rows, vocab, 0.1, rows * 7 + vocab + k)
    for T in (1.0, 0.7, 2.0):
        check(a, b, k, T, f"{rows}x{vocab}")


@pytest.mark.parametrize("k", [1, 10, 33, 64])
def test_ties(k):
    """Logits on a coarse grid: many exact ties at and around the K-th place."""
    g = np.random.Generator(np.random.PCG64(17 + k))
    a = (np.round(g.standard_normal((9, 3001)) * 4) / 2).astype(np.float32)
    b = (a + g.standard_normal(a.shape) * 0.2).astype(np.float32)
    a[3] = 0.0                                   # a whole row tied: the first K tokens
    check(a, b, k, 1.0, "ties")
    check(a, b, k, 0.5, "ties")


def test_full_vocabulary_matches_ear_kl():
    a, b = S.fidelity_logits(6, 64, 0.2, 4)
    e1, k1, m1 = slq.slq_ear_kl_topk(gpu(a), gpu(b), 64, 1.0)
    e0, k0, m0 = slq.slq_ear_kl(gpu(a), gpu(b))
    assert np.abs(e1.cpu().numpy() - e0.cpu().numpy()).max() <= FID_TOL
    assert np.abs(k1.cpu().numpy() - k0.cpu().numpy()).max() <= FID_TOL
    check(a, b, 64, 1.0, "K = vocab")


def test_extreme_logits():
    """Large-magnitude logits and a temperature that sharpens them."""
    g = np.random.Generator(np.random.PCG64(5))
    a = (g.standard_normal((4, 5000)) * 30).astype(np.float32)
    b = (a + g.standard_normal(a.shape) * 0.5).astype(np.float32)
    a[0, 100] = 1e4
    check(a, b, 10, 1.0, "extreme")
    check(a, b, 10, 0.25, "extreme")
    check(a - np.float32(500), b + np.float32(500), 10, 3.0, "extreme shifted")


@pytest.mark.parametrize("sigma", S.FIDELITY_SIGMAS)
def test_workload_512x151936_k10(sigma):
    a, b = S.fidelity_logits(S.FIDELITY_ROWS, S.VOCAB, sigma, S.seed_for(6) + int(sigma * 1000))
    ear, kl, means = check(a, b, 10, 1.0, f"512x151936 sigma={sigma}")
    ear2, kl2, means2 = slq.slq_ear_kl_topk(gpu(a), gpu(b), 10, 1.0)
    assert np.array_equal(ear2.cpu().numpy(), ear) and np.array_equal(kl2.cpu().numpy(), kl)
    assert np.array_equal(means2.cpu().numpy(), means)


def test_workload_512x151936_k64_temperature():
    a, b = S.fidelity_logits(S.FIDELITY_ROWS, S.VOCAB, 0.05, S.seed_for(7))
    check(a, b, 64, 0.8, "512x151936")


@pytest.mark.parametrize("order", ["ascending", "descending"])
def test_sorted_rows(order):
    """Rising logits admit every element to the candidate buffers (the most
    cut-backs); falling ones admit almost none after the first."""
    base = np.linspace(-20, 20, 40000, dtype=np.float32)
    a = np.stack([base if order == "ascending" else base[::-1]] * 3)
    b = (a + np.random.Generator(np.random.PCG64(2)).standard_normal(a.shape) * 0.1).astype(np.float32)
    for k in (1, 10, 64):
        check(a, b, k, 1.0, order)


def test_more_rows_than_one_grid_column():
    """70000 rows: more than one launch of the (chunk, row) grid."""
    a, b = S.fidelity_logits(70000, 12, 0.3, 21)
    check(a, b, 5, 1.0, "70000x12")
    ear, kl, means = slq.slq_ear_kl(gpu(a), gpu(b))
    e_ref, k_ref, m_ref = oracle.ear_kl(a, b)
    assert np.abs(ear.cpu().numpy() - e_ref).max() <= FID_TOL
    assert np.abs(kl.cpu().numpy() - k_ref).max() <= FID_TOL
    lse = slq.slq_row_lse(gpu(a)).cpu().numpy()
    assert np.abs(lse - oracle.row_lse(a)).max() <= 1e-6 * max(1.0, np.abs(lse).max())
