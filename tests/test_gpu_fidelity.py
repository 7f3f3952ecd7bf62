"""GPU parity of the fidelity reductions (row log-normalizer, EAR, KL) against
the fp64 oracle within 1e-5 absolute, and of the gamma-squared noise sums."""
import math

import numpy as np
import pytest
import torch

import oracle
import slq_synth as S
import weight_only_mixed_amd as slq
from tests.gpu_util import DEV, FID_TOL, gpu, say

pytestmark = pytest.mark.gpu


def check(a, b, what):
    ear, kl, means = slq.slq_ear_kl(gpu(a), gpu(b))
    torch.cuda.synchronize()
    e_ref, k_ref, m_ref = oracle.ear_kl(a, b)
    ear, kl, means = ear.cpu().numpy(), kl.cpu().numpy(), means.cpu().numpy()
    de, dk = np.abs(ear - e_ref).max(), np.abs(kl - k_ref).max()
    dm = np.abs(means - m_ref).max()
    say(f"{what}: max|dEAR|={de:.2e} max|dKL|={dk:.2e} means {means} vs {m_ref}")
    assert de <= FID_TOL and dk <= FID_TOL and dm <= FID_TOL, what
    return ear, kl, means


@pytest.mark.parametrize("rows,vocab", [(1, 2), (3, 1000), (7, 4099), (64, 20000), (2, 151936)])
def test_small_shapes(rows, vocab):
    for sigma in (0.0, 0.05, 1.0):
        a, b = S.fidelity_logits(rows, vocab, sigma, rows + vocab)
        ear, kl, _ = check(a, b, f"{rows}x{vocab} sigma={sigma}")
        if sigma == 0.0:
            assert np.all(np.abs(ear - 1) <= 1e-6) and np.all(np.abs(kl) <= 1e-6)
    lse = slq.slq_row_lse(gpu(a)).cpu().numpy()
    assert np.abs(lse - oracle.row_lse(a)).max() <= 1e-6 * max(1.0, np.abs(lse).max())


def test_closed_form_and_shift():
    a = np.array([[0.0, 0.0]], np.float32)
    b = np.array([[math.log(3.0), 0.0]], np.float32)
    ear, kl, _ = check(a, b, "two tokens")
    assert abs(ear[0] - 0.75) < 1e-6 and abs(kl[0] - 0.5 * math.log(4 / 3)) < 1e-6
    g = np.random.Generator(np.random.PCG64(3))
    a = (np.round(g.standard_normal((4, 5000)) * 3 * 1024) / 1024).astype(np.float32)
    b = (np.round((a + g.standard_normal((4, 5000)) * 0.1) * 1024) / 1024).astype(np.float32)
    e0, k0, _ = check(a, b, "base")
    e1, k1, _ = check(a + np.float32(1000.0), b - np.float32(1000.0), "shifted")
    assert np.abs(e0 - e1).max() <= 2e-6 and np.abs(k0 - k1).max() <= 2e-6


@pytest.mark.parametrize("sigma", S.FIDELITY_SIGMAS)
def test_workload_512x151936(sigma):
    a, b = S.fidelity_logits(S.FIDELITY_ROWS, S.VOCAB, sigma, S.seed_for(5) + int(sigma * 1000))
    ear, kl, means = check(a, b, f"512x151936 sigma={sigma}")
    # repeatable bit for bit
    ear2, kl2, means2 = slq.slq_ear_kl(gpu(a), gpu(b))
    assert np.array_equal(ear2.cpu().numpy(), ear) and np.array_equal(means2.cpu().numpy(), means)


def _ratio_gpu(W, bits):
    Wd = gpu(W)
    out = {}
    for grid in (slq.SLQ_ASYM, slq.SLQ_SYM):
        pw = slq.slq_quantize_pack(Wd, bits, grid=grid)
        out[grid] = slq.slq_quant_error(Wd, pw).cpu().numpy()
    return out


@pytest.mark.parametrize("bits", [3, 4, 8])
def test_quant_error_matches_oracle(bits):
    W = S.skewed_weights(300, 1024, bits)
    res = _ratio_gpu(W, bits)
    for grid, sym in ((slq.SLQ_ASYM, False), (slq.SLQ_SYM, True)):
        q, s, z = oracle.quantize(W, bits, symmetric=sym)
        sse, s2 = oracle.quant_error(W, oracle.dequantize(q, s, z), s)
        assert abs(res[grid][0] - sse) <= 1e-9 * sse and abs(res[grid][1] - s2) <= 1e-9 * s2


def test_gamma_squared_workload_layer():
    """5120-input x 25600-output skewed layer, INT4 g128, symmetric vs
    asymmetric: measured noise ratio within 5% of the s^2-weighted gamma^2."""
    W = S.skewed_weights(25600, 5120, S.seed_for(5))
    res = _ratio_gpu(W, 4)
    measured = res[slq.SLQ_SYM][0] / res[slq.SLQ_ASYM][0]
    predicted = res[slq.SLQ_SYM][1] / res[slq.SLQ_ASYM][1]
    say(f"gamma^2 law: measured {measured:.4f} predicted {predicted:.4f}")
    assert res[slq.SLQ_ASYM][0] < res[slq.SLQ_SYM][0]
    assert abs(measured / predicted - 1) < 0.05
