"""GPU GPTQ against the fp64 oracle (published algorithm: Frantar et al., ICLR
2023; named by the SLQ README, Pipeline, as the code-choice step).

The inverse-Hessian factor U is compared in fp64.  With H = c I no error is
propagated and the codes are the plain quantizer's, bit for bit.  Otherwise
the column loop runs in fp32 on the GPU and in fp64 in the oracle, so a few
codes near a rounding boundary may differ: the test bounds their share and
compares the layer-output loss tr((W - W_hat) H (W - W_hat)^T)."""
import numpy as np
import pytest
import torch

import oracle
import slq_synth as S
import weight_only_mixed_amd as slq
from oracle import gptq as G
from tests.gpu_util import gpu, host_packed, say

pytestmark = pytest.mark.gpu


def gpu_gptq(W, H, bits, with_u=False):
    pw, U = slq.slq_gptq_quantize(gpu(W), gpu(H), bits, with_u=with_u)
    codes, scales, zeros = host_packed(pw)
    q = oracle.unpack(codes, W.shape[1], bits)
    return q, scales, zeros, (U.cpu().numpy() if with_u else None)


@pytest.mark.parametrize("k", [128, 512, 1024])
def test_inverse_factor(k):
    H = S.gptq_hessian(k, 5 + k)
    H[3, :] = 0.0
    H[:, 3] = 0.0                    # a dead input
    W = S.skewed_weights(8, k, 6)
    _, _, _, U = gpu_gptq(W, H, 4, with_u=True)
    Hp, _ = G.prepare_hessian(H, W)
    U_ref = G.upper_inverse_factor(Hp)
    err = np.abs(U - U_ref).max() / np.abs(U_ref).max()
    say(f"U k={k}: max rel err {err:.2e}")
    assert err < 1e-9 and np.all(np.tril(U, -1) == 0)


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_identity_hessian_is_round_to_nearest(bits):
    W = S.skewed_weights(70, 384, 9 + bits, row_offset_std=0.005)
    q, s, z, _ = gpu_gptq(W, (3.0 * np.eye(384)).astype(np.float32), bits)
    q0, s0, z0 = oracle.quantize(W, bits)
    assert np.array_equal(s.view(np.uint32), s0.view(np.uint32))
    assert np.array_equal(z, z0) and np.array_equal(q, q0)


@pytest.mark.parametrize("bits", [3, 4, 8])
def test_against_oracle(bits):
    n, k = 96, 1024
    H = S.gptq_hessian(k, 40 + bits)
    W = S.skewed_weights(n, k, 41 + bits)
    q, s, z, _ = gpu_gptq(W, H, bits)
    qr, sr, zr, _ = G.gptq(W, H, bits)
    agree = (q == qr).mean()
    l_gpu = G.proxy_loss(W, oracle.dequantize(q, s, z), H)
    l_ref = G.proxy_loss(W, oracle.dequantize(qr, sr, zr), H)
    q0, s0, z0 = oracle.quantize(W, bits)
    l_rtn = G.proxy_loss(W, oracle.dequantize(q0, s0, z0), H)
    say(f"gptq bits={bits}: codes agree {agree:.4f}, loss gpu {l_gpu:.4g} oracle {l_ref:.4g} "
        f"rtn {l_rtn:.4g}")
    assert agree >= 0.99
    assert abs(l_gpu - l_ref) <= 0.01 * l_ref
    assert l_gpu < 0.6 * l_rtn


def test_dead_input_and_full_layer():
    k = 4096
    H = S.gptq_hessian(k, 77, tokens=2 * k)
    H[100, :] = 0.0
    H[:, 100] = 0.0
    W = S.skewed_weights(512, k, 78)
    q, s, z, _ = gpu_gptq(W, H, 4)
    wh = oracle.dequantize(q, s, z)
    assert np.all(wh[:, 100] == 0.0)
    q0, s0, z0 = oracle.quantize(W, 4)
    l_gpu = G.proxy_loss(W, wh, H)
    l_rtn = G.proxy_loss(W, oracle.dequantize(q0, s0, z0), H)
    say(f"gptq 512x4096: loss {l_gpu:.4g} vs rtn {l_rtn:.4g}")
    assert l_gpu < 0.6 * l_rtn


def test_full_q_layer_sampled_rows():
    """Llama-3-8B q projection (4096 x 4096) with a 4096^2 Hessian: rows are
    independent given H, so the oracle runs on 24 sampled rows of the layer
    the GPU quantized whole."""
    k = 4096
    H = S.gptq_hessian(k, 91, tokens=2 * k)
    W = S.skewed_weights(4096, k, 92, row_offset_std=0.005)
    q, s, z, _ = gpu_gptq(W, H, 4)
    rows = np.random.default_rng(93).choice(4096, 24, replace=False)
    qr, sr, zr, _ = G.gptq(W[rows], H, 4)
    agree = (q[rows] == qr).mean()
    l_gpu = G.proxy_loss(W[rows], oracle.dequantize(q[rows], s[rows], z[rows]), H)
    l_ref = G.proxy_loss(W[rows], oracle.dequantize(qr, sr, zr), H)
    say(f"gptq 4096x4096 sampled: codes agree {agree:.4f}, loss {l_gpu:.4g} vs {l_ref:.4g}")
    assert agree >= 0.99 and abs(l_gpu - l_ref) <= 0.01 * l_ref
