"""GPU GPTQ against the oracle (published algorithm: Frantar et al., ICLR
2023, Algorithm 1 with lazy 128-column blocks; named by the SLQ README,
Pipeline paragraph, as the code-choice step).

The factor U is compared in fp64 (a floating-point result: 1e-9 relative).
The column pass runs in fp32 with one rounding per operation in a stated
order on both sides (oracle.c, oracle_gptq_columns; include/slq.h,
slq_gptq_columns), so its integer outputs are compared exactly: codes, scale
bit patterns and zero points.  Given the same fp32 factor the two column
passes must agree bit for bit.  From a Hessian the two sides' factors (fp64,
different routes) may round to fp32 differently in a few entries; the
composed result is then checked by code agreement and layer loss, and
exactly wherever the rounded factors are equal."""
import numpy as np
import pytest
import torch

import oracle
import slq_synth as S
import weight_only_mixed_amd as slq
from oracle import gptq as G
from tests.gpu_util import gpu, host_packed, say

pytestmark = pytest.mark.gpu


def unpacked(pw, k, bits):
    codes, scales, zeros = host_packed(pw)
    return oracle.unpack(codes, k, bits), scales, zeros


def gpu_gptq(W, H, bits, with_u=False):
    pw, U = slq.slq_gptq_quantize(gpu(W), gpu(H), bits, with_u=with_u)
    q, s, z = unpacked(pw, W.shape[1], bits)
    return q, s, z, (U.cpu().numpy() if with_u else None)


def assert_same_codes(got, ref, what):
    q, s, z = got
    qr, sr, zr = ref
    assert np.array_equal(s.view(np.uint32), sr.view(np.uint32)), f"{what}: scales differ"
    assert np.array_equal(z, zr), f"{what}: zero points differ"
    bad = np.argwhere(q != qr)
    assert bad.size == 0, f"{what}: {len(bad)} codes differ, first at {tuple(bad[0])}"


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
    Uf, dead, U64 = slq.slq_gptq_factor(gpu(H), with_u64=True)
    assert np.array_equal(U64.cpu().numpy(), U)
    assert np.array_equal(Uf.cpu().numpy(), U.astype(np.float32))
    assert np.array_equal(dead.cpu().numpy(), G.dead_inputs(H).astype(np.uint8))


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_column_pass_is_exact(bits):
    """Same fp32 factor and dead-input mask on both sides (a seeded synthetic
    factor): codes, scales and zero points equal bit for bit, on a row count
    that leaves a partial update tile and a partial quantization block."""
    n, k = 150, 640
    W = S.skewed_weights(n, k, 100 + bits, row_offset_std=0.005)
    U = S.gptq_factor(k, 101 + bits)
    dead = np.zeros(k, bool)
    dead[[7, 300]] = True
    pw = slq.slq_gptq_columns(gpu(W), gpu(U), bits, dead=gpu(dead.astype(np.uint8)))
    got = unpacked(pw, k, bits)
    ref = oracle.gptq_columns(W, U, bits, dead=dead)
    assert_same_codes(got, ref, f"column pass bits={bits}")
    q0, _, _ = oracle.quantize(W, bits)
    say(f"column pass bits={bits}: exact; {(ref[0] != q0).mean():.3f} of codes moved off round-to-nearest")


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_identity_hessian_is_round_to_nearest(bits):
    W = S.skewed_weights(70, 384, 9 + bits, row_offset_std=0.005)
    q, s, z, _ = gpu_gptq(W, (3.0 * np.eye(384)).astype(np.float32), bits)
    assert_same_codes((q, s, z), oracle.quantize(W, bits), f"identity bits={bits}")


def factor_gap(a, b):
    """Entries where two fp32 factors differ, and the largest difference in
    units of 2^-24 of the factor's largest magnitude (one rounding step of the
    largest entries; small entries that differ by a few of their own ulps count
    well below one)."""
    d = np.abs(a.astype(np.float64) - b.astype(np.float64))
    return int((d > 0).sum()), float(d.max() / (np.abs(b).max() * 2.0 ** -24))


@pytest.mark.parametrize("bits", [3, 4, 8])
def test_against_oracle(bits):
    """From a correlated Hessian.  The factor is floating point: the two sides
    compute it by different fp64 routes (within 1e-9), so its fp32 rounding
    may differ in a few entries by at most one rounding step of the largest
    entries; every other entry is equal.  The column pass is exact given its factor (the test
    above), so codes can differ only through those entries: almost all codes
    are equal, and the layer loss matches to 1e-4."""
    n, k = 96, 1024
    H = S.gptq_hessian(k, 40 + bits)
    W = S.skewed_weights(n, k, 41 + bits)
    Uf, _, _ = slq.slq_gptq_factor(gpu(H))
    q, s, z, _ = gpu_gptq(W, H, bits)
    qr, sr, zr, Ur = G.gptq32(W, H, bits)
    ndiff, gap = factor_gap(Uf.cpu().numpy(), Ur.astype(np.float32))
    agree = (q == qr).mean()
    l_gpu = G.proxy_loss(W, oracle.dequantize(q, s, z), H)
    l_ref = G.proxy_loss(W, oracle.dequantize(qr, sr, zr), H)
    q0, s0, z0 = oracle.quantize(W, bits)
    l_rtn = G.proxy_loss(W, oracle.dequantize(q0, s0, z0), H)
    say(f"gptq bits={bits}: {ndiff} factor entries differ (largest gap {gap:.3f} of 2^-24 max|U|); "
        f"codes agree {agree:.6f}; loss {l_gpu:.6g} vs {l_ref:.6g}, rtn {l_rtn:.4g}")
    assert gap <= 1.0 and ndiff <= 1e-4 * k * k
    if ndiff == 0:
        assert_same_codes((q, s, z), (qr, sr, zr), f"gptq bits={bits}")
    assert agree >= 0.9999
    assert abs(l_gpu - l_ref) <= 1e-4 * l_ref
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


def test_full_layer_column_pass_sampled_rows():
    """Llama-3-8B q projection (4096 x 4096) through the GPU column pass with
    a 4096-input factor: rows are independent given U, so the oracle runs on
    24 sampled rows of the layer the GPU quantized whole; exact."""
    k = 4096
    W = S.skewed_weights(4096, k, 92, row_offset_std=0.005)
    U = S.gptq_factor(k, 93)
    pw = slq.slq_gptq_columns(gpu(W), gpu(U), 4)
    q, s, z = unpacked(pw, k, 4)
    rows = np.random.default_rng(94).choice(4096, 24, replace=False)
    ref = oracle.gptq_columns(W[rows], U, 4)
    assert_same_codes((q[rows], s[rows], z[rows]), ref, "4096x4096 sampled rows")


def test_full_q_layer_from_hessian_sampled_rows():
    """The whole pipeline on the 4096 x 4096 layer with a 4096^2 Hessian: the
    fp32 factors differ in a few entries by at most one rounding step of the
    largest entries, and the codes of 24 sampled rows agree with the oracle's."""
    k = 4096
    H = S.gptq_hessian(k, 91, tokens=2 * k)
    W = S.skewed_weights(4096, k, 92, row_offset_std=0.005)
    Uf, _, _ = slq.slq_gptq_factor(gpu(H))
    q, s, z, _ = gpu_gptq(W, H, 4)
    rows = np.random.default_rng(93).choice(4096, 24, replace=False)
    qr, sr, zr, Ur = G.gptq32(W[rows], H, 4)
    ndiff, gap = factor_gap(Uf.cpu().numpy(), Ur.astype(np.float32))
    agree = (q[rows] == qr).mean()
    say(f"gptq 4096x4096 sampled: {ndiff} factor entries differ (largest gap {gap:.3f} of 2^-24 "
        f"max|U|); codes agree {agree:.6f}")
    assert gap <= 1.0 and ndiff <= 1e-4 * k * k
    if ndiff == 0:
        assert_same_codes((q[rows], s[rows], z[rows]), (qr, sr, zr), "4096x4096 from H")
    assert agree >= 0.9999
