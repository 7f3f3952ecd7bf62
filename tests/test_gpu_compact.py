"""GPU parity of the compact metadata layout (SLQ README, Search: 0.156 bits
per parameter of scale and zero point, 20 bits per 128-group): quantize/pack
bit-exact against the oracle (codes, binary16 scale bits, packed zero points),
reconstruction bit-exact, and every matmul path within the matmul tolerance of
the oracle's product on the compact reconstruction."""
import numpy as np
import pytest
import torch

import oracle
import slq_synth as S
import weight_only_mixed_amd as slq
from tests.gpu_util import assert_gemm_close, gpu, say, x_gpu
from tests.test_gpu_quantize import edge_weights

pytestmark = pytest.mark.gpu

BITS = [2, 3, 4, 5, 6, 7, 8]


def pack_compact(W, bits, sym=False):
    pw = slq.slq_quantize_pack(gpu(W), bits, grid=slq.SLQ_SYM if sym else slq.SLQ_ASYM,
                               meta=slq.SLQ_META_COMPACT)
    torch.cuda.synchronize()
    return pw


def oracle_compact(W, bits, sym=False):
    q, s16, z = oracle.quantize_compact(W, bits, symmetric=sym)
    zp = oracle.pack_zeros(z, bits)
    return q, s16, zp


@pytest.mark.parametrize("bits", BITS)
def test_quantize_pack_bit_exact(bits):
    for (n, k) in [(1, 128), (7, 384), (33, 256), (64, 1024), (300, 4096)]:
        for sym in (False, True):
            W = edge_weights(n, k, 3 * bits + n)
            say(f"compact quantize bits={bits} {n}x{k} sym={sym}")
            pw = pack_compact(W, bits, sym)
            q, s16, zp = oracle_compact(W, bits, sym)
            assert np.array_equal(pw.codes.cpu().numpy().view(np.uint32), oracle.pack(q, bits))
            assert np.array_equal(pw.scales.cpu().numpy().view(np.uint16), s16.ravel())
            assert np.array_equal(pw.zeros.cpu().numpy(), zp), (bits, n, k, sym)
            wh = slq.slq_dequantize(pw).cpu().numpy()
            assert np.array_equal(wh.view(np.uint32),
                                  oracle.dequantize_compact(q, s16, zp, bits).view(np.uint32))


def test_sizes():
    L = slq.lib()
    assert L.slq_scales_bytes(10, 1024, 1) == 10 * 8 * 2
    assert L.slq_zeros_bytes(10, 1024, 4, 1) == 40 and L.slq_zeros_bytes(7, 384, 3, 1) == 11
    assert L.slq_zeros_bytes(10, 1024, 5, 1) == 80 and L.slq_scales_bytes(10, 1024, 0) == 320


@pytest.mark.parametrize("bits", BITS)
def test_matmul_paths(bits):
    """Decode (vector and scalar metadata staging, per-lane activations, the
    row-split kernel) and prefill, all reading the compact layout."""
    cases = [(300, 1024, (1, 8, 16, 17, 64)), (50, 384, (1, 5, 16, 40)),
             (70, 8192, (1, 8, 16, 33, 64)), (256, 640, (65, 129))]
    for (n, k, ms) in cases:
        W = S.skewed_weights(n, k, 11 * bits + n, row_offset_std=0.005)
        pw = pack_compact(W, bits)
        q, s16, zp = oracle_compact(W, bits)
        wh = oracle.dequantize_compact(q, s16, zp, bits)
        for m in ms:
            say(f"compact matmul bits={bits} m={m} {n}x{k}: {slq.kernel_name(m, pw)}")
            x = S.activations_bf16(m, k, m + n + bits)
            y = slq.slq_dequant_gemm(x_gpu(x), pw).cpu().numpy()
            yr, br = oracle.gemm(x, wh)
            assert_gemm_close(y, yr, br, what=f"compact b{bits} m{m} {n}x{k}")


@pytest.mark.parametrize("bits", BITS)
def test_prefill_wide_and_split_compact(bits):
    """The wide-tile prefill kernel and its split-k form reading the compact
    layout: split k compared in full, the wide grid on sampled outputs plus its
    whole last row and column."""
    n, k, m = 300, 640, 1100
    W = S.skewed_weights(n, k, 17 * bits, row_offset_std=0.005)
    pw = pack_compact(W, bits)
    assert slq.kernel_name(m, pw).startswith("slq::gemm_wide_kernel") and slq.gemm_workspace_bytes(m, pw) > 0
    q, s16, zp = oracle_compact(W, bits)
    wh = oracle.dequantize_compact(q, s16, zp, bits)
    x = S.activations_bf16(m, k, 5 * bits)
    y = slq.slq_dequant_gemm(x_gpu(x), pw).cpu().numpy()
    yr, br = oracle.gemm(x, wh)
    assert_gemm_close(y, yr, br, what=f"compact split b{bits}")
    n, k, m = 16130, 256, 4095
    W = S.skewed_weights(n, k, 19 * bits, row_offset_std=0.005)
    pw = pack_compact(W, bits)
    assert slq.kernel_name(m, pw).startswith("slq::gemm_wide_kernel") and slq.gemm_workspace_bytes(m, pw) == 0
    q, s16, zp = oracle_compact(W, bits)
    wh = oracle.dequantize_compact(q, s16, zp, bits)
    x = S.activations_bf16(m, k, 7 * bits)
    yd = slq.slq_dequant_gemm(x_gpu(x), pw)
    g = np.random.default_rng(bits)
    mi = np.concatenate([g.integers(0, m, 2000), np.full(n, m - 1), np.arange(m)]).astype(np.int64)
    ni = np.concatenate([g.integers(0, n, 2000), np.arange(n), np.full(m, n - 1)]).astype(np.int64)
    ys = yd[torch.from_numpy(mi).to(yd.device), torch.from_numpy(ni).to(yd.device)].cpu().numpy()
    yr, br = oracle.gemm_pairs(x, wh, mi, ni)
    assert_gemm_close(ys, yr, br, what=f"compact wide b{bits}")


def test_one_hot_exact_and_zero_rows():
    n, k = 40, 512
    W = S.skewed_weights(n, k, 77)
    W[7] = 0.0
    for bits in (3, 4, 8):
        pw = pack_compact(W, bits)
        q, s16, zp = oracle_compact(W, bits)
        wh = oracle.dequantize_compact(q, s16, zp, bits)
        for k0 in (0, 127, 300):
            xb = np.zeros((1, k), np.uint16)
            xb[0, k0] = 0x3F80
            y = slq.slq_dequant_gemm(x_gpu(xb), pw).cpu().numpy()
            assert np.array_equal(y[0], wh[:, k0]), (bits, k0)
        xb = S.activations_bf16(16, k, 5)
        y = slq.slq_dequant_gemm(x_gpu(xb), pw).cpu().numpy()
        assert (y[:, 7] == 0).all()


def test_quant_error_compact():
    W = S.skewed_weights(128, 1024, 9)
    for bits in (3, 4, 6):
        pw = pack_compact(W, bits)
        out = slq.slq_quant_error(gpu(W), pw).cpu().numpy()
        q, s16, zp = oracle_compact(W, bits)
        wh = oracle.dequantize_compact(q, s16, zp, bits)
        sv = np.vectorize(oracle.f16_value)(s16).astype(np.float32)
        sse, s2 = oracle.quant_error(W, wh, sv)
        assert abs(out[0] - sse) <= 1e-9 * sse and abs(out[1] - s2) <= 1e-12 * s2


@pytest.mark.parametrize("bits", [3, 4, 8])
def test_full_sweep_shapes_bit_exact(bits):
    """Compact quantize/pack at the decode sweep's gate/up and down shapes."""
    for (n, k) in [(14336, 4096), (4096, 14336)]:
        W = S.skewed_weights(n, k, 500 + bits, row_offset_std=0.005)
        pw = pack_compact(W, bits)
        q, s16, zp = oracle_compact(W, bits)
        assert np.array_equal(pw.codes.cpu().numpy().view(np.uint32), oracle.pack(q, bits))
        assert np.array_equal(pw.scales.cpu().numpy().view(np.uint16), s16.ravel())
        assert np.array_equal(pw.zeros.cpu().numpy(), zp)
