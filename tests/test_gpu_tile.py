"""GPU parity of the 17..64-row decode kernel for large layers
(`gemv_tile_kernel`) against the oracle's fp64 product, within
|y - y_ref| <= 1e-2 * sum_k |x| |w_hat| per output, plus exact pins: one-hot
activations give w_hat exactly, all-zero weight rows give 0, identical
activation rows give identical outputs, repeated calls are bit-identical."""
import numpy as np
import pytest
import torch

import oracle
import slq_synth as S
import weight_only_mixed_amd as slq
from tests.gpu_util import (DEV, assert_gemm_close, gpu, oracle_sampled, sample_pairs, say,
                            x_gpu)

pytestmark = pytest.mark.gpu

BITS = [2, 3, 4, 5, 6, 7, 8]
TILE = "slq::gemv_tile_kernel"


def _splits(m, pw):
    """k-blocks of the decode plan, from the workspace it asks for (tickets,
    then one fp32 partial per k-block and output)."""
    ws = slq.gemm_workspace_bytes(m, pw)
    return (ws - 65536) // (4 * m * pw.n) if ws else 1


def _sampled(y, W, bits, x, count, seed, what):
    m, n = y.shape
    mi, ni = sample_pairs(m, n, count, seed=seed)
    yr, br = oracle_sampled(W, bits, x, mi, ni)
    return assert_gemm_close(y[mi, ni], yr, br, what=what)


@pytest.mark.parametrize("bits", BITS)
def test_tile_kernel_sampled_and_pins(bits):
    """8200 x 4096: one k-block, a ragged last 64-row tile, three all-zero
    weight rows (first, middle, last); m from 17 to 64 (one and two
    activation-row halves, ragged m-tiles)."""
    n, k = 8200, 4096
    W = S.skewed_weights(n, k, 60 + bits, row_offset_std=0.005)
    zero_rows = [0, 4100, n - 1]
    W[zero_rows] = 0.0
    pw = slq.slq_quantize_pack(gpu(W), bits)
    worst = 0.0
    for m in (17, 32, 33, 48, 64):
        name = slq.kernel_name(m, pw)
        say(f"tile bits={bits} m={m} {n}x{k}: {name}")
        assert name.startswith(TILE) and _splits(m, pw) == 1
        x = S.activations_bf16(m, k, 7 * m + bits)
        x[m // 2] = x[0]
        y = slq.slq_dequant_gemm(x_gpu(x), pw)
        y2 = slq.slq_dequant_gemm(x_gpu(x), pw)
        torch.cuda.synchronize()
        assert torch.equal(y, y2)
        yh = y.cpu().numpy()
        assert (yh[:, zero_rows] == 0).all()
        assert np.array_equal(yh[0], yh[m // 2])
        worst = max(worst, _sampled(yh, W, bits, x, 3000, 100 * bits + m, f"tile b{bits} m{m}"))
    q, s, z = oracle.quantize(W, bits)
    wh = oracle.dequantize(q, s, z)
    for m in (20, 64):
        for k0 in (0, 129, k - 1):
            xb = np.zeros((m, k), np.uint16)
            xb[:, k0] = 0x3F80   # bf16 1.0
            y = slq.slq_dequant_gemm(x_gpu(xb), pw).cpu().numpy()
            assert np.array_equal(y, np.broadcast_to(wh[:, k0], (m, n))), (bits, m, k0)
    say(f"tile bits={bits}: worst err/bound {worst:.3e}")


@pytest.mark.parametrize("bits", [3, 5, 6, 8])
def test_tile_kernel_split_k(bits):
    """k split across workgroups, the last workgroup of each row tile adding
    the partials: 2100 x 16384 (128 groups: more than a workgroup's metadata
    stages hold; 5 k-blocks at 20 and 40 rows, where the split also fills
    the chip, 4 at 64 rows) and 5500 x 6144 at 24 rows (2 k-blocks, only to
    fill the chip); ragged row edges; sampled outputs plus the whole last row and
    column; bit-identical repeats; the tickets are back at zero."""
    for (n, k), m, ks in (((2100, 16384), 20, 5), ((2100, 16384), 40, 5), ((2100, 16384), 64, 4),
                          ((5500, 6144), 24, 2)):
        W = S.skewed_weights(n, k, 70 + bits + n, row_offset_std=0.005)
        pw = slq.slq_quantize_pack(gpu(W), bits)
        name = slq.kernel_name(m, pw)
        say(f"tile split bits={bits} m={m} {n}x{k}: {name}")
        assert name.startswith(TILE) and _splits(m, pw) == ks
        x = S.activations_bf16(m, k, 3 * m + bits)
        ws = torch.zeros(slq.gemm_workspace_bytes(m, pw), dtype=torch.uint8, device=DEV)
        y = slq.slq_dequant_gemm(x_gpu(x), pw, ws=ws)
        y2 = slq.slq_dequant_gemm(x_gpu(x), pw, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(y, y2)
        assert int(ws[:65536].sum()) == 0
        yh = y.cpu().numpy()
        g = np.random.default_rng(bits + m)
        mi = np.concatenate([g.integers(0, m, 2000), np.full(n, m - 1), np.arange(m)]).astype(np.int64)
        ni = np.concatenate([g.integers(0, n, 2000), np.arange(n), np.full(m, n - 1)]).astype(np.int64)
        yr, br = oracle_sampled(W, bits, x, mi, ni)
        assert_gemm_close(yh[mi, ni], yr, br, what=f"tile split b{bits} m{m} {n}x{k}")
        del pw, y, y2, ws
        torch.cuda.empty_cache()


@pytest.mark.parametrize("bits", [3, 4, 7])
def test_tile_kernel_compact_metadata(bits):
    """The compact layout (binary16 scales, nibble or byte zero points) read
    by the tile kernel, against the oracle's compact reconstruction."""
    n, k, m = 8200, 4096, 40
    W = S.skewed_weights(n, k, 80 + bits, row_offset_std=0.005)
    pw = slq.slq_quantize_pack(gpu(W), bits, meta=slq.SLQ_META_COMPACT)
    assert slq.kernel_name(m, pw).startswith(TILE)
    q, s16, z = oracle.quantize_compact(W, bits)
    wh = oracle.dequantize_compact(q, s16, oracle.pack_zeros(z, bits), bits)
    x = S.activations_bf16(m, k, 9 + bits)
    yd = slq.slq_dequant_gemm(x_gpu(x), pw)
    mi, ni = sample_pairs(m, n, 3000, seed=bits)
    ys = yd[torch.from_numpy(mi).to(DEV), torch.from_numpy(ni).to(DEV)].cpu().numpy()
    yr, br = oracle.gemm_pairs(x, wh, mi, ni)
    assert_gemm_close(ys, yr, br, what=f"tile compact b{bits}")
