"""GPU parity of quantize/pack and reconstruction: bit-exact against the oracle
on codes (packed words), scales and zero points, for every width 2..8 and both
grids, from a single group to the full workload layers."""
import numpy as np
import pytest
import torch

import oracle
import slq_synth as S
import weight_only_mixed_amd as slq
from tests.gpu_util import DEV, gpu, host_packed, say

pytestmark = pytest.mark.gpu

BITS = [2, 3, 4, 5, 6, 7, 8]


def edge_weights(n, k, seed):
    W = S.skewed_weights(n, k, seed, row_offset_std=0.005)
    if n >= 4:
        W[1] = 0.0                                   # all-zero row
        W[2, :128] = 0.0
        W[2, 5] = 0.7                                # one nonzero in a group
        W[3, 128:256] = np.abs(W[3, 128:256])        # one-signed group
    if n >= 6:
        W[4, :128] = np.linspace(-1, 1, 128, dtype=np.float32)   # exact .5 ties occur
        W[5, :] *= np.float32(1e-30)                 # tiny magnitudes
    return W


def check_exact(W, bits, sym, what):
    Wd = gpu(W)
    pw = slq.slq_quantize_pack(Wd, bits, grid=slq.SLQ_SYM if sym else slq.SLQ_ASYM)
    codes, scales, zeros = host_packed(pw)
    q, s, z = oracle.quantize(W, bits, symmetric=sym)
    words = oracle.pack(q, bits)
    assert np.array_equal(scales.view(np.uint32), s.view(np.uint32)), f"{what}: scales"
    assert np.array_equal(zeros, z), f"{what}: zeros"
    assert np.array_equal(codes, words), f"{what}: codes"
    return pw


@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("bits", BITS)
def test_small_shapes_bit_exact(bits, sym):
    for (n, k) in [(1, 128), (6, 256), (37, 640), (300, 1024)]:
        say(f"quantize bits={bits} sym={sym} n={n} k={k}")
        W = edge_weights(n, k, 100 * bits + n)
        check_exact(W, bits, sym, f"b{bits} {n}x{k}")


@pytest.mark.parametrize("bits", BITS)
def test_dequantize_matches_oracle(bits):
    W = edge_weights(77, 512, 7 + bits)
    pw = slq.slq_quantize_pack(gpu(W), bits)
    wh = slq.slq_dequantize(pw).cpu().numpy()
    q, s, z = oracle.quantize(W, bits)
    ref = oracle.dequantize(q, s, z)
    assert np.array_equal(wh.view(np.uint32), ref.view(np.uint32))


def test_workload_layers_bit_exact():
    """Full-size layers: the single-layer decode case, every Llama-3-8B and
    Llama-3.3-70B projection shape, and the 5120x25600 layer, at the widths
    the workloads use."""
    cases = [((4096, 4096), 4, 0.0, S.seed_for(1))]
    for i, (name, shape) in enumerate(S.LLAMA3_8B_PROJ.items()):
        if name in ("k", "up", "o"):
            continue
        for b in (3, 4, 8):
            cases.append((shape, b, 0.005, S.seed_for(2, 0, i)))
    for i, (name, shape) in enumerate(S.LLAMA33_70B_PROJ.items()):
        if name in ("q", "k", "gate", "up"):
            cases.append((shape, 4 if name != "k" else 6, 0.005, S.seed_for(4, 0, i)))
    cases.append(((25600, 5120), 4, 0.0, S.seed_for(5)))
    for (n, k), b, off, seed in cases:
        say(f"full-size quantize {n}x{k} bits={b}")
        W = S.skewed_weights(n, k, seed, row_offset_std=off)
        check_exact(W, b, False, f"{n}x{k} b{b}")
        del W
        torch.cuda.empty_cache()


def test_repeatable_and_empty():
    W = edge_weights(64, 1024, 3)
    a = host_packed(slq.slq_quantize_pack(gpu(W), 5))
    b = host_packed(slq.slq_quantize_pack(gpu(W), 5))
    assert all(np.array_equal(u, v) for u, v in zip(a, b))
    empty = slq.slq_quantize_pack(torch.empty((0, 256), dtype=torch.float32, device=DEV), 4)
    assert empty.codes.numel() == 0


def test_stream_read_covers_every_word():
    """The read-ceiling probe reads every 16-byte word once: workgroup i's
    fold is the XOR of the 32-bit words of bytes [16 KiB i, 16 KiB (i + 1))."""
    rng = np.random.default_rng(5)
    for nbytes in (16, 4096 * 16 + 48, 3 * 2 ** 20 + 4096):
        words = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
        nf = slq.stream_read_words(nbytes)
        folds = torch.zeros(nf, dtype=torch.int32, device=DEV)
        slq.slq_stream_read(gpu(words), folds)
        got = folds.cpu().numpy().view(np.uint32)
        per = 16384 // 4
        expect = np.array([np.bitwise_xor.reduce(words[i * per:(i + 1) * per]) for i in range(nf)],
                          np.uint32)
        assert np.array_equal(got, expect), nbytes
