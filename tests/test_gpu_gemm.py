"""GPU parity of the weight-only dequantize matmul (decode m <= 64 and prefill
m > 64) against the oracle's fp64 product, within
|y - y_ref| <= 1e-2 * sum_k |x| |w_hat| per output, plus exact pins."""
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


def run(W, bits, x_bits):
    pw = slq.slq_quantize_pack(gpu(W), bits)
    y = slq.slq_dequant_gemm(x_gpu(x_bits), pw)
    torch.cuda.synchronize()
    return y.cpu().numpy(), pw


def full_ref(W, bits, x_bits):
    q, s, z = oracle.quantize(W, bits)
    wh = oracle.dequantize(q, s, z)
    y, b = oracle.gemm(x_bits, wh)
    return y, b, wh


@pytest.mark.parametrize("bits", BITS)
def test_decode_small_shapes(bits):
    # k = 8192 and 8320 (64 and 65 groups) reach the long-k decode variant,
    # with and without whole 4-group metadata vectors
    for (n, k) in [(1, 128), (50, 384), (300, 1024), (1000, 4096), (70, 8192), (130, 8320)]:
        W = S.skewed_weights(n, k, 10 * bits + n, row_offset_std=0.005)
        for m in (1, 3, 8, 16, 17, 32, 64):
            say(f"decode bits={bits} m={m} n={n} k={k}")
            x = S.activations_bf16(m, k, m + n + bits)
            y, _ = run(W, bits, x)
            yr, br, _ = full_ref(W, bits, x)
            assert_gemm_close(y, yr, br, what=f"b{bits} m{m} {n}x{k}")


@pytest.mark.parametrize("bits", BITS)
def test_prefill_small_shapes(bits):
    for (m, n, k) in [(65, 70, 256), (129, 300, 640), (256, 128, 1024)]:
        say(f"prefill bits={bits} m={m} n={n} k={k}")
        W = S.skewed_weights(n, k, 7 * bits + n, row_offset_std=0.005)
        x = S.activations_bf16(m, k, m + bits)
        y, _ = run(W, bits, x)
        yr, br, _ = full_ref(W, bits, x)
        assert_gemm_close(y, yr, br, what=f"b{bits} m{m} {n}x{k}")


@pytest.mark.parametrize("bits", BITS)
def test_prefill_wide_tiles_ragged(bits):
    """Grids of at least 256 tiles of 256 x 256 (the wide-tile kernel) with
    ragged m and n edges; k = 128 is the shortest pipeline (two k steps).
    Sampled outputs plus the whole last row and the whole last column."""
    for (m, n, k) in [(4000, 16000, 128), (4095, 16130, 640)]:
        say(f"prefill wide bits={bits} m={m} n={n} k={k}")
        W = S.skewed_weights(n, k, 11 * bits + k, row_offset_std=0.005)
        x = S.activations_bf16(m, k, m + bits + k)
        pw = slq.slq_quantize_pack(gpu(W), bits)
        assert slq.kernel_name(m, pw).startswith("slq::gemm_wide_kernel")
        y = slq.slq_dequant_gemm(x_gpu(x), pw)
        mi, ni = sample_pairs(m, n, 3000, seed=bits + k)
        mi = np.concatenate([mi, np.full(n, m - 1), np.arange(m)])
        ni = np.concatenate([ni, np.arange(n), np.full(m, n - 1)])
        ys = y[torch.from_numpy(mi).to(DEV), torch.from_numpy(ni).to(DEV)].cpu().numpy()
        yr, br = oracle_sampled(W, bits, x, mi, ni)
        assert_gemm_close(ys, yr, br, what=f"wide b{bits} {m}x{n}x{k}")
        del y, pw
        torch.cuda.empty_cache()


@pytest.mark.parametrize("bits", BITS)
def test_prefill_split_k(bits):
    """Grids of fewer than 256 wide tiles with m >= 1024 split k across
    workgroups (partial tiles in the workspace, summed in split order):
    m*n divisible by 4 and not, uneven last split (k = 640: 10 steps in
    splits of 4, 4, 2), ragged edges.  Every output against the oracle, and
    bit-identical results across calls."""
    for (m, n, k) in [(1100, 700, 640), (1025, 301, 384), (2048, 96, 256)]:
        say(f"prefill split bits={bits} m={m} n={n} k={k}")
        W = S.skewed_weights(n, k, 13 * bits + n, row_offset_std=0.005)
        x = S.activations_bf16(m, k, 3 * m + bits)
        pw = slq.slq_quantize_pack(gpu(W), bits)
        assert slq.kernel_name(m, pw).startswith("slq::gemm_wide_kernel")
        assert slq.gemm_workspace_bytes(m, pw) > 65536
        y = slq.slq_dequant_gemm(x_gpu(x), pw)
        y2 = slq.slq_dequant_gemm(x_gpu(x), pw)
        torch.cuda.synchronize()
        assert torch.equal(y, y2)
        yr, br, _ = full_ref(W, bits, x)
        assert_gemm_close(y.cpu().numpy(), yr, br, what=f"split b{bits} {m}x{n}x{k}")


def test_prefill_rows_beyond_one_grid():
    """More activation rows than one launch grid holds (65535 tiles of 256
    rows): the rows go in chunks; sampled rows on both sides of the chunk
    boundary and the last row against the oracle."""
    m, n, k, bits = 65535 * 256 + 300, 3, 128, 4
    W = S.skewed_weights(n, k, 23, row_offset_std=0.005)
    pw = slq.slq_quantize_pack(gpu(W), bits)
    assert slq.kernel_name(m, pw).startswith("slq::gemm_wide_kernel")
    g = torch.Generator(device=DEV).manual_seed(29)
    x = torch.randn(m, k, device=DEV, generator=g).to(torch.bfloat16)
    y = slq.slq_dequant_gemm(x, pw)
    torch.cuda.synchronize()
    edge = 65535 * 256
    rows = np.concatenate([np.random.default_rng(31).integers(0, m, 500),
                           np.arange(edge - 3, edge + 3), [m - 1]]).astype(np.int64)
    rows_t = torch.from_numpy(rows).to(DEV)
    xs = x[rows_t].view(torch.int16).cpu().numpy().view(np.uint16)
    ys = y[rows_t].cpu().numpy()
    del x, y
    torch.cuda.empty_cache()
    mi = np.repeat(np.arange(len(rows)), n).astype(np.int64)
    ni = np.tile(np.arange(n), len(rows)).astype(np.int64)
    yr, br = oracle_sampled(W, bits, xs, mi, ni)
    assert_gemm_close(ys[mi, ni], yr, br, what="prefill rows beyond one grid")


@pytest.mark.parametrize("bits", BITS)
def test_exact_pins(bits):
    """One-hot activations give w_hat exactly (decode path); zero rows give 0;
    identical activation rows give identical outputs."""
    n, k = 40, 512
    W = S.skewed_weights(n, k, 5 + bits)
    W[7] = 0.0
    q, s, z = oracle.quantize(W, bits)
    wh = oracle.dequantize(q, s, z)
    pw = slq.slq_quantize_pack(gpu(W), bits)
    for k0 in (0, 1, 127, 128, 300, 511):
        for m in (1, 16, 64):
            xb = np.zeros((m, k), np.uint16)
            xb[:, k0] = 0x3F80                     # bf16 1.0
            y = slq.slq_dequant_gemm(x_gpu(xb), pw).cpu().numpy()
            assert np.array_equal(y, np.broadcast_to(wh[:, k0], (m, n))), (bits, k0, m)
    for m in (1, 5, 33, 64, 100):
        xb = S.activations_bf16(m, k, 9)
        xb[m // 2] = xb[0]
        y = slq.slq_dequant_gemm(x_gpu(xb), pw).cpu().numpy()
        assert (y[:, 7] == 0).all()
        assert np.array_equal(y[0], y[m // 2])
    # the same decode pins on the mid-width 33..64-row kernel (ragged last
    # row tile, an all-zero first and last row)
    n2 = 2050
    W2 = S.skewed_weights(n2, k, 6 + bits)
    W2[0] = 0.0
    W2[n2 - 1] = 0.0
    q2, s2, z2 = oracle.quantize(W2, bits)
    wh2 = oracle.dequantize(q2, s2, z2)
    pw2 = slq.slq_quantize_pack(gpu(W2), bits)
    for m in (48, 50, 64):
        assert slq.kernel_name(m, pw2).startswith("slq::gemv_mk_kernel")
        for k0 in (0, 129, 511):
            xb = np.zeros((m, k), np.uint16)
            xb[:, k0] = 0x3F80
            y = slq.slq_dequant_gemm(x_gpu(xb), pw2).cpu().numpy()
            assert np.array_equal(y, np.broadcast_to(wh2[:, k0], (m, n2))), (bits, k0, m)
        xb = S.activations_bf16(m, k, 11)
        xb[m // 2] = xb[0]
        y = slq.slq_dequant_gemm(x_gpu(xb), pw2).cpu().numpy()
        assert (y[:, 0] == 0).all() and (y[:, n2 - 1] == 0).all()
        assert np.array_equal(y[0], y[m // 2])
    # prefill one-hot: within bf16 rounding of w_hat
    xb = np.zeros((96, k), np.uint16)
    xb[:, 300] = 0x3F80
    y = slq.slq_dequant_gemm(x_gpu(xb), pw).cpu().numpy()
    assert np.all(np.abs(y - wh[:, 300]) <= np.abs(wh[:, 300]) * 2 ** -8)


@pytest.mark.parametrize("bits", [3, 8])
def test_decode_plans_whole_k_and_odd_k(bits):
    """Decode plans that hold a layer's whole k range in one workgroup (16-row
    tiles of 16 waves, 64-row tiles of 8 waves, the latter up to the LDS
    ceiling with 63 groups), and layers whose group count is not a multiple of
    4 (metadata staged per group), against the oracle on sampled outputs."""
    cases = [(8192, 8064, (1, 5, 8, 12, 16)), (5000, 7936, (4, 5, 16)), (2000, 4096, (5, 16)),
             (14336, 4096, (12, 16)), (4096, 4096, (12, 16))]
    for (n, k, ms) in cases:
        W = S.skewed_weights(n, k, 41 * bits + n, row_offset_std=0.005)
        pw = slq.slq_quantize_pack(gpu(W), bits)
        for m in ms:
            say(f"decode plan bits={bits} m={m} {n}x{k}: {slq.kernel_name(m, pw)}")
            x = S.activations_bf16(m, k, 3 * m + n)
            y = slq.slq_dequant_gemm(x_gpu(x), pw)
            mi, ni = sample_pairs(m, n, 1500, seed=m + n)
            ys = y[torch.from_numpy(mi).to(DEV), torch.from_numpy(ni).to(DEV)].cpu().numpy()
            yr, br = oracle_sampled(W, bits, x, mi, ni)
            assert_gemm_close(ys, yr, br, what=f"plan b{bits} m{m} {n}x{k}")
        del pw
        torch.cuda.empty_cache()


def test_decode_deterministic_and_workspace_reset():
    n, k = 4096, 14336   # 16 rows on this layer split k four ways
    W = S.skewed_weights(n, k, 1)
    pw = slq.slq_quantize_pack(gpu(W), 4)
    x = x_gpu(S.activations_bf16(16, k, 2))
    nb = slq.gemm_workspace_bytes(16, pw)
    assert nb > 0
    ws = torch.zeros(nb, dtype=torch.uint8, device=DEV)
    y1 = slq.slq_dequant_gemm(x, pw, ws=ws).clone()
    y2 = slq.slq_dequant_gemm(x, pw, ws=ws).clone()
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    # tickets (first 64 KiB of the workspace) are back to zero
    assert int(ws[:65536].sum()) == 0
    # a smaller plan after a larger one reuses the buffer: tickets still valid
    W2 = S.skewed_weights(14336, 4096, 3)
    pw2 = slq.slq_quantize_pack(gpu(W2), 3)
    assert slq.gemm_workspace_bytes(1, pw2) <= nb
    xs = S.activations_bf16(1, 4096, 4)
    y3 = slq.slq_dequant_gemm(x_gpu(xs), pw2, ws=ws).cpu().numpy()
    mi, ni = sample_pairs(1, 14336, 2048, seed=5)
    yr, br = oracle_sampled(W2, 3, xs, mi, ni)
    assert_gemm_close(y3[mi, ni], yr, br, what="reused workspace")
    assert int(ws[:65536].sum()) == 0


def test_single_layer_decode_workload():
    """M=1, 4096x4096, asymmetric INT4 g128: every output against the oracle."""
    W = S.skewed_weights(4096, 4096, S.seed_for(1))
    x = S.activations_bf16(1, 4096, S.seed_for(1) + 1)
    y, _ = run(W, 4, x)
    yr, br, _ = full_ref(W, 4, x)
    r = assert_gemm_close(y, yr, br, what="single layer")
    say(f"single-layer decode max err/bound = {r:.3e}")


def test_decode_sweep_workload_sampled():
    """Llama-3-8B projections x bits {3,4,8} x M {1,8,16} at full size, in the
    launch configuration the bench times; 4096 sampled outputs per point."""
    shapes = {"q": (4096, 4096), "kv": (1024, 4096), "gateup": (14336, 4096), "down": (4096, 14336)}
    worst = 0.0
    for i, (name, (n, k)) in enumerate(shapes.items()):
        W = S.skewed_weights(n, k, S.seed_for(2, 0, i), row_offset_std=0.005)
        Wd = gpu(W)
        for bits in (3, 4, 8):
            pw = slq.slq_quantize_pack(Wd, bits)
            for m in (1, 8, 16):
                say(f"sweep {name} {n}x{k} bits={bits} m={m}")
                x = S.activations_bf16(m, k, S.seed_for(2, m, i))
                y = slq.slq_dequant_gemm(x_gpu(x), pw).cpu().numpy()
                mi, ni = sample_pairs(m, n, 4096, seed=i * 100 + bits * 10 + m)
                yr, br = oracle_sampled(W, bits, x, mi, ni)
                worst = max(worst, assert_gemm_close(y[mi, ni], yr, br, what=f"{name} b{bits} m{m}"))
    say(f"sweep worst err/bound = {worst:.3e}")


def test_mixed_stack_workload_sampled():
    """32 layers x 7 projections of Llama-3-8B shape with the seeded per-layer
    bit map (k/v 7-8, q/o 5-6, MLP 3-4), M in {1, 32, 64}: the bench's recipe
    (one layer of fp32 weights quantized at every layer's widths), sampled
    outputs of all 224 matmuls."""
    bmap = S.mixed_bit_map()
    Ws = {p: S.skewed_weights(*S.LLAMA3_8B_PROJ[p], S.seed_for(3, 0, j), row_offset_std=0.005)
          for j, p in enumerate(S.PROJ_ORDER)}
    Wd = {p: gpu(w) for p, w in Ws.items()}
    xs = {m: {k: S.activations_bf16(m, k, S.seed_for(3, m, k % 97)) for k in (4096, 14336)}
          for m in (1, 32, 64)}
    xd = {m: {k: x_gpu(v) for k, v in d.items()} for m, d in xs.items()}
    refcache = {}
    for layer in range(32):
        say(f"stack layer {layer}: {bmap[layer]}")
        for j, p in enumerate(S.PROJ_ORDER):
            b = bmap[layer][p]
            n, k = S.LLAMA3_8B_PROJ[p]
            pw = slq.slq_quantize_pack(Wd[p], b)
            for m in (1, 32, 64):
                y = slq.slq_dequant_gemm(xd[m][k], pw).cpu().numpy()
                mi, ni = sample_pairs(m, n, 256, seed=layer * 1000 + j * 10 + m)
                key = (p, b, m, layer)
                yr, br = oracle_sampled(Ws[p], b, xs[m][k], mi, ni)
                assert_gemm_close(y[mi, ni], yr, br, what=f"L{layer} {p} b{b} m{m}")
        torch.cuda.empty_cache()


@pytest.mark.parametrize("bits", [4, 6])
def test_prefill_workload_sampled(bits):
    """M=4096 on Llama-3.3-70B projection shapes, 4096 sampled outputs each."""
    x = S.activations_bf16(4096, 8192, S.seed_for(4) + bits)
    x28 = None
    for i, name in enumerate(("q", "k", "gate", "down")):
        n, k = S.LLAMA33_70B_PROJ[name]
        say(f"prefill {name} {n}x{k} bits={bits}")
        W = S.skewed_weights(n, k, S.seed_for(4, 0, i), row_offset_std=0.005)
        if k == 8192:
            xb = x
        else:
            x28 = x28 if x28 is not None else S.activations_bf16(4096, k, S.seed_for(4) + 10 + bits)
            xb = x28
        pw = slq.slq_quantize_pack(gpu(W), bits)
        y = slq.slq_dequant_gemm(x_gpu(xb), pw)
        mi, ni = sample_pairs(4096, n, 4096, seed=bits * 10 + i)
        ys = y[torch.from_numpy(mi).to(DEV), torch.from_numpy(ni).to(DEV)].cpu().numpy()
        yr, br = oracle_sampled(W, bits, xb, mi, ni)
        assert_gemm_close(ys, yr, br, what=f"prefill {name} b{bits}")
        del y, pw, W
        torch.cuda.empty_cache()


def _splits(m, pw):
    """k-blocks of the decode plan, from the workspace it asks for (tickets,
    then one fp32 partial per k-block and output)."""
    ws = slq.gemm_workspace_bytes(m, pw)
    return (ws - 65536) // (4 * m * pw.n) if ws else 1


@pytest.mark.parametrize("bits", [3, 4, 8])
def test_decode_split_tails_and_mid_width_kernel(bits):
    """The split-k tail (the last workgroup of a row block adds the k-blocks'
    partials, several outputs and up to eight partial loads in flight per
    thread) with more than eight and a non-multiple of eight k-blocks, in all
    three decode kernels; and the mid-width 33..64-row kernel with whole and
    uneven k-blocks, a ragged row edge and a trailing group outside its
    two-group ring blocks.  Every output against the oracle, and bit-identical
    results across calls."""
    cases = [((16, 200, 20480), "slq::gemv_kernel", 20),
             ((8, 300, 16384), "slq::gemv_kernel", 13),
             ((40, 256, 32768), "slq::gemv_rows_kernel", 32),
             ((64, 2048, 4096), "slq::gemv_mk_kernel", 8),
             ((60, 3000, 8320), "slq::gemv_mk_kernel", 6),
             ((64, 8191, 1152), "slq::gemv_mk_kernel", 2),
             ((49, 2100, 640), "slq::gemv_mk_kernel", 1),
             ((40, 2500, 8320), "slq::gemv_mk_kernel", None),
             ((48, 2048, 1152), "slq::gemv_mk_kernel", None)]
    for (m, n, k), kname, ks in cases:
        say(f"split tails bits={bits} m={m} n={n} k={k}")
        W = S.skewed_weights(n, k, 17 * bits + n + m, row_offset_std=0.005)
        x = S.activations_bf16(m, k, 5 * m + bits + k)
        pw = slq.slq_quantize_pack(gpu(W), bits)
        assert slq.kernel_name(m, pw).startswith(kname)
        assert ks is None or _splits(m, pw) == ks
        y = slq.slq_dequant_gemm(x_gpu(x), pw)
        y2 = slq.slq_dequant_gemm(x_gpu(x), pw)
        torch.cuda.synchronize()
        assert torch.equal(y, y2)
        yr, br, _ = full_ref(W, bits, x)
        assert_gemm_close(y.cpu().numpy(), yr, br, what=f"tails b{bits} m{m} {n}x{k}")
        del y, y2, pw
        torch.cuda.empty_cache()


def test_stack_parallel_branches_match_one_stream():
    """Calls that overlap on different streams, each with its own split-k
    workspace, give bit-identical outputs to the same calls in sequence on one
    stream: a layer's independent projections as parallel graph branches
    (q || k || v, then o, then gate || up, then down), eagerly and on every
    replay of the captured graph, with the tickets back at zero."""
    m = 64
    bmap = S.mixed_bit_map()
    Ws = {p: gpu(S.skewed_weights(*S.LLAMA3_8B_PROJ[p], S.seed_for(3, 0, j), row_offset_std=0.005))
          for j, p in enumerate(S.PROJ_ORDER)}
    layers = [{p: slq.slq_quantize_pack(Ws[p], bmap[layer][p]) for p in S.PROJ_ORDER}
              for layer in (0, 31)]
    del Ws
    xk = {k: x_gpu(S.activations_bf16(m, k, 40 + k % 97)) for k in (4096, 14336)}
    wsb = max(slq.gemm_workspace_bytes(m, pw) for lay in layers for pw in lay.values())
    wss = [torch.zeros(max(wsb, 256), dtype=torch.uint8, device=DEV) for _ in range(3)]
    ys = [{p: torch.empty((m, pw.n), dtype=torch.float32, device=DEV) for p, pw in lay.items()}
          for lay in layers]

    def gemm(li, p, w):
        pw = layers[li][p]
        slq.slq_dequant_gemm(xk[pw.k], pw, y=ys[li][p], ws=wss[w])

    side = [torch.cuda.Stream(device=DEV) for _ in range(2)]

    def branches():
        main = torch.cuda.current_stream()
        for li in range(len(layers)):
            for sd in side:
                sd.wait_stream(main)
            with torch.cuda.stream(side[0]):
                gemm(li, "k", 1)
            with torch.cuda.stream(side[1]):
                gemm(li, "v", 2)
            gemm(li, "q", 0)
            for sd in side:
                main.wait_stream(sd)
            gemm(li, "o", 0)
            side[0].wait_stream(main)
            with torch.cuda.stream(side[0]):
                gemm(li, "up", 1)
            gemm(li, "gate", 0)
            main.wait_stream(side[0])
            gemm(li, "down", 0)

    for li in range(len(layers)):
        for p in S.PROJ_ORDER:
            gemm(li, p, 0)
    torch.cuda.synchronize()
    ref = [{p: y.clone() for p, y in d.items()} for d in ys]
    branches()
    torch.cuda.synchronize()
    for li in range(len(layers)):
        for p in S.PROJ_ORDER:
            assert torch.equal(ys[li][p], ref[li][p]), ("eager branches", li, p)
    cap = torch.cuda.Stream(device=DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        branches()
    for rep in range(3):
        for d in ys:
            for y in d.values():
                y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for li in range(len(layers)):
            for p in S.PROJ_ORDER:
                assert torch.equal(ys[li][p], ref[li][p]), ("graph replay", rep, li, p)
    for w in wss:
        assert int(w[:65536].sum()) == 0
