"""The allocation-free matmul (slq_dequant_gemm_noalloc, for callers that
cannot allocate) against slq_dequant_gemm, through the C ABI: the same kernels
read the split-k scratch from the library's static per-GPU array instead of a
caller workspace, so outputs must be bit-identical.  Two calls in a row, the
second smaller, on shapes that split k (so the array's tickets and partial
sums are used) and on one that does not; the second call must not see the
first call's partial sums."""
import numpy as np
import pytest
import torch

import slq_synth as S
import weight_only_mixed_amd as slq
from tests.gpu_util import DEV, gpu, say, x_gpu

pytestmark = pytest.mark.gpu


def run_pair(first, second):
    outs = []
    for (m, n, k, bits) in (first, second):
        W = S.skewed_weights(n, k, 500 + n % 97 + bits, row_offset_std=0.005)
        pw = slq.slq_quantize_pack(gpu(W), bits)
        x = x_gpu(S.activations_bf16(m, k, 600 + m))
        ws_bytes = slq.gemm_workspace_bytes(m, pw)
        y_ref = slq.slq_dequant_gemm(x, pw)
        y = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
        slq.slq_dequant_gemm_noalloc(x, pw, y)
        torch.cuda.synchronize()
        a, b = y.cpu().numpy(), y_ref.cpu().numpy()
        say(f"noalloc m={m} n={n} k={k} bits={bits}: workspace {ws_bytes} B, "
            f"kernel {slq.kernel_name(m, pw)}, identical {np.array_equal(a, b)}")
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), (m, n, k, bits)
        outs.append(ws_bytes)
    return outs


@pytest.mark.parametrize("first,second", [
    ((16, 4096, 14336, 8), (8, 4096, 4096, 4)),     # decode split k, then a smaller decode
    ((64, 4096, 14336, 3), (40, 1024, 4096, 7)),    # many-row decode splits
    ((1024, 512, 8192, 4), (300, 520, 2560, 6)),    # prefill split k (partial tiles), then no split
])
def test_noalloc_matches_workspace_path(first, second):
    ws = run_pair(first, second)
    assert ws[0] > 0   # the first call of each pair uses the scratch array


def test_noalloc_rejects_oversized_scratch():
    W = S.skewed_weights(1024, 8192, 9)
    pw = slq.slq_quantize_pack(gpu(W), 4)
    x = x_gpu(S.activations_bf16(4096, 8192, 10))
    y = torch.empty((4096, 1024), dtype=torch.float32, device=DEV)
    with pytest.raises(slq.SlqError) as e:
        slq.slq_dequant_gemm_noalloc(x, pw, y)
    assert e.value.status == slq.SLQ_ESCRATCH
