"""Helpers for the GPU parity tests (HIP path through the C ABI vs the oracle)."""
import sys

import numpy as np
import torch

import oracle
import slq_synth as S
import weight_only_mixed_amd as slq

DEV = "cuda:0"
TOL = 1e-2          # |y - y_ref| <= TOL * sum |x| |w_hat|
FID_TOL = 1e-5      # absolute, EAR and KL


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def x_gpu(x_bits: np.ndarray) -> torch.Tensor:
    return gpu(x_bits.view(np.int16)).view(torch.bfloat16)


def host_packed(pw):
    torch.cuda.synchronize()
    return (pw.codes.cpu().numpy().view(np.uint32), pw.scales.cpu().numpy(),
            pw.zeros.cpu().numpy())


def assert_gemm_close(y, y_ref, bound, tol=TOL, what=""):
    y = np.asarray(y, np.float64)
    err = np.abs(y - y_ref)
    bad = err > tol * bound
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} outputs out of tolerance; first at {tuple(i)}: "
                             f"y={y[tuple(i)]!r} ref={y_ref[tuple(i)]!r} bound={bound[tuple(i)]!r}")
    return float((err / np.maximum(bound, 1e-300)).max())


def sample_pairs(m, n, count, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    if m * n <= count:
        mi, ni = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
        return mi.ravel().astype(np.int64), ni.ravel().astype(np.int64)
    return (g.integers(0, m, count).astype(np.int64), g.integers(0, n, count).astype(np.int64))


def oracle_sampled(W, bits, x_bits, mi, ni):
    """Oracle y and bound at (mi, ni): quantize/dequantize only the sampled rows of W."""
    rows, inv = np.unique(ni, return_inverse=True)
    q, s, z = oracle.quantize(W[rows], bits)
    wh = oracle.dequantize(q, s, z)
    return oracle.gemm_pairs(x_bits, wh, mi, inv.astype(np.int64))
