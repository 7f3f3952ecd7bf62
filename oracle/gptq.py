"""GPTQ code selection, plain fp64 numpy -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use
this module.  The pages name GPTQ as the code-choice step of the pipeline
(SLQ README, Pipeline: layer-wise GPTQ at every bit-width, asymmetric INT,
group size 128) without defining it; this follows the published algorithm
(Frantar, Ashkboos, Hoefler and Alistarh, "GPTQ: Accurate Post-Training
Quantization for Generative Pre-trained Transformers", ICLR 2023: Algorithm 1
with the Cholesky form of the inverse Hessian), column by column.

Two column passes follow the same steps: `gptq_columns64` (fp64 weights,
every column's update applied to all later columns at once) and the C
oracle's fp32 pass with the algorithm's lazy 128-column blocks
(`oracle.gptq_columns`, the form the GPU runs, operation for operation);
`gptq` and `gptq32` run them from a Hessian.

Parity is pinned by properties, not by the pages: an identity Hessian gives
round-to-nearest exactly; the first column's update equals the closed-form
optimal-brain-surgeon step from an explicitly inverted Hessian; on correlated
Hessians the proxy loss is below round-to-nearest's; on inputs where every
fp32 operation is exact the two column passes agree code for code.
"""
from __future__ import annotations

import numpy as np

import oracle


def prepare_hessian(H, W, damp: float = 0.01):
    """Dead inputs (zero diagonal) get H_ii = 1 and a zeroed weight column;
    then H += damp * mean(diag H) * I.  Returns (H fp64, W fp64)."""
    H = np.array(H, np.float64, copy=True)
    W = np.array(W, np.float64, copy=True)
    dead = np.diag(H) == 0
    H[dead, dead] = 1.0
    W[:, dead] = 0.0
    H[np.diag_indices_from(H)] += damp * np.mean(np.diag(H))
    return H, W


def upper_inverse_factor(H):
    """U upper triangular with H^-1 = U^T U (the Cholesky factor of the
    inverse Hessian, as the algorithm uses it)."""
    Hinv = np.linalg.inv(H)
    return np.linalg.cholesky(Hinv).T


def group_params(w32, bits: int):
    """Asymmetric scale and zero point of one group of fp32 values, by the
    steps of the oracle's plain quantizer (R1-R4)."""
    maxq = np.float32(2 ** bits - 1)
    lo = min(np.float32(0), w32.min())
    hi = max(np.float32(0), w32.max())
    s = np.float32(np.float32(hi - lo) / maxq)
    if s == 0:
        return np.float32(1), 0
    z = int(np.clip(np.rint(np.float32(-lo) / s), 0, maxq))
    return s, z


def gptq(W, H, bits: int, group: int = 128, damp: float = 0.01):
    """Codes uint8 [n][k], scales fp32 [n][G], zeros uint8 [n][G], and the
    factor U.  Weights are updated in fp64; each quantization step works on the
    fp32-rounded current weights with the plain quantizer's fp32 steps."""
    H, Wk = prepare_hessian(H, W, damp)
    U = upper_inverse_factor(H)
    q, scales, zeros = gptq_columns64(Wk, U, bits, group)
    return q, scales, zeros, U


def dead_inputs(H):
    """Inputs whose Hessian diagonal is zero (they never fire)."""
    return np.diag(np.asarray(H)) == 0


def gptq32(W, H, bits: int, group: int = 128, damp: float = 0.01):
    """The fp32 lazy-block form from a Hessian: U in fp64 as in `gptq`,
    rounded to fp32, then the C oracle's column pass.  Returns codes, scales,
    zeros and the fp64 U."""
    Hp, _ = prepare_hessian(H, W, damp)
    U = upper_inverse_factor(Hp)
    q, s, z = oracle.gptq_columns(np.asarray(W, np.float32), U.astype(np.float32), bits,
                                  dead=dead_inputs(H), group=group)
    return q, s, z, U


def gptq_columns64(W, U, bits: int, group: int = 128):
    """Column pass with fp64 weights, given the upper factor U of the inverse
    Hessian: column i is quantized from its fp32-rounded current weight, its
    error is divided by U_ii and every later column moves at once."""
    Wk = np.array(W, np.float64, copy=True)
    U = np.asarray(U, np.float64)
    n, k = Wk.shape
    G = k // group
    maxq = 2 ** bits - 1
    q = np.zeros((n, k), np.uint8)
    scales = np.zeros((n, G), np.float32)
    zeros = np.zeros((n, G), np.uint8)
    for i in range(k):
        g = i // group
        if i % group == 0:
            for r in range(n):
                s, z = group_params(Wk[r, i:i + group].astype(np.float32), bits)
                scales[r, g], zeros[r, g] = s, z
        w32 = Wk[:, i].astype(np.float32)
        s = scales[:, g]
        z = zeros[:, g].astype(np.float32)
        t = np.rint(w32 / s)
        qi = np.clip(t + z, 0, maxq).astype(np.uint8)
        q[:, i] = qi
        w_hat = ((qi.astype(np.int32) - zeros[:, g]).astype(np.float32) * s).astype(np.float64)
        err = (Wk[:, i] - w_hat) / U[i, i]
        Wk[:, i + 1:] -= np.outer(err, U[i, i + 1:])
    return q, scales, zeros


def proxy_loss(W, w_hat, H):
    """tr((W - W_hat) H (W - W_hat)^T): the layer-output error the algorithm
    minimizes greedily (H = 2 X X^T)."""
    D = np.asarray(W, np.float64) - np.asarray(w_hat, np.float64)
    return float(((D @ np.asarray(H, np.float64)) * D).sum())
