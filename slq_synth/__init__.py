"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module draws random numbers and nothing else: it holds none of the
quantization, matmul or fidelity arithmetic.  Both the HIP path and the CPU
oracle receive the same host arrays from here.

Workload shapes follow the layers the pages evaluate (Llama-3-8B and
Llama-3.3-70B projections, a 151936-entry vocabulary, 512 calibration rows).
Generator: numpy PCG64 with the seed recipe ``1000*config + 7*layer + proj``.

Distributional readings (stated once here, repeated in the design notes):
  * "N(0.003, 0.02)" is mean 0.003 and standard deviation 0.02.
  * "0.5% outliers at +-0.3": every element independently, with probability
    0.005, is replaced by +0.3 or -0.3 with equal odds.
  * "per-row mean offsets N(0, 0.005)": one draw per output row n, added to
    that row's non-outlier elements.
  * the logit "top-20 boost": 20 distinct uniform indices per row get +8.
  * quantized-model logits are the reference plus N(0, sigma) noise, in fp32.
"""
from __future__ import annotations

import numpy as np

# Output-by-input (N, K) shapes of one decoder layer's seven projections.
LLAMA3_8B_PROJ = {
    "q": (4096, 4096),
    "k": (1024, 4096),
    "v": (1024, 4096),
    "o": (4096, 4096),
    "gate": (14336, 4096),
    "up": (14336, 4096),
    "down": (4096, 14336),
}
LLAMA33_70B_PROJ = {
    "q": (8192, 8192),
    "k": (1024, 8192),
    "v": (1024, 8192),
    "o": (8192, 8192),
    "gate": (28672, 8192),
    "up": (28672, 8192),
    "down": (8192, 28672),
}
PROJ_ORDER = ("q", "k", "v", "o", "gate", "up", "down")

# Bit-width classes of the mixed-precision stack: sensitive K/V projections
# get 7-8 bits, attention q/o 5-6, MLP 3-4.
BIT_CLASSES = {
    "q": (5, 6), "o": (5, 6),
    "k": (7, 8), "v": (7, 8),
    "gate": (3, 4), "up": (3, 4), "down": (3, 4),
}

VOCAB = 151936
FIDELITY_ROWS = 512
FIDELITY_SIGMAS = (0.01, 0.05, 0.2)


def seed_for(config: int, layer: int = 0, proj: int = 0) -> int:
    return 1000 * config + 7 * layer + proj


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def skewed_weights(n: int, k: int, seed: int, row_offset_std: float = 0.0,
                   mean: float = 0.003, std: float = 0.02,
                   outlier_p: float = 0.005, outlier_mag: float = 0.3) -> np.ndarray:
    """fp32 weight matrix W[n][k] (n outputs, k inputs, k contiguous)."""
    g = rng(seed)
    w = g.standard_normal((n, k), dtype=np.float32)
    w *= np.float32(std)
    w += np.float32(mean)
    if row_offset_std > 0.0:
        off = (g.standard_normal(n, dtype=np.float32) * np.float32(row_offset_std))
        w += off[:, None]
    if outlier_p > 0.0:
        mask = g.random((n, k), dtype=np.float32) < np.float32(outlier_p)
        sign = g.random((n, k), dtype=np.float32) < np.float32(0.5)
        w[mask] = np.where(sign[mask], np.float32(outlier_mag), np.float32(-outlier_mag))
    return w


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def activations_bf16(m: int, k: int, seed: int) -> np.ndarray:
    """Activations x[m][k] ~ N(0,1) as bf16 bit patterns (uint16)."""
    g = rng(seed)
    return to_bf16_bits(g.standard_normal((m, k), dtype=np.float32))


def fidelity_logits(rows: int, vocab: int, sigma: float, seed: int,
                    std: float = 3.0, boost: float = 8.0, top: int = 20):
    """Reference logits a[rows][vocab] and perturbed logits b = a + N(0, sigma)."""
    g = rng(seed)
    a = g.standard_normal((rows, vocab), dtype=np.float32)
    a *= np.float32(std)
    top = min(top, vocab)
    for r in range(rows):
        idx = g.choice(vocab, size=top, replace=False)
        a[r, idx] += np.float32(boost)
    noise = g.standard_normal((rows, vocab), dtype=np.float32)
    noise *= np.float32(sigma)
    b = a + noise
    return a, b


def mixed_bit_map(layers: int = 32, seed: int = seed_for(3)):
    """Per-(layer, projection) bit widths drawn uniformly inside each class."""
    g = rng(seed)
    out = []
    for _ in range(layers):
        row = {}
        for p in PROJ_ORDER:
            lo, hi = BIT_CLASSES[p]
            row[p] = int(g.integers(lo, hi + 1))
        out.append(row)
    return out


def allocation_table(layers: int = 32, shapes=None, bits=tuple(range(2, 9)),
                     meta_bits: int = 40, seed: int = seed_for(3, 1)):
    """Synthetic per-(projection, bit-width) table for the bit-width allocation
    of a `layers`-deep decoder (Llama-3-8B projection shapes by default).

    sizes[i][j]: storage of projection i at bits[j] in budget units of
    (unit groups) x 8 bits, i.e. G_i / unit * (128 * b + meta_bits) / 8 with
    G_i = n * k / 128 groups and unit = gcd of the G_i.
    costs[i][j]: a stand-in for the Shapley cost table, s_i * 4^-b (rounding
    noise variance falls by 4 per bit), with a per-size sensitivity of 256 for
    k/v, 16 for q/o and 1 for the MLP (a lognormal jitter of 0.3 per
    projection), so that the optimum at the class mid-points puts k/v, q/o and
    the MLP in the bit-width classes of the mixed stack.
    tau: the cost of the class mid-points, sum_i s_i (4^-lo + 4^-hi) / 2.
    Returns (sizes int64 [L][nb], costs float64 [L][nb], tau, names)."""
    shapes = LLAMA3_8B_PROJ if shapes is None else shapes
    g = rng(seed)
    groups = {p: shapes[p][0] * shapes[p][1] // 128 for p in PROJ_ORDER}
    unit = int(np.gcd.reduce(np.array(list(groups.values()), np.int64)))
    per = {"q": 16.0, "o": 16.0, "k": 256.0, "v": 256.0, "gate": 1.0, "up": 1.0, "down": 1.0}
    assert (128 * np.array(bits) + meta_bits).min() % 8 == 0 and meta_bits % 8 == 0
    sizes, costs, names = [], [], []
    tau = 0.0
    for layer in range(layers):
        for p in PROJ_ORDER:
            u = groups[p] // unit
            sizes.append([u * (128 * b + meta_bits) // 8 for b in bits])
            sens = u * per[p] * float(np.exp(0.3 * g.standard_normal()))
            costs.append([sens * 4.0 ** (-b) for b in bits])
            lo, hi = BIT_CLASSES[p]
            tau += sens * (4.0 ** (-lo) + 4.0 ** (-hi)) / 2
            names.append(f"{layer}.{p}")
    return np.array(sizes, np.int64), np.array(costs, np.float64), tau, names


def gptq_hessian(k: int, seed: int, tokens: int | None = None, rank: int = 8) -> np.ndarray:
    """Synthetic layer Hessian H = 2 X X^T / T (float32 [k][k]) from T seeded
    activation vectors with correlated channels: a rank-`rank` shared
    component plus independent noise, and lognormal per-channel scales (a few
    strong channels, as in transformer activations)."""
    g = rng(seed)
    T = tokens if tokens is not None else 2 * k
    scale = np.exp(0.5 * g.standard_normal(k))
    B = g.standard_normal((k, rank)) / np.sqrt(rank)
    X = (B @ g.standard_normal((rank, T)) + 0.5 * g.standard_normal((k, T))) * scale[:, None]
    return (2.0 * (X @ X.T) / T).astype(np.float32)


def gptq_factor(k: int, seed: int, coupling: float = 0.5) -> np.ndarray:
    """A synthetic inverse-Hessian factor for the GPTQ column pass: float32
    [k][k] upper triangular, diagonal lognormal around 1 (a few strong inputs),
    entries above it N(0, (coupling / sqrt(k))^2), zeros below."""
    g = rng(seed)
    U = np.triu(g.standard_normal((k, k)) * (coupling / np.sqrt(k)), 1)
    U[np.arange(k), np.arange(k)] = np.exp(0.3 * g.standard_normal(k))
    return U.astype(np.float32)


def uniform_group_weights(n_groups: int, lo: float, hi: float, seed: int,
                          group: int = 128) -> np.ndarray:
    """Rows of uniform[lo, hi] samples with both endpoints pinned in every group.

    Used for the worked centering example: a group spanning [-0.4, 0.6] has
    max |w| = 0.6 and range 1.0.
    """
    g = rng(seed)
    w = g.uniform(lo, hi, size=(n_groups, group)).astype(np.float32)
    w[:, 0] = np.float32(lo)
    w[:, 1] = np.float32(hi)
    return w
