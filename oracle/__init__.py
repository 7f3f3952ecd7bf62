"""ctypes front-end of the SLQ CPU oracle -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use
this package.  It takes and returns numpy host arrays and never touches the
HIP library.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
_u32p = np.ctypeslib.ndpointer(np.uint32, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64
_int = ctypes.c_int


def load(path: str):
    """Load an oracle build from `path` and declare its C signatures."""
    L = ctypes.CDLL(path)
    L.oracle_num_threads.restype = _int
    L.oracle_set_threads.argtypes = [_int]
    L.oracle_quantize.argtypes = [_f32p, _i64, _i64, _int, _int, _int, _u8p, _f32p, _u8p]
    L.oracle_pack.argtypes = [_u8p, _i64, _i64, _int, _u32p]
    L.oracle_unpack.argtypes = [_u32p, _i64, _i64, _int, _u8p]
    L.oracle_dequantize.argtypes = [_u8p, _f32p, _u8p, _i64, _i64, _int, _f32p]
    L.oracle_gemm.argtypes = [_u16p, _i64, _i64, _f32p, _i64, _f64p, _f64p]
    L.oracle_gemm_pairs.argtypes = [_u16p, _i64, _f32p, _i64p, _i64p, _i64, _f64p, _f64p]
    L.oracle_row_lse.argtypes = [_f32p, _i64, _i64, _f64p]
    L.oracle_ear_kl.argtypes = [_f32p, _f32p, _i64, _i64, _f64p, _f64p, _f64p]
    L.oracle_ear_kl_topk.argtypes = [_f32p, _f32p, _i64, _i64, _i64, ctypes.c_double, _f64p, _f64p,
                                     _f64p]
    L.oracle_quant_error.argtypes = [_f32p, _f32p, _f32p, _i64, _i64, _int, _f64p]
    L.oracle_bits_per_param.argtypes = [_int, _int, _int]
    L.oracle_bits_per_param.restype = ctypes.c_double
    L.oracle_mckp_search.argtypes = [_i64, _int, _i64p, _f64p, _i64, ctypes.c_double,
                                     np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS"),
                                     ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64),
                                     ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
    L.oracle_mckp_search.restype = _int
    L.oracle_f16_value.argtypes = [ctypes.c_uint16]
    L.oracle_f16_value.restype = ctypes.c_double
    L.oracle_f16_round_up.argtypes = [ctypes.c_float]
    L.oracle_f16_round_up.restype = ctypes.c_uint16
    L.oracle_compact_zero_bits.argtypes = [_int]
    L.oracle_compact_zero_bits.restype = _int
    L.oracle_quantize_compact.argtypes = [_f32p, _i64, _i64, _int, _int, _int, _u8p, _u16p, _u8p]
    L.oracle_pack_zeros.argtypes = [_u8p, _i64, _int, _u8p]
    L.oracle_pack_zeros.restype = _i64
    L.oracle_dequantize_compact.argtypes = [_u8p, _u16p, _u8p, _i64, _i64, _int, _int, _f32p]
    L.oracle_gptq_columns.argtypes = [_f32p, _f32p, ctypes.c_void_p, _i64, _i64, _int, _int, _u8p,
                                      _f32p, _u8p]
    return L


def lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(HERE, "liboracle.so")
        if not os.path.exists(path):
            from oracle.build import build
            build()
        _LIB = load(path)
    return _LIB


def use(L):
    """Point this module at another oracle build (mutation tests); returns the old one."""
    global _LIB
    old, _LIB = _LIB, L
    return old


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def quantize(W, bits: int, group: int = 128, symmetric: bool = False):
    """Codes q[n][k] (uint8), scales[n][G] (fp32), zeros[n][G] (uint8)."""
    W = _c(W, np.float32)
    n, k = W.shape
    G = k // group
    q = np.empty((n, k), np.uint8)
    s = np.empty((n, G), np.float32)
    z = np.empty((n, G), np.uint8)
    lib().oracle_quantize(W, n, k, bits, group, int(symmetric), q, s, z)
    return q, s, z


def pack(q, bits: int):
    q = _c(q, np.uint8)
    n, k = q.shape
    out = np.empty((n, k * bits // 32), np.uint32)
    lib().oracle_pack(q, n, k, bits, out)
    return out


def unpack(words, k: int, bits: int):
    words = _c(words, np.uint32)
    n = words.shape[0]
    q = np.empty((n, k), np.uint8)
    lib().oracle_unpack(words, n, k, bits, q)
    return q


def dequantize(q, scales, zeros, group: int = 128):
    q = _c(q, np.uint8)
    n, k = q.shape
    out = np.empty((n, k), np.float32)
    lib().oracle_dequantize(q, _c(scales, np.float32), _c(zeros, np.uint8), n, k, group, out)
    return out


def gemm(x_bf16, w_hat):
    """fp64 y[m][n] = x . w_hat^T and bound[m][n] = |x| . |w_hat|^T."""
    x = _c(x_bf16, np.uint16)
    w = _c(w_hat, np.float32)
    m, k = x.shape
    n = w.shape[0]
    y = np.empty((m, n), np.float64)
    b = np.empty((m, n), np.float64)
    lib().oracle_gemm(x, m, k, w, n, y, b)
    return y, b


def gemm_pairs(x_bf16, w_hat_rows, xi, wi):
    x = _c(x_bf16, np.uint16)
    w = _c(w_hat_rows, np.float32)
    xi = _c(xi, np.int64)
    wi = _c(wi, np.int64)
    y = np.empty(len(xi), np.float64)
    b = np.empty(len(xi), np.float64)
    lib().oracle_gemm_pairs(x, x.shape[1], w, xi, wi, len(xi), y, b)
    return y, b


def row_lse(a):
    a = _c(a, np.float32)
    out = np.empty(a.shape[0], np.float64)
    lib().oracle_row_lse(a, a.shape[0], a.shape[1], out)
    return out


def ear_kl(a, b):
    """Per-row EAR and KL(p||q) in fp64, plus their means (ear_mean, kl_mean)."""
    a = _c(a, np.float32)
    b = _c(b, np.float32)
    rows, vocab = a.shape
    ear = np.empty(rows, np.float64)
    kl = np.empty(rows, np.float64)
    means = np.empty(2, np.float64)
    lib().oracle_ear_kl(a, b, rows, vocab, ear, kl, means)
    return ear, kl, means


def ear_kl_topk(a, b, k: int, temperature: float = 1.0):
    """Per-row top-K EAR and top-K KL(p||q) at a temperature (fp64), plus means.
    The top-K set is the K largest reference logits, ties to the lower index."""
    a = _c(a, np.float32)
    b = _c(b, np.float32)
    rows, vocab = a.shape
    if not (1 <= k <= min(vocab, 4096)):
        raise ValueError("k must be in [1, min(vocab, 4096)]")
    ear = np.empty(rows, np.float64)
    kl = np.empty(rows, np.float64)
    means = np.empty(2, np.float64)
    lib().oracle_ear_kl_topk(a, b, rows, vocab, k, float(temperature), ear, kl, means)
    return ear, kl, means


def quant_error(W, w_hat, scales, group: int = 128):
    """(sum (w - w_hat)^2, sum_g s_g^2) in fp64."""
    W = _c(W, np.float32)
    n, k = W.shape
    out = np.empty(2, np.float64)
    lib().oracle_quant_error(W, _c(w_hat, np.float32), _c(scales, np.float32), n, k, group, out)
    return float(out[0]), float(out[1])


def bits_per_param(bits: int, meta_bits: int, group: int = 128) -> float:
    return lib().oracle_bits_per_param(bits, meta_bits, group)


def mckp_search(sizes, costs, W: int, tau: float, with_best: bool = False):
    """Bit-width allocation: exact multiple-choice knapsack over the cost table
    for every budget 0..W, then the smallest budget whose optimal cost is <= tau.

    sizes int64 [L][nb] (budget units; a negative size: an option never taken),
    costs float64 [L][nb].  Returns
    (status, choice int32 [L], budget, size, cost[, best float64 [W+1]]);
    status 0: found, 1: W does not meet tau (choice at W), 2: nothing fits."""
    sizes = _c(sizes, np.int64)
    costs = _c(costs, np.float64)
    L, nb = sizes.shape
    if costs.shape != sizes.shape or not (1 <= nb <= 127) or W < 0:
        raise ValueError("bad knapsack instance")
    choice = np.empty(L, np.int32)
    budget, size, cost = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_double()
    best = np.empty(W + 1, np.float64) if with_best else None
    st = lib().oracle_mckp_search(L, nb, sizes, costs, int(W), float(tau), choice,
                                  ctypes.byref(budget), ctypes.byref(size), ctypes.byref(cost),
                                  best.ctypes.data if with_best else None)
    out = (st, choice, budget.value, size.value, cost.value)
    return out + (best,) if with_best else out


def f16_value(bits: int) -> float:
    return lib().oracle_f16_value(int(bits))


def f16_round_up(s: float) -> int:
    """Bits of the smallest binary16 value >= s (s > 0), saturating at 65504."""
    return int(lib().oracle_f16_round_up(float(s)))


def compact_zero_bits(bits: int) -> int:
    return lib().oracle_compact_zero_bits(bits)


def quantize_compact(W, bits: int, group: int = 128, symmetric: bool = False):
    """Codes uint8 [n][k], binary16 scale bits uint16 [n][G], zero points uint8 [n][G]."""
    W = _c(W, np.float32)
    n, k = W.shape
    q = np.empty((n, k), np.uint8)
    s16 = np.empty((n, k // group), np.uint16)
    z = np.empty((n, k // group), np.uint8)
    lib().oracle_quantize_compact(W, n, k, bits, group, int(symmetric), q, s16, z)
    return q, s16, z


def pack_zeros(zeros, bits: int):
    """Compact zero points: nibbles (b <= 4, low nibble first) or bytes."""
    z = _c(zeros, np.uint8).ravel()
    out = np.empty(len(z), np.uint8)
    nb = lib().oracle_pack_zeros(z, len(z), bits, out)
    return out[:nb].copy()


def dequantize_compact(q, scales16, zpacked, bits: int, group: int = 128):
    q = _c(q, np.uint8)
    n, k = q.shape
    out = np.empty((n, k), np.float32)
    lib().oracle_dequantize_compact(q, _c(scales16, np.uint16).ravel(), _c(zpacked, np.uint8),
                                    n, k, group, bits, out)
    return out


def gptq_columns(W, U, bits: int, dead=None, group: int = 128):
    """fp32 GPTQ column pass with lazy 128-column blocks (oracle.c,
    oracle_gptq_columns): W fp32 [n][k], U fp32 [k][k] upper factor of the
    inverse Hessian, dead bool [k] or None.  Returns codes uint8 [n][k],
    scales fp32 [n][G], zeros uint8 [n][G]."""
    W = _c(W, np.float32)
    U = _c(U, np.float32)
    n, k = W.shape
    q = np.zeros((n, k), np.uint8)
    s = np.zeros((n, k // group), np.float32)
    z = np.zeros((n, k // group), np.uint8)
    d = None
    if dead is not None:
        d = _c(np.asarray(dead).astype(np.uint8), np.uint8)
    lib().oracle_gptq_columns(W, U, None if d is None else d.ctypes.data, n, k, bits, group, q, s, z)
    return q, s, z
