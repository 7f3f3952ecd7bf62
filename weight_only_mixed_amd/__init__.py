"""Python binding of libslq (SLQ hot path on MI355X / gfx950).

Thin ctypes marshalling over the C ABI in include/slq.h: every computation runs
in the HIP kernels of libslq.so.  torch provides device memory and the current
stream.  There is no fallback: if the library is missing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libslq.so")

SLQ_OK, SLQ_EINVAL, SLQ_ENOTSUP, SLQ_EHIP, SLQ_ESCRATCH = 0, 1, 2, 3, 4
SLQ_ASYM, SLQ_SYM = 0, 1
SLQ_META_F32, SLQ_META_COMPACT = 0, 1
GROUP = 128


class SlqError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {lib().slq_strerror(status).decode()} (status {status})")


class SlqPacked(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("group", ctypes.c_int32),
                ("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("zeros", ctypes.c_void_p), ("meta", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


_LIB = None
_i64, _int, _vp, _sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
_pp = ctypes.POINTER(SlqPacked)


def lib():
    """Load libslq.so (built in-tree by weight_only_mixed_amd/build.py)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with weight_only_mixed_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        L.slq_codes_bytes.argtypes = [_i64, _i64, _int]
        L.slq_codes_bytes.restype = _sz
        L.slq_scales_bytes.argtypes = [_i64, _i64, ctypes.c_int32]
        L.slq_scales_bytes.restype = _sz
        L.slq_zeros_bytes.argtypes = [_i64, _i64, _int, ctypes.c_int32]
        L.slq_zeros_bytes.restype = _sz
        L.slq_quantize_pack.argtypes = [_vp, _i64, _i64, _int, _int, _int, _pp, _vp]
        L.slq_dequantize.argtypes = [_pp, _vp, _vp]
        L.slq_gemm_workspace_bytes.argtypes = [_i64, _pp]
        L.slq_gemm_workspace_bytes.restype = _sz
        L.slq_dequant_gemm.argtypes = [_vp, _pp, _i64, _vp, _vp, _vp]
        L.slq_dequant_gemm_noalloc.argtypes = [_vp, _pp, _i64, _vp, _vp]
        L.slq_noalloc_scratch_bytes.argtypes = []
        L.slq_noalloc_scratch_bytes.restype = _sz
        L.slq_ear_kl_workspace_bytes.argtypes = [_i64, _i64]
        L.slq_ear_kl_workspace_bytes.restype = _sz
        L.slq_row_lse.argtypes = [_vp, _i64, _i64, _vp, _vp, _vp]
        L.slq_ear_kl.argtypes = [_vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp]
        L.slq_ear_kl_topk.argtypes = [_vp, _vp, _i64, _i64, _i64, ctypes.c_double, _vp, _vp, _vp,
                                      _vp, _vp]
        L.slq_gptq_workspace_bytes.argtypes = [_i64, _i64]
        L.slq_gptq_workspace_bytes.restype = _sz
        L.slq_gptq_quantize.argtypes = [_vp, _vp, _i64, _i64, _int, _int, ctypes.c_double, _pp, _vp,
                                        _vp, _vp]
        L.slq_gptq_factor_workspace_bytes.argtypes = [_i64]
        L.slq_gptq_factor_workspace_bytes.restype = _sz
        L.slq_gptq_factor.argtypes = [_vp, _i64, ctypes.c_double, _vp, _vp, _vp, _vp, _vp]
        L.slq_gptq_columns_workspace_bytes.argtypes = [_i64, _i64]
        L.slq_gptq_columns_workspace_bytes.restype = _sz
        L.slq_gptq_columns.argtypes = [_vp, _vp, _vp, _i64, _i64, _int, _int, _pp, _vp, _vp]
        L.slq_mckp_workspace_bytes.argtypes = [_i64, _i64]
        L.slq_mckp_workspace_bytes.restype = _sz
        L.slq_mckp_search.argtypes = [_vp, _vp, _i64, ctypes.c_int32, _i64, ctypes.c_double, _vp,
                                      _vp, _vp, _vp, _vp, _vp]
        L.slq_quant_error_workspace_bytes.argtypes = [_pp]
        L.slq_quant_error_workspace_bytes.restype = _sz
        L.slq_quant_error.argtypes = [_vp, _pp, _vp, _vp, _vp]
        L.slq_dequant_gemm_kernel_name.argtypes = [_i64, _pp]
        L.slq_dequant_gemm_kernel_name.restype = ctypes.c_char_p
        L.slq_stream_read.argtypes = [_vp, _sz, _vp, _vp]
        L.slq_stream_read_words.argtypes = [_sz]
        L.slq_stream_read_words.restype = _sz
        L.slq_strerror.argtypes = [_int]
        L.slq_strerror.restype = ctypes.c_char_p
        for f in ("slq_quantize_pack", "slq_dequantize", "slq_dequant_gemm", "slq_row_lse",
                  "slq_ear_kl", "slq_ear_kl_topk", "slq_mckp_search", "slq_gptq_quantize",
                  "slq_quant_error"):
            getattr(L, f).restype = _int
        _LIB = L
    return _LIB


def _check(status: int, what: str):
    if status != SLQ_OK:
        raise SlqError(status, what)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


@dataclass
class PackedWeight:
    """A packed weight: codes uint32 [n][k*bits/32]; metadata SLQ_META_F32:
    scales fp32 [n][G], zeros uint8 [n][G]; SLQ_META_COMPACT: scales binary16
    bits int16 [n*G], zeros nibbles (bits <= 4) uint8 [ceil(n*G/2)] or bytes."""
    bits: int
    n: int
    k: int
    codes: torch.Tensor
    scales: torch.Tensor
    zeros: torch.Tensor
    group: int = GROUP
    meta: int = SLQ_META_F32

    def c(self) -> SlqPacked:
        return SlqPacked(self.bits, self.group, self.n, self.k, _ptr(self.codes),
                         _ptr(self.scales), _ptr(self.zeros), self.meta, 0)

    @property
    def nbytes(self) -> int:
        return (self.codes.numel() * 4 + self.scales.numel() * self.scales.element_size() +
                self.zeros.numel())


def alloc_packed(n: int, k: int, bits: int, device, group: int = GROUP,
                 meta: int = SLQ_META_F32) -> PackedWeight:
    G = k // group
    if meta == SLQ_META_COMPACT:
        scales = torch.empty((n * G,), dtype=torch.int16, device=device)
        zeros = torch.empty(((n * G + 1) // 2 if bits <= 4 else n * G,), dtype=torch.uint8,
                            device=device)
    else:
        scales = torch.empty((n, G), dtype=torch.float32, device=device)
        zeros = torch.empty((n, G), dtype=torch.uint8, device=device)
    return PackedWeight(bits, n, k,
                        torch.empty((n, k * bits // 32), dtype=torch.int32, device=device),
                        scales, zeros, group, meta)


def slq_quantize_pack(W: torch.Tensor, bits: int, group: int = GROUP, grid: int = SLQ_ASYM,
                      out: PackedWeight | None = None, meta: int = SLQ_META_F32) -> PackedWeight:
    """Quantize fp32 W[n][k] to `bits` (asymmetric by default) and pack it, with
    fp32 (SLQ_META_F32) or 20-bit (SLQ_META_COMPACT) group metadata."""
    assert W.dtype == torch.float32 and W.is_cuda and W.is_contiguous()
    n, k = W.shape
    pw = out if out is not None else alloc_packed(n, k, bits, W.device, group, meta)
    desc = pw.c()
    _check(lib().slq_quantize_pack(_ptr(W), n, k, bits, group, grid, ctypes.byref(desc),
                                   _stream(W)), "slq_quantize_pack")
    return pw


def slq_dequantize(pw: PackedWeight, out: torch.Tensor | None = None) -> torch.Tensor:
    out = out if out is not None else torch.empty((pw.n, pw.k), dtype=torch.float32,
                                                  device=pw.codes.device)
    desc = pw.c()
    _check(lib().slq_dequantize(ctypes.byref(desc), _ptr(out), _stream(out)), "slq_dequantize")
    return out


_WS: dict = {}


def workspace(nbytes: int, device, tag: str = "gemm") -> torch.Tensor | None:
    """A zero-filled workspace cached per (tag, device, stream); grown on demand.

    The library leaves a gemm workspace zero-filled after every completed call,
    so one buffer serves all calls issued on the same stream."""
    if nbytes == 0:
        return None
    dev = torch.device(device)
    key = (tag, dev.index, torch.cuda.current_stream(dev).cuda_stream)
    buf = _WS.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.zeros(((nbytes + 255) // 256) * 256, dtype=torch.uint8, device=dev)
        _WS[key] = buf
    return buf


def gemm_workspace_bytes(m: int, pw: PackedWeight) -> int:
    desc = pw.c()
    return lib().slq_gemm_workspace_bytes(m, ctypes.byref(desc))


def slq_dequant_gemm_noalloc(x: torch.Tensor, pw: PackedWeight, y: torch.Tensor) -> torch.Tensor:
    """slq_dequant_gemm without a workspace: the split-k scratch is the
    library's static per-GPU array (calls overlapping on one GPU race)."""
    assert x.dtype in (torch.bfloat16, torch.int16, torch.uint16) and x.is_cuda
    assert x.is_contiguous() and x.shape[-1] == pw.k and y.is_contiguous()
    m = x.numel() // pw.k if pw.k else x.shape[0]
    desc = pw.c()
    _check(lib().slq_dequant_gemm_noalloc(_ptr(x), ctypes.byref(desc), m, _ptr(y), _stream(x)),
           "slq_dequant_gemm_noalloc")
    return y


def kernel_name(m: int, pw: PackedWeight) -> str:
    """Profiler name of the kernel slq_dequant_gemm launches for (m, pw)."""
    desc = pw.c()
    return lib().slq_dequant_gemm_kernel_name(m, ctypes.byref(desc)).decode()


def slq_dequant_gemm(x: torch.Tensor, pw: PackedWeight, y: torch.Tensor | None = None,
                     ws: torch.Tensor | None = None) -> torch.Tensor:
    """y[m][n] = x[m][k] . w_hat[n][k]^T with bf16 x, fp32 y."""
    assert x.dtype in (torch.bfloat16, torch.int16, torch.uint16) and x.is_cuda
    assert x.is_contiguous() and x.shape[-1] == pw.k
    m = x.numel() // pw.k if pw.k else x.shape[0]
    y = y if y is not None else torch.empty((m, pw.n), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = workspace(gemm_workspace_bytes(m, pw), x.device)
    desc = pw.c()
    _check(lib().slq_dequant_gemm(_ptr(x), ctypes.byref(desc), m, _ptr(y), _ptr(ws), _stream(x)),
           "slq_dequant_gemm")
    return y


def slq_row_lse(logits: torch.Tensor) -> torch.Tensor:
    assert logits.dtype == torch.float32 and logits.is_cuda and logits.is_contiguous()
    rows, vocab = logits.shape
    lse = torch.empty(rows, dtype=torch.float64, device=logits.device)
    ws = workspace(lib().slq_ear_kl_workspace_bytes(rows, vocab), logits.device, "fidelity")
    _check(lib().slq_row_lse(_ptr(logits), rows, vocab, _ptr(lse), _ptr(ws), _stream(logits)),
           "slq_row_lse")
    return lse


def slq_ear_kl(logits_p: torch.Tensor, logits_q: torch.Tensor):
    """Per-row EAR and KL(p||q) (fp32) and their means (fp64 [2]) on the device."""
    assert logits_p.shape == logits_q.shape and logits_p.dtype == torch.float32
    assert logits_p.is_contiguous() and logits_q.is_contiguous()
    rows, vocab = logits_p.shape
    dev = logits_p.device
    ear = torch.empty(rows, dtype=torch.float32, device=dev)
    kl = torch.empty(rows, dtype=torch.float32, device=dev)
    means = torch.empty(2, dtype=torch.float64, device=dev)
    ws = workspace(lib().slq_ear_kl_workspace_bytes(rows, vocab), dev, "fidelity")
    _check(lib().slq_ear_kl(_ptr(logits_p), _ptr(logits_q), rows, vocab, _ptr(ear), _ptr(kl),
                            _ptr(means), _ptr(ws), _stream(logits_p)), "slq_ear_kl")
    return ear, kl, means


def slq_ear_kl_topk(logits_p: torch.Tensor, logits_q: torch.Tensor, k: int,
                    temperature: float = 1.0):
    """Top-k EAR and top-k KL(p||q) at a temperature, per row (fp32), and their
    means (fp64 [2]) on the device."""
    assert logits_p.shape == logits_q.shape and logits_p.dtype == torch.float32
    assert logits_p.is_contiguous() and logits_q.is_contiguous()
    rows, vocab = logits_p.shape
    dev = logits_p.device
    ear = torch.empty(rows, dtype=torch.float32, device=dev)
    kl = torch.empty(rows, dtype=torch.float32, device=dev)
    means = torch.empty(2, dtype=torch.float64, device=dev)
    ws = workspace(lib().slq_ear_kl_workspace_bytes(rows, vocab), dev, "fidelity")
    _check(lib().slq_ear_kl_topk(_ptr(logits_p), _ptr(logits_q), rows, vocab, int(k),
                                 float(temperature), _ptr(ear), _ptr(kl), _ptr(means), _ptr(ws),
                                 _stream(logits_p)), "slq_ear_kl_topk")
    return ear, kl, means


def slq_gptq_quantize(W: torch.Tensor, H: torch.Tensor, bits: int, damp: float = 0.01,
                      with_u: bool = False):
    """GPTQ codes for fp32 W[n][k] against the layer Hessian H[k][k] (fp32,
    device): a PackedWeight (fp32 metadata), and U (fp64 [k][k]) on request."""
    assert W.dtype == torch.float32 and H.dtype == torch.float32
    assert W.is_contiguous() and H.is_contiguous()
    n, k = W.shape
    pw = alloc_packed(n, k, bits, W.device)
    desc = pw.c()
    U = torch.empty((k, k), dtype=torch.float64, device=W.device) if with_u else None
    ws = workspace(lib().slq_gptq_workspace_bytes(n, k), W.device, "gptq")
    _check(lib().slq_gptq_quantize(_ptr(W), _ptr(H), n, k, bits, GROUP, float(damp),
                                   ctypes.byref(desc), _ptr(U), _ptr(ws), _stream(W)),
           "slq_gptq_quantize")
    return pw, U


def stream_read_words(nbytes: int) -> int:
    return lib().slq_stream_read_words(nbytes)


def slq_stream_read(buf: torch.Tensor, folds: torch.Tensor, nbytes: int | None = None):
    """One plain read of the first nbytes (default: all) of a device buffer
    (measurement aid: the read ceiling and per-launch floor); folds: int32
    [stream_read_words(nbytes)] receives one XOR fold per 16 KiB."""
    n = buf.numel() * buf.element_size() if nbytes is None else nbytes
    assert folds.numel() >= stream_read_words(n)
    _check(lib().slq_stream_read(_ptr(buf), n, _ptr(folds), _stream(buf)), "slq_stream_read")


def slq_gptq_factor(H: torch.Tensor, damp: float = 0.01, with_u64: bool = False):
    """The GPTQ inverse-Hessian factor of H[k][k] (fp32, device): U fp32
    [k][k], the dead-input mask uint8 [k], and U in fp64 on request."""
    assert H.dtype == torch.float32 and H.is_contiguous()
    k = H.shape[0]
    U = torch.empty((k, k), dtype=torch.float32, device=H.device)
    dead = torch.empty(k, dtype=torch.uint8, device=H.device)
    U64 = torch.empty((k, k), dtype=torch.float64, device=H.device) if with_u64 else None
    ws = workspace(lib().slq_gptq_factor_workspace_bytes(k), H.device, "gptq_factor")
    _check(lib().slq_gptq_factor(_ptr(H), k, float(damp), _ptr(U), _ptr(dead), _ptr(U64), _ptr(ws),
                                 _stream(H)), "slq_gptq_factor")
    return U, dead, U64


def slq_gptq_columns(W: torch.Tensor, U: torch.Tensor, bits: int, dead: torch.Tensor | None = None):
    """The GPTQ column pass of fp32 W[n][k] given the fp32 factor U[k][k] and
    an optional dead-input mask (uint8 [k]): a PackedWeight (fp32 metadata)."""
    assert W.dtype == torch.float32 and U.dtype == torch.float32
    assert W.is_contiguous() and U.is_contiguous()
    assert dead is None or (dead.dtype == torch.uint8 and dead.is_contiguous())
    n, k = W.shape
    pw = alloc_packed(n, k, bits, W.device)
    desc = pw.c()
    ws = workspace(lib().slq_gptq_columns_workspace_bytes(n, k), W.device, "gptq_columns")
    _check(lib().slq_gptq_columns(_ptr(W), _ptr(U), _ptr(dead), n, k, bits, GROUP,
                                  ctypes.byref(desc), _ptr(ws), _stream(W)), "slq_gptq_columns")
    return pw


def slq_mckp_search(sizes: torch.Tensor, costs: torch.Tensor, W: int, tau: float,
                    with_best: bool = False):
    """Bit-width allocation on the device: exact multiple-choice knapsack for
    budgets 0..W, smallest budget whose best cost is <= tau.  sizes int64
    [L][nb], costs float64 [L][nb] (device).  Returns (choice int32 [L],
    result int64 [3] = status, budget, size; cost float64 [1]; best or None)."""
    assert sizes.dtype == torch.int64 and costs.dtype == torch.float64
    assert sizes.shape == costs.shape and sizes.is_contiguous() and costs.is_contiguous()
    L, nb = sizes.shape
    dev = sizes.device
    choice = torch.empty(L, dtype=torch.int32, device=dev)
    result = torch.empty(3, dtype=torch.int64, device=dev)
    cost = torch.empty(1, dtype=torch.float64, device=dev)
    best = torch.empty(W + 1, dtype=torch.float64, device=dev) if with_best else None
    ws = workspace(lib().slq_mckp_workspace_bytes(L, W), dev, "mckp")
    _check(lib().slq_mckp_search(_ptr(sizes), _ptr(costs), L, nb, int(W), float(tau),
                                 _ptr(choice), _ptr(result), _ptr(cost),
                                 _ptr(best) if with_best else None, _ptr(ws), _stream(sizes)),
           "slq_mckp_search")
    return choice, result, cost, best


def slq_quant_error(W: torch.Tensor, pw: PackedWeight) -> torch.Tensor:
    """fp64 [2] on the device: (sum (w - w_hat)^2, sum_g s_g^2)."""
    desc = pw.c()
    out = torch.empty(2, dtype=torch.float64, device=W.device)
    ws = workspace(lib().slq_quant_error_workspace_bytes(ctypes.byref(desc)), W.device, "qerr")
    _check(lib().slq_quant_error(_ptr(W), ctypes.byref(desc), _ptr(out), _ptr(ws), _stream(W)),
           "slq_quant_error")
    return out


__all__ = ["lib", "SlqError", "SlqPacked", "PackedWeight", "alloc_packed", "workspace",
           "gemm_workspace_bytes", "kernel_name", "slq_quantize_pack", "slq_dequantize", "slq_dequant_gemm",
           "slq_row_lse", "slq_ear_kl", "slq_ear_kl_topk", "slq_mckp_search", "slq_gptq_quantize", "slq_quant_error",
           "SLQ_META_F32", "SLQ_META_COMPACT", "SLQ_ASYM", "SLQ_SYM", "GROUP"]
