"""C ABI checks that need no GPU: the library loads, exports every function
include/slq.h declares, and rejects invalid requests before any HIP call.

Pointers here are fake device addresses; validation never dereferences them
and an invalid request returns before the HIP runtime is touched.
"""
import ctypes
import os
import re

import pytest

import weight_only_mixed_amd as slq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "slq.h")

A = 0x10000000          # fake, 256-byte aligned "device" addresses far apart
B = 0x20000000
C = 0x30000000
D = 0x40000000
E = 0x50000000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(slq_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = slq.lib()
    names = declared_functions()
    assert len(names) == 27
    for name in names:
        assert hasattr(L, name), name


def test_noalloc_validation():
    """Argument faults and an oversized split-k request are rejected before
    any HIP call (the static scratch is not touched)."""
    L = slq.lib()
    assert L.slq_noalloc_scratch_bytes() == 32 * 2 ** 20
    w = packed()
    N = L.slq_dequant_gemm_noalloc
    assert N(A, ctypes.byref(packed(bits=9)), 1, E, None) == slq.SLQ_EINVAL
    assert N(A, ctypes.byref(packed(group=32)), 1, E, None) == slq.SLQ_ENOTSUP
    assert N(A, ctypes.byref(w), -1, E, None) == slq.SLQ_EINVAL
    assert N(A, ctypes.byref(w), 0, E, None) == slq.SLQ_OK
    assert N(A, ctypes.byref(w), 1, A, None) == slq.SLQ_EINVAL          # y overlaps x
    assert N(None, ctypes.byref(w), 1, E, None) == slq.SLQ_EINVAL
    assert N(A, ctypes.byref(w), 1, E + 4, None) == slq.SLQ_EINVAL      # misaligned y
    # a prefill product whose split-k partial tiles exceed the 32 MiB array
    big = slq.SlqPacked(4, 128, 1024, 8192, B, C, D)
    assert L.slq_gemm_workspace_bytes(4096, ctypes.byref(big)) > 32 * 2 ** 20
    assert N(A, ctypes.byref(big), 4096, E, None) == slq.SLQ_ESCRATCH
    assert b"scratch" in L.slq_strerror(slq.SLQ_ESCRATCH)


def test_stream_read_validation():
    L = slq.lib()
    assert L.slq_stream_read(A, 0, B, None) == slq.SLQ_OK          # nothing to read
    assert L.slq_stream_read(A, 100, B, None) == slq.SLQ_EINVAL    # not whole 16-byte words
    assert L.slq_stream_read(A + 8, 4096, B, None) == slq.SLQ_EINVAL   # misaligned
    assert L.slq_stream_read(None, 4096, B, None) == slq.SLQ_EINVAL
    assert L.slq_stream_read(A, 4096, None, None) == slq.SLQ_EINVAL
    assert L.slq_stream_read(A, 4096, A + 64, None) == slq.SLQ_EINVAL  # folds inside the buffer
    assert L.slq_stream_read_words(16384) == 1 and L.slq_stream_read_words(16400) == 2


def packed(bits=4, group=128, n=64, k=256, codes=B, scales=C, zeros=D):
    return slq.SlqPacked(bits, group, n, k, codes, scales, zeros)


def call_qp(W=A, n=64, k=256, bits=4, group=128, grid=0, out=None):
    out = out if out is not None else packed(0, 0, 0, 0)
    st = slq.lib().slq_quantize_pack(W, n, k, bits, group, grid, ctypes.byref(out), None)
    return st, out


def test_quantize_pack_validation():
    assert call_qp(bits=1)[0] == slq.SLQ_EINVAL
    assert call_qp(bits=9)[0] == slq.SLQ_EINVAL
    assert call_qp(group=64)[0] == slq.SLQ_ENOTSUP
    assert call_qp(group=0)[0] == slq.SLQ_EINVAL
    assert call_qp(k=200)[0] == slq.SLQ_EINVAL
    assert call_qp(n=-1)[0] == slq.SLQ_EINVAL
    assert call_qp(grid=7)[0] == slq.SLQ_EINVAL
    assert call_qp(W=None)[0] == slq.SLQ_EINVAL
    assert call_qp(W=A + 4)[0] == slq.SLQ_EINVAL                      # misaligned
    assert slq.lib().slq_quantize_pack(A, 4, 128, 4, 128, 0, None, None) == slq.SLQ_EINVAL
    # outputs overlapping the input or each other
    st, _ = call_qp(out=packed(codes=A + 4096, scales=C, zeros=D))
    assert st == slq.SLQ_EINVAL
    st, _ = call_qp(out=packed(codes=B, scales=B + 64, zeros=D))
    assert st == slq.SLQ_EINVAL
    # the descriptor is untouched on error
    out = packed(bits=0, group=0, n=0, k=0)
    st, out = call_qp(bits=9, out=out)
    assert st == slq.SLQ_EINVAL and out.bits == 0 and out.n == 0
    # empty input: valid no-op that fills the descriptor, no HIP call
    out = packed(bits=0, group=0, n=0, k=0)
    st, out = call_qp(n=0, out=out)
    assert st == slq.SLQ_OK and (out.bits, out.group, out.n, out.k) == (4, 128, 0, 256)


def test_dequant_gemm_validation():
    L = slq.lib()
    w = packed()
    y = E
    assert L.slq_dequant_gemm(A, ctypes.byref(packed(bits=9)), 1, y, None, None) == slq.SLQ_EINVAL
    assert L.slq_dequant_gemm(A, ctypes.byref(packed(group=32)), 1, y, None, None) == slq.SLQ_ENOTSUP
    assert L.slq_dequant_gemm(A, ctypes.byref(packed(k=100)), 1, y, None, None) == slq.SLQ_EINVAL
    assert L.slq_dequant_gemm(A, ctypes.byref(packed(codes=0)), 1, y, None, None) == slq.SLQ_EINVAL
    assert L.slq_dequant_gemm(A, ctypes.byref(packed(codes=B + 4)), 1, y, None, None) == slq.SLQ_EINVAL
    assert L.slq_dequant_gemm(A, ctypes.byref(w), -1, y, None, None) == slq.SLQ_EINVAL
    assert L.slq_dequant_gemm(None, ctypes.byref(w), 1, y, None, None) == slq.SLQ_EINVAL
    assert L.slq_dequant_gemm(A, ctypes.byref(w), 1, None, None, None) == slq.SLQ_EINVAL
    assert L.slq_dequant_gemm(A, ctypes.byref(w), 1, A, None, None) == slq.SLQ_EINVAL  # y aliases x
    assert L.slq_dequant_gemm(A, ctypes.byref(w), 1, B, None, None) == slq.SLQ_EINVAL  # y aliases codes
    assert L.slq_dequant_gemm(A, None, 1, y, None, None) == slq.SLQ_EINVAL
    # split-K workspace required when the plan uses one (16 activation rows on
    # a 4096 x 14336 layer: the plan splits k four ways for parallelism)
    big = packed(n=4096, k=14336)
    assert L.slq_gemm_workspace_bytes(16, ctypes.byref(big)) > 0
    assert L.slq_dequant_gemm(A, ctypes.byref(big), 16, y, None, None) == slq.SLQ_EINVAL
    assert L.slq_dequant_gemm(A, ctypes.byref(big), 16, y, E + 0x100000 + 8, None) == slq.SLQ_EINVAL
    # m == 0: valid no-op
    assert L.slq_dequant_gemm(None, ctypes.byref(w), 0, None, None, None) == slq.SLQ_OK


def test_decode_plan_beyond_grid_is_not_supported():
    """A decode plan whose k splits exceed a launch grid's y limit (65535) is
    reported as not supported before any HIP call: 4 activation rows over
    600M-long weight rows need 73,243 splits of 64 groups."""
    L = slq.lib()
    G64 = 1 << 36            # fake addresses 64 GiB apart (the codes span 4.8 GB)
    w = slq.SlqPacked(4, 128, 16, 600_000_000, G64, 2 * G64, 3 * G64)
    assert L.slq_gemm_workspace_bytes(4, ctypes.byref(w)) == 0
    assert L.slq_dequant_gemm(4 * G64, ctypes.byref(w), 4, 5 * G64, None, None) == slq.SLQ_ENOTSUP


def test_fidelity_and_error_validation():
    L = slq.lib()
    assert L.slq_ear_kl(A, B, 4, 0, C, C + 64, D, E, None) == slq.SLQ_EINVAL       # empty vocab
    assert L.slq_ear_kl(A, B, -1, 10, C, C + 64, D, E, None) == slq.SLQ_EINVAL
    assert L.slq_ear_kl(A, B, 4, 10, C, C, D, E, None) == slq.SLQ_EINVAL           # ear == kl
    assert L.slq_ear_kl(A, B, 4, 10, C, C + 64, D, None, None) == slq.SLQ_EINVAL   # no workspace
    assert L.slq_ear_kl(A + 4, B, 4, 12, C, C + 64, D, E, None) == slq.SLQ_EINVAL  # misaligned
    assert L.slq_ear_kl(A, B, 0, 10, None, None, None, None, None) == slq.SLQ_OK
    T = L.slq_ear_kl_topk
    assert T(A, B, 4, 100, 0, 1.0, C, C + 64, D, E, None) == slq.SLQ_EINVAL      # K = 0
    assert T(A, B, 4, 100, 65, 1.0, C, C + 64, D, E, None) == slq.SLQ_EINVAL     # K > SLQ_TOPK_MAX
    assert T(A, B, 4, 8, 9, 1.0, C, C + 64, D, E, None) == slq.SLQ_EINVAL        # K > vocab
    assert T(A, B, 4, 100, 10, 0.0, C, C + 64, D, E, None) == slq.SLQ_EINVAL     # T = 0
    assert T(A, B, 4, 100, 10, -1.0, C, C + 64, D, E, None) == slq.SLQ_EINVAL
    assert T(A, B, 4, 100, 10, float("nan"), C, C + 64, D, E, None) == slq.SLQ_EINVAL
    assert T(A, B, 4, 100, 10, float("inf"), C, C + 64, D, E, None) == slq.SLQ_EINVAL
    assert T(A, B, 4, 100, 10, 1e-300, C, C + 64, D, E, None) == slq.SLQ_EINVAL  # log2(e)/T overflows fp32
    assert T(A, B, 4, 100, 10, 1e300, C, C + 64, D, E, None) == slq.SLQ_EINVAL   # log2(e)/T underflows
    assert T(A, B, 4, 100, 10, 1.0, C, C, D, E, None) == slq.SLQ_EINVAL          # ear == kl
    assert T(A, B, 4, 100, 10, 1.0, C, C + 64, D, None, None) == slq.SLQ_EINVAL  # no workspace
    assert T(A + 4, B, 4, 100, 10, 1.0, C, C + 64, D, E, None) == slq.SLQ_EINVAL  # misaligned
    assert T(A, B, 4, 0, 1, 1.0, C, C + 64, D, E, None) == slq.SLQ_EINVAL        # empty vocab
    assert T(A, B, 0, 10, 5, 1.0, None, None, None, None, None) == slq.SLQ_OK
    Q = L.slq_gptq_quantize
    assert Q(A, B, 64, 200, 4, 128, 0.01, ctypes.byref(packed()), None, E, None) == slq.SLQ_EINVAL
    assert Q(A, B, 64, 256, 9, 128, 0.01, ctypes.byref(packed()), None, E, None) == slq.SLQ_EINVAL
    assert Q(A, B, 64, 256, 4, 64, 0.01, ctypes.byref(packed()), None, E, None) == slq.SLQ_ENOTSUP
    assert Q(A, B, 64, 256, 4, 128, 0.0, ctypes.byref(packed()), None, E, None) == slq.SLQ_EINVAL
    assert Q(A, B, 64, 256, 4, 128, 0.01, ctypes.byref(packed()), None, None, None) == slq.SLQ_EINVAL
    cp = packed()
    cp.meta = 1
    assert Q(A, B, 64, 256, 4, 128, 0.01, ctypes.byref(cp), None, E, None) == slq.SLQ_ENOTSUP
    assert Q(A, A, 64, 256, 4, 128, 0.01, ctypes.byref(packed(codes=A)), None, E, None) == slq.SLQ_EINVAL
    assert L.slq_gptq_workspace_bytes(64, 256) > 2 * 256 * 256 * 8
    assert L.slq_gptq_workspace_bytes(64, 200) == 0
    # factor and column pass alone
    Fc = L.slq_gptq_factor
    assert Fc(A, 200, 0.01, B, C, None, E, None) == slq.SLQ_EINVAL               # k % 128
    assert Fc(A, 256, -1.0, B, C, None, E, None) == slq.SLQ_EINVAL               # damp <= 0
    assert Fc(A, 256, 0.01, None, C, None, E, None) == slq.SLQ_EINVAL            # no U
    assert Fc(A, 256, 0.01, B, None, None, E, None) == slq.SLQ_EINVAL            # no mask
    assert Fc(A, 256, 0.01, A + 4096, C, None, E, None) == slq.SLQ_EINVAL        # U overlaps H
    assert Fc(A, 256, 0.01, B, B + 16, None, E, None) == slq.SLQ_EINVAL          # mask overlaps U
    assert Fc(A, 256, 0.01, B, C, D + 4, E, None) == slq.SLQ_EINVAL              # misaligned fp64 U
    assert L.slq_gptq_factor_workspace_bytes(256) >= 2 * 256 * 256 * 8
    assert L.slq_gptq_factor_workspace_bytes(100) == 0
    Cp = L.slq_gptq_columns
    assert Cp(A, B, None, 64, 256, 9, 128, ctypes.byref(packed()), E, None) == slq.SLQ_EINVAL
    assert Cp(A, B, None, 64, 256, 4, 64, ctypes.byref(packed()), E, None) == slq.SLQ_ENOTSUP
    assert Cp(A, B, None, 0, 256, 4, 128, ctypes.byref(packed()), E, None) == slq.SLQ_EINVAL
    assert Cp(A, None, None, 64, 256, 4, 128, ctypes.byref(packed()), E, None) == slq.SLQ_EINVAL
    assert Cp(A, B, None, 64, 256, 4, 128, ctypes.byref(packed()), None, None) == slq.SLQ_EINVAL
    assert Cp(A, B, None, 64, 256, 4, 128, ctypes.byref(cp), E, None) == slq.SLQ_ENOTSUP
    assert Cp(A, B, None, 64, 256, 4, 128, ctypes.byref(packed(codes=B + 64)), E, None) == slq.SLQ_EINVAL
    assert Cp(A, B, C + 8, 64, 256, 4, 128, ctypes.byref(packed(scales=C)), E, None) == slq.SLQ_EINVAL
    assert L.slq_gptq_columns_workspace_bytes(64, 256) == 64 * 256 * 4 + 64 * 128 * 4
    assert L.slq_gptq_columns_workspace_bytes(64, 200) == 0
    M = L.slq_mckp_search
    assert M(A, B, 0, 7, 100, 1.0, C, C + 256, C + 512, None, E, None) == slq.SLQ_EINVAL   # L = 0
    assert M(A, B, 4, 0, 100, 1.0, C, C + 256, C + 512, None, E, None) == slq.SLQ_EINVAL   # nb = 0
    assert M(A, B, 4, 128, 100, 1.0, C, C + 256, C + 512, None, E, None) == slq.SLQ_EINVAL  # nb > 127
    assert M(A, B, 4, 7, -1, 1.0, C, C + 256, C + 512, None, E, None) == slq.SLQ_EINVAL   # W < 0
    assert M(A, B, 4, 7, 100, float("nan"), C, C + 256, C + 512, None, E, None) == slq.SLQ_EINVAL
    assert M(A, B, 4, 7, 100, 1.0, C, C + 256, C + 512, None, None, None) == slq.SLQ_EINVAL  # no ws
    assert M(A, B, 4, 7, 100, 1.0, C, C, C + 512, None, E, None) == slq.SLQ_EINVAL        # aliasing
    assert M(A, B, 4, 7, 100, 1.0, A, C + 256, C + 512, None, E, None) == slq.SLQ_EINVAL  # over sizes
    assert M(A + 4, B, 4, 7, 100, 1.0, C, C + 256, C + 512, None, E, None) == slq.SLQ_EINVAL  # align
    assert L.slq_mckp_workspace_bytes(224, 221312) >= 2 * 221313 * 8 + 224 * 221313
    assert L.slq_mckp_workspace_bytes(0, 10) == 0
    assert L.slq_row_lse(A, 4, 0, C, E, None) == slq.SLQ_EINVAL
    assert L.slq_row_lse(A, 4, 10, A, E, None) == slq.SLQ_EINVAL                   # lse aliases input
    bad_meta = packed()
    bad_meta.meta = 2
    assert L.slq_dequantize(ctypes.byref(bad_meta), E, None) == slq.SLQ_EINVAL            # layout
    assert L.slq_dequantize(ctypes.byref(packed(scales=C + 4)), E, None) == slq.SLQ_EINVAL  # align
    assert L.slq_scales_bytes(10, 1024, 1) == 160 and L.slq_scales_bytes(10, 1024, 0) == 320
    assert L.slq_zeros_bytes(7, 384, 3, 1) == 11 and L.slq_zeros_bytes(7, 384, 5, 1) == 21
    assert L.slq_zeros_bytes(7, 384, 3, 2) == 0 and L.slq_scales_bytes(7, 100, 0) == 0
    assert L.slq_quant_error(A, ctypes.byref(packed(bits=1)), C, E, None) == slq.SLQ_EINVAL
    assert L.slq_quant_error(A, ctypes.byref(packed()), None, E, None) == slq.SLQ_EINVAL
    assert L.slq_quant_error(A, ctypes.byref(packed()), C, None, None) == slq.SLQ_EINVAL
    assert L.slq_dequantize(ctypes.byref(packed()), None, None) == slq.SLQ_EINVAL
    assert L.slq_dequantize(ctypes.byref(packed()), B, None) == slq.SLQ_EINVAL     # aliases codes


def test_sizes_and_strings():
    L = slq.lib()
    for b in range(2, 9):
        assert L.slq_codes_bytes(4096, 4096, b) == 4096 * 4096 * b // 8
    assert L.slq_codes_bytes(3, 256, 3) == 3 * 256 * 3 // 8
    assert L.slq_codes_bytes(3, 256, 9) == 0
    assert L.slq_gemm_workspace_bytes(1, ctypes.byref(packed(n=1, k=128))) == 0
    assert L.slq_ear_kl_workspace_bytes(512, 151936) > 0
    assert L.slq_quant_error_workspace_bytes(ctypes.byref(packed())) > 0
    name = L.slq_dequant_gemm_kernel_name(1, ctypes.byref(packed(n=4096, k=4096)))
    assert name.startswith(b"slq::gemv_kernel<4, 1,")
    # decode routing by activation rows and layer width (planning only)
    mid, wide = packed(n=4096, k=4096), packed(n=14336, k=4096)
    assert L.slq_dequant_gemm_kernel_name(64, ctypes.byref(mid)) == b"slq::gemv_mk_kernel<4, 4, 1, false>"
    assert L.slq_dequant_gemm_kernel_name(49, ctypes.byref(mid)) == b"slq::gemv_mk_kernel<4, 4, 1, false>"
    assert L.slq_dequant_gemm_kernel_name(48, ctypes.byref(mid)) == b"slq::gemv_mk_kernel<4, 3, 1, false>"
    assert L.slq_dequant_gemm_kernel_name(40, ctypes.byref(mid)).startswith(b"slq::gemv_kernel<4, 3,")
    # layers of 2^25 parameters or more take the tile kernel from 17 rows
    deep = packed(n=4096, k=14336)
    assert L.slq_dequant_gemm_kernel_name(40, ctypes.byref(deep)) == b"slq::gemv_tile_kernel<4, 3, 1, 4, false>"
    assert L.slq_dequant_gemm_kernel_name(49, ctypes.byref(deep)) == b"slq::gemv_tile_kernel<4, 2, 2, 4, false>"
    assert L.slq_dequant_gemm_kernel_name(32, ctypes.byref(deep)) == b"slq::gemv_tile_kernel<4, 2, 1, 4, false>"
    assert L.slq_dequant_gemm_kernel_name(17, ctypes.byref(wide)) == b"slq::gemv_tile_kernel<4, 2, 1, 4, false>"
    assert L.slq_dequant_gemm_kernel_name(64, ctypes.byref(wide)) == b"slq::gemv_tile_kernel<4, 2, 2, 4, false>"
    assert L.slq_dequant_gemm_kernel_name(16, ctypes.byref(wide)).startswith(b"slq::gemv_kernel<4, 1,")
    assert L.slq_dequant_gemm_kernel_name(64, ctypes.byref(packed(n=2048, k=16384))) == (
        b"slq::gemv_tile_kernel<4, 2, 2, 4, false>")
    assert L.slq_dequant_gemm_kernel_name(64, ctypes.byref(packed(n=2047, k=16384))) == (
        b"slq::gemv_rows_kernel<4, 4, false>")
    assert L.slq_dequant_gemm_kernel_name(64, ctypes.byref(packed(n=1024, k=4096))).startswith(
        b"slq::gemv_kernel<4, 4,")
    assert L.slq_dequant_gemm_kernel_name(100, ctypes.byref(packed())) == b"slq::gemm_kernel<4, false>"
    assert L.slq_dequant_gemm_kernel_name(1, ctypes.byref(packed(bits=9))) == b""
    for s in range(4):
        assert L.slq_strerror(s)
    assert L.slq_strerror(0) == b"ok"
