"""Pins for the gamma-squared variance law and the storage accounting (CPU only).

The pages' worked example (gamma = 1.2 raises the noise variance by 44%) and
their bits-per-parameter figures are the fixed values here.
"""
import json
import os

import numpy as np
import pytest

import slq_synth as S

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_worked_values.json")))


def _ratio(orc, W, bits):
    qa, sa, za = orc.quantize(W, bits)
    qs, ss, zs = orc.quantize(W, bits, symmetric=True)
    sse_a, s2_a = orc.quant_error(W, orc.dequantize(qa, sa, za), sa)
    sse_s, s2_s = orc.quant_error(W, orc.dequantize(qs, ss, zs), ss)
    return sse_s / sse_a, s2_s / s2_a, sse_a, sse_s


def test_worked_example_gamma_1p2(orc):
    ex = GOLDEN["gamma_example"]
    g = ex["gamma"]
    # groups uniform on [-0.4, 0.6]: max|w| = 0.6, range 1.0, gamma = 1.2
    W = S.uniform_group_weights(4096, -0.4, 0.6, 31)
    measured, predicted, _, _ = _ratio(orc, W, 4)
    assert abs(predicted - g * g) < 1e-5
    assert abs(measured / (1 + ex["noise_variance_increase"]) - 1) < 0.05


def test_symmetric_data_has_gamma_one(orc):
    W = S.uniform_group_weights(2048, -0.5, 0.5, 32)
    measured, predicted, _, _ = _ratio(orc, W, 4)
    assert abs(predicted - GOLDEN["gamma_symmetric"]["gamma"]) < 1e-6
    assert abs(measured - 1.0) < 0.05


@pytest.mark.parametrize("bits", [3, 4, 6, 8])
def test_skewed_layer_law_and_asymmetry_wins(orc, bits):
    """Skewed layer (the 5120-input layer of the fidelity workload, fewer rows):
    asymmetric SSE is below symmetric at every width, and from 4 bits up the
    measured ratio tracks the s^2-weighted gamma^2 prediction within 5%.  The
    law assumes rounding noise uniform over a bin (s^2/12); at 3 bits the
    +-0.3 outliers make the bins coarse against the bulk of the weights and the
    measured ratio falls below the prediction, so only the ordering is pinned
    there."""
    W = S.skewed_weights(1024, 5120, 500 + bits)
    measured, predicted, sse_a, sse_s = _ratio(orc, W, bits)
    assert sse_a < sse_s
    assert predicted > 1.5
    if bits >= 4:
        assert abs(measured / predicted - 1) < 0.05


def test_direct_sse_matches_quant_error(orc):
    W = S.skewed_weights(16, 256, 9)
    q, s, z = orc.quantize(W, 4)
    wh = orc.dequantize(q, s, z)
    sse, s2 = orc.quant_error(W, wh, s)
    assert abs(sse - ((W.astype(np.float64) - wh) ** 2).sum()) <= 1e-12 * sse
    assert abs(s2 - (s.astype(np.float64) ** 2).sum()) <= 1e-12 * s2


def test_bits_per_param_matches_pages(orc):
    m = GOLDEN["bpp_overhead_map"]
    for b, printed in m["map"].items():
        # 20 bits of scale + zero point per 128-group
        assert round(orc.bits_per_param(int(b), 20, m["group"]), m["printed_decimals"]) == printed
    u = GOLDEN["uniform4_bpp"]
    assert round(orc.bits_per_param(u["bits"], 20, u["group"]), u["printed_decimals"]) == u["bpp"]
    # the fp32 scale + u8 zero layout used by the library: 40 bits per group
    assert orc.bits_per_param(4, 40, 128) == 4.3125
