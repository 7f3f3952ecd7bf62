"""The oracle's pins must catch plausible mistakes (CPU only).

Each case plants one mistake into a copy of oracle/oracle.c (a dropped term,
a wrong sign, a wrong index, a transposed operand, the wrong rounding or
reduction), builds it into a temporary library, points the oracle module at
it and runs every pin.  At least one pin must fail for every mutant; the real
oracle must pass them all.
"""
import inspect
import os
import subprocess
import tempfile

import pytest

import oracle
from tests import (test_oracle_compact, test_oracle_fidelity, test_oracle_gamma, test_oracle_gemm,
                   test_oracle_gptq32, test_oracle_mckp, test_oracle_pack, test_oracle_quant,
                   test_oracle_topk)

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")
HDR_DIR = os.path.dirname(SRC)

MUTANTS = {
    "code_drops_zero_point": ("float v = clamp_code(t + (float)z, maxq);", "float v = clamp_code(t, maxq);"),
    "zero_point_sign": ("rintf((-lo) / s)", "rintf(lo / s)"),
    "codes_floor_not_rint": ("float t = rintf(w[i] / s);", "float t = floorf(w[i] / s);"),
    "codes_half_away_from_zero": ("float t = rintf(w[i] / s);", "float t = roundf(w[i] / s);"),
    "range_excludes_zero": ("float lo = 0.0f, hi = 0.0f;", "float lo = w[0], hi = w[0];"),
    "levels_off_by_one": ("s = range / (float)maxq;", "s = range / (float)(maxq + 1);"),
    "symmetric_center": ("z = 1 << (bits - 1);", "z = (1 << (bits - 1)) - 1;"),
    "pack_bit_order_in_code": ("int64_t bit = j * bits + t;\n        if ((code",
                               "int64_t bit = j * bits + (bits - 1 - t);\n        if ((code"),
    "pack_bit_order_in_word": ("out[bit / 32] |= (1u << (bit % 32));", "out[bit / 32] |= (1u << (31 - bit % 32));"),
    "dequant_group_index": ("int64_t g = j / group;", "int64_t g = j % G;"),
    "dequant_drops_zero": ("float d = (float)((int)q[r * k + j] - (int)zeros[r * G + g]);",
                           "float d = (float)((int)q[r * k + j]);"),
    "gemm_transposed_weight": ("double wv = (double)w_hat[c * k + j];", "double wv = (double)w_hat[j * n + c];"),
    "gemm_bound_without_abs": ("b += fabs(xv) * fabs(wv);\n      }\n      y[i",
                               "b += xv * wv;\n      }\n      y[i"),
    "lse_drops_max": ("z += exp((double)a[v] - m);\n  return m + log(z);",
                      "z += exp((double)a[v] - m);\n  return log(z);"),
    "ear_max_not_min": ("double q = exp(lq);\n      e += (p < q) ? p : q;",
                        "double q = exp(lq);\n      e += (p > q) ? p : q;"),
    "kl_reversed": ("double q = exp(lq);\n      e += (p < q) ? p : q;\n      d += p * (lp - lq);",
                    "double q = exp(lq);\n      e += (p < q) ? p : q;\n      d += q * (lq - lp);"),
    "topk_tie_to_higher_index": ("if (cnt == K && !(ar[v] > ar[best[K - 1]])) continue;",
                                 "if (cnt == K && !(ar[v] >= ar[best[K - 1]])) continue;"),
    "topk_selects_smallest": ("while (pos > 0 && ar[v] > ar[best[pos - 1]]) {",
                              "while (pos > 0 && ar[v] < ar[best[pos - 1]]) {"),
    "topk_ear_max_not_min": ("const double p = exp(lp), q = exp(lq);\n      e += (p < q) ? p : q;",
                             "const double p = exp(lp), q = exp(lq);\n      e += (p > q) ? p : q;"),
    "topk_temperature_only_on_p": ("const double lq = (double)br[v] / T - B;",
                                   "const double lq = (double)br[v] - B;"),
    "kl_wrong_normalizer_sign": ("double lq = (double)br[v] - B;", "double lq = (double)br[v] + B;"),
    "mean_over_rows_minus_one": ("means[0] = rows > 0 ? se / (double)rows : 0.0;",
                                 "means[0] = rows > 1 ? se / (double)(rows - 1) : 0.0;"),
    "sse_not_squared": ("rs += e * e;", "rs += fabs(e);"),
    "bpp_meta_per_group": ("(double)meta_bits / (double)group", "(double)meta_bits / (double)(2 * group)"),
    "mckp_size_strictly_below": ("if (sz < 0 || sz > w) continue;", "if (sz < 0 || sz >= w) continue;"),
    "mckp_negative_size_taken": ("if (sz < 0 || sz > w) continue;", "if (sz > w || w - sz >= NW) continue;"),
    "mckp_max_not_min": ("        if (v < b) {\n          b = v;", "        if (!(v < b) || isinf(b)) {\n          b = v;"),
    "mckp_ties_to_higher": ("        if (v < b) {\n          b = v;", "        if (v <= b) {\n          b = v;"),
    "mckp_search_off_by_one": ("      else lo = mid + 1;", "      else lo = mid + 2;"),
    "mckp_readback_wrong_row": ("const int j = pick[l * NW + w];", "const int j = pick[(L - 1 - l) * NW + w];"),
    "f16_round_to_nearest": ("const double r = ceil(v / spacing) * spacing;",
                             "const double r = rint(v / spacing) * spacing;"),
    "f16_spacing_off_by_one": ("ldexp(1.0, E - 10);\n", "ldexp(1.0, E - 9);\n"),
    "f16_value_bias": ("return ldexp(1.0 + (double)f / 1024.0, e - 15);", "return ldexp(1.0 + (double)f / 1024.0, e - 14);"),
    "compact_zero_from_fp32_scale": ("        s = (float)oracle_f16_value(h);\n        z =",
                                     "        z ="),
    "compact_nibble_high_first": ("out[i / 2] |= (uint8_t)((zeros[i] & 15) << (4 * (i % 2)));",
                                  "out[i / 2] |= (uint8_t)((zeros[i] & 15) << (4 * (1 - i % 2)));"),
    "gptq_trailing_sign": ("          w[c] = w[c] - a;", "          w[c] = w[c] + a;"),
    "gptq_no_block_update": ("for (int64_t j = i + 1; j < i1 + group; ++j) w[j] = fmaf(-e[p], U[i * k + j], w[j]);",
                             "/* block update dropped */"),
    "gptq_error_not_scaled": ("e[p] = d / U[i * k + i];", "e[p] = d;"),
    "gptq_trailing_transposed": ("a = fmaf(e[p], U[(i1 + p) * k + c], a);", "a = fmaf(e[p], U[c * k + (i1 + p)], a);"),
    "gptq_trailing_drops_last_term": ("for (int p = 0; p < group; ++p) a = fmaf(",
                                      "for (int p = 0; p < group - 1; ++p) a = fmaf("),
    "gptq_params_from_original": ("          if (w[i1 + p] < glo) glo = w[i1 + p];\n          if (w[i1 + p] > ghi) ghi = w[i1 + p];",
                                  "          if (W[r * k + i1 + p] < glo) glo = W[r * k + i1 + p];\n          if (W[r * k + i1 + p] > ghi) ghi = W[r * k + i1 + p];"),
    "gptq_dead_kept": ("w[c] = (dead && dead[c]) ? 0.0f : W[r * k + c];", "w[c] = W[r * k + c];"),
    "compact_zero_bits_always_4": ("int oracle_compact_zero_bits(int bits) { return bits <= 4 ? 4 : 8; }",
                                   "int oracle_compact_zero_bits(int bits) { return 4; }"),
}


def _pin_calls():
    """Every pin with every parameter value, as zero-argument callables."""
    calls = []
    for mod in (test_oracle_quant, test_oracle_pack, test_oracle_gemm,
                test_oracle_fidelity, test_oracle_gamma, test_oracle_topk, test_oracle_mckp,
                test_oracle_compact, test_oracle_gptq32):
        for name, fn in inspect.getmembers(mod, inspect.isfunction):
            if not name.startswith("test_") or fn.__module__ != mod.__name__:
                continue
            params = inspect.signature(fn).parameters
            grids = [{}]
            for mark in getattr(fn, "pytestmark", []):
                if mark.name == "parametrize":
                    argname, values = mark.args[0], mark.args[1]
                    grids = [dict(g, **{argname: v}) for g in grids for v in values]
            for g in grids:
                kwargs = dict(g)
                if "orc" in params:
                    kwargs["orc"] = oracle
                calls.append((f"{mod.__name__}.{name}{g or ''}", fn, kwargs))
    return calls


def _failures(calls):
    failed = []
    for label, fn, kwargs in calls:
        try:
            fn(**kwargs)
        except Exception:   # AssertionError or a crash-free numerical error
            failed.append(label)
    return failed


@pytest.fixture(scope="module")
def calls():
    return _pin_calls()


def _build(src_text, tmp):
    c = os.path.join(tmp, "oracle.c")
    with open(c, "w") as f:
        f.write(src_text)
    so = os.path.join(tmp, "libmut.so")
    subprocess.run(["gcc", "-O2", "-std=c99", "-fno-fast-math", "-ffp-contract=off", "-fPIC",
                    "-fopenmp", "-I", HDR_DIR, "-shared", c, "-o", so, "-lm"], check=True)
    return oracle.load(so)


def test_real_oracle_passes_all_pins(calls):
    assert len(calls) > 50
    assert _failures(calls) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, calls):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor not unique: {name}"
    with tempfile.TemporaryDirectory() as tmp:
        L = _build(text.replace(old, new), tmp)
        prev = oracle.use(L)
        try:
            failed = _failures(calls)
        finally:
            oracle.use(prev)
    assert failed, f"no pin catches mutant {name}"
