"""The GPTQ oracle's pins must catch plausible mistakes (CPU only): each case
plants one mistake into a copy of oracle/gptq.py, loads it as a module, points
the pins at it and runs them; at least one pin must fail."""
import importlib.util
import inspect
import os
import sys
import tempfile

import pytest

from oracle import gptq as G_real
from tests import test_oracle_gptq as T

SRC = G_real.__file__

MUTANTS = {
    "error_not_scaled_by_diagonal": ("err = (Wk[:, i] - w_hat) / U[i, i]", "err = (Wk[:, i] - w_hat)"),
    "update_sign": ("Wk[:, i + 1:] -= np.outer(err, U[i, i + 1:])",
                    "Wk[:, i + 1:] += np.outer(err, U[i, i + 1:])"),
    "lower_factor": ("return np.linalg.cholesky(Hinv).T", "return np.linalg.cholesky(Hinv)"),
    "factor_of_hessian_not_inverse": ("Hinv = np.linalg.inv(H)\n    return", "Hinv = H\n    return"),
    "group_params_from_original_weights": ("s, z = group_params(Wk[r, i:i + group]",
                                           "s, z = group_params(W[r, i:i + group]"),
    "dead_columns_kept": ("    W[:, dead] = 0.0\n", "    pass\n"),
}


def _load(text, tmp):
    path = os.path.join(tmp, "gptq_mutant.py")
    with open(path, "w") as f:
        f.write(text)
    spec = importlib.util.spec_from_file_location("gptq_mutant", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _pins():
    calls = []
    for name, fn in inspect.getmembers(T, inspect.isfunction):
        if not name.startswith("test_") or fn.__module__ != T.__name__:
            continue
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if params:
            argname, values = params[0].args
            for v in values:
                calls.append(lambda fn=fn, a=argname, v=v: fn(**{a: v}))
        else:
            calls.append(fn)
    return calls


def test_real_oracle_passes():
    for c in _pins():
        c()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor not unique: {name}"
    with tempfile.TemporaryDirectory() as tmp:
        mod = _load(text.replace(old, new), tmp)
        prev = T.G
        T.G = mod
        failed = 0
        try:
            for c in _pins():
                try:
                    c()
                except Exception:
                    failed += 1
        finally:
            T.G = prev
    assert failed, f"no pin catches mutant {name}"
