"""GPU parity of the bit-width allocation (gist.science summary, 3. The SLQ
Pipeline: a multiple-choice knapsack over the cost table, solved exactly under
a budget; SLQ README, Pipeline: the budget is found by bisection until the target is met).

Both sides run the same exact recurrence in fp64 with the same order of
additions and the same tie rule, so every output must be identical: the best
cost for every budget, the budget found, the selection and its size."""
import numpy as np
import pytest
import torch

import oracle
import slq_synth as S
import weight_only_mixed_amd as slq
from tests.gpu_util import gpu, say

pytestmark = pytest.mark.gpu


def check(sizes, costs, W, tau, what):
    ch, res, cost, best = slq.slq_mckp_search(gpu(sizes), gpu(costs), W, tau, with_best=True)
    torch.cuda.synchronize()
    st, och, obud, osize, ocost, obest = oracle.mckp_search(sizes, costs, W, tau, with_best=True)
    ch, res, cost, best = ch.cpu().numpy(), res.cpu().numpy(), cost.cpu().numpy(), best.cpu().numpy()
    say(f"{what}: L={sizes.shape[0]} nb={sizes.shape[1]} W={W} tau={tau:.4g} -> status {res[0]} "
        f"budget {res[1]} size {res[2]} cost {cost[0]:.6g}")
    assert res[0] == st and res[1] == obud and res[2] == osize, (what, res, st, obud, osize)
    assert np.array_equal(ch, och), what
    assert cost[0] == ocost or (np.isinf(cost[0]) and np.isinf(ocost)), what
    assert np.array_equal(best, obest), what
    return ch, res


@pytest.mark.parametrize("seed", range(8))
def test_random_instances(seed):
    g = np.random.default_rng(seed)
    L, nb = int(g.integers(1, 40)), int(g.integers(1, 8))
    sizes = g.integers(0, 50, (L, nb)).astype(np.int64)
    costs = g.random((L, nb)) * 10
    W = int(sizes.max(axis=1).sum())
    mid = float(np.sort(costs, axis=1)[:, nb // 2].sum())
    for tau in (np.inf, mid, float(costs.min(axis=1).sum()), -1.0):
        check(sizes, costs, W, tau, f"seed {seed}")
    check(sizes, costs, max(0, int(sizes.min(axis=1).sum()) - 1), np.inf, "too small a budget")


def test_ties_and_integer_costs():
    """Integer costs make many equal sums: the lower option wins everywhere."""
    g = np.random.default_rng(3)
    sizes = g.integers(1, 6, (30, 5)).astype(np.int64)
    costs = g.integers(0, 4, (30, 5)).astype(np.float64)
    for tau in (np.inf, 20.0, 5.0):
        check(sizes, costs, int(sizes.sum(axis=1).max()) * 3, tau, "ties")


def test_llama3_8b_stack_table():
    """224 projections x bit-widths 2..8 over 221k budgets: the search lands
    k/v, q/o and the MLP in the bit-width classes of the mixed stack."""
    sizes, costs, tau, names = S.allocation_table()
    W = int(sizes.max(axis=1).sum())
    ch, res = check(sizes, costs, W, tau, "Llama-3-8B table")
    bits = np.arange(2, 9)[ch]
    for name, b in zip(names, bits):
        lo, hi = S.BIT_CLASSES[name.split(".")[1]]
        assert lo <= b <= hi, (name, b)
    ch2, res2, cost2, _ = slq.slq_mckp_search(gpu(sizes), gpu(costs), W, tau)
    assert np.array_equal(ch2.cpu().numpy(), ch) and np.array_equal(res2.cpu().numpy(), res)
