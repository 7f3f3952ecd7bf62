"""Pins of the oracle's bit-width allocation (gist.science summary, "3. The SLQ
Pipeline": a multiple-choice knapsack solved exactly under a budget; SLQ
README, Pipeline: the budget is found by bisection until the target is met).

Readings: one option (bit-width) per item; sizes are integers in budget units;
best(w) is the least total cost with total size <= w; the search returns the
smallest budget whose best cost is <= tau; equal costs go to the lower option
index while reading the selection back from the last item."""
import itertools

import numpy as np
import pytest

import oracle


def brute(sizes, costs, W):
    """All nb^L selections: least cost for every budget, and the argmin set."""
    L, nb = sizes.shape
    best = np.full(W + 1, np.inf)
    for sel in itertools.product(range(nb), repeat=L):
        sz = sum(sizes[l, j] for l, j in enumerate(sel))
        c = sum(costs[l, j] for l, j in enumerate(sel))
        if sz <= W:
            best[sz:] = np.minimum(best[sz:], c)
    return best


def random_instance(rng, L, nb, smax):
    sizes = rng.integers(0, smax + 1, (L, nb)).astype(np.int64)
    costs = rng.random((L, nb))
    return sizes, costs


@pytest.mark.parametrize("seed", range(12))
def test_brute_force(seed):
    rng = np.random.default_rng(seed)
    L, nb = int(rng.integers(1, 6)), int(rng.integers(1, 5))
    sizes, costs = random_instance(rng, L, nb, 6)
    W = int(sizes.sum(axis=1).max() * L // 2 + 3)
    ref = brute(sizes, costs, W)
    for tau in (np.inf, float(np.median(costs.sum(axis=1))), ref[W] + 1e-9, ref[W] - 1e-9):
        st, choice, budget, size, cost, best = oracle.mckp_search(sizes, costs, W, tau, True)
        fin = np.isfinite(ref)
        np.testing.assert_allclose(best[fin], ref[fin], rtol=0, atol=1e-12)
        assert np.array_equal(np.isinf(best), np.isinf(ref))
        ok = np.nonzero(np.isfinite(ref) & (ref <= tau))[0]
        if np.isinf(ref[W]):
            assert st == 2 and (choice == -1).all()
        elif len(ok) == 0:
            assert st == 1 and budget == -1
        else:
            assert st == 0 and budget == ok[0]
            # the selection read back is feasible and optimal at that budget
            sz = sum(sizes[l, j] for l, j in enumerate(choice))
            c = sum(costs[l, j] for l, j in enumerate(choice))
            assert sz == size <= budget and abs(c - cost) < 1e-12 and abs(c - ref[budget]) < 1e-12


def test_monotone_and_no_tau():
    rng = np.random.default_rng(5)
    sizes, costs = random_instance(rng, 12, 7, 20)
    W = int(sizes.sum(axis=1).max() * 12 // 2)
    st, choice, budget, size, cost, best = oracle.mckp_search(sizes, costs, W, np.inf, True)
    fin = best[np.isfinite(best)]
    assert np.all(np.diff(fin) <= 0)
    # tau = inf: the smallest budget is the sum of the items' smallest sizes
    assert st == 0 and budget == sizes.min(axis=1).sum()


def test_convex_items_match_marginal_greedy():
    """Separable convex costs with unit size steps (option j of item l: size j,
    cost a_l 4^-j, the noise-variance law per bit): the optimum at budget w
    takes the w largest marginal gains, a textbook exchange argument."""
    rng = np.random.default_rng(9)
    L, nb = 9, 7
    a = rng.random(L) * 10 + 0.5
    sizes = np.tile(np.arange(nb, dtype=np.int64), (L, 1))
    costs = a[:, None] * 4.0 ** -np.arange(nb)[None, :]
    W = L * (nb - 1)
    st, choice, budget, size, cost, best = oracle.mckp_search(sizes, costs, W, np.inf, True)
    gains = np.sort((a[:, None] * (4.0 ** -np.arange(nb - 1) - 4.0 ** -np.arange(1, nb))).ravel())[::-1]
    for w in range(W + 1):
        assert abs(best[w] - (costs[:, 0].sum() - gains[:w].sum())) < 1e-9


def test_single_item_and_infeasible():
    sizes = np.array([[3, 5, 8]], np.int64)
    costs = np.array([[9.0, 4.0, 1.0]])
    st, choice, budget, size, cost, best = oracle.mckp_search(sizes, costs, 10, 4.0, True)
    assert list(best) == [np.inf] * 3 + [9.0] * 2 + [4.0] * 3 + [1.0] * 3
    assert st == 0 and budget == 5 and choice[0] == 1 and size == 5 and cost == 4.0
    st, choice, *_ = oracle.mckp_search(sizes, costs, 2, 4.0)
    assert st == 2 and choice[0] == -1
    st, choice, budget, size, cost = oracle.mckp_search(sizes, costs, 6, 0.5)
    assert st == 1 and budget == -1 and choice[0] == 1 and cost == 4.0


def test_ties_go_to_the_lower_option():
    sizes = np.array([[1, 1, 1], [2, 2, 2]], np.int64)
    costs = np.array([[1.0, 1.0, 1.0], [2.0, 2.0, 2.0]])
    st, choice, budget, size, cost = oracle.mckp_search(sizes, costs, 5, 3.0)
    assert st == 0 and budget == 3 and list(choice) == [0, 0]


def test_negative_sizes_are_never_selected():
    """An option with a negative size is not available: the optimum equals the
    brute force over the remaining options (a very negative size would
    otherwise look like free storage), for every budget."""
    rng = np.random.default_rng(77)
    for t in range(6):
        sizes, costs = random_instance(rng, 4, 3, 5)
        sizes[rng.integers(0, 4), rng.integers(0, 3)] = -1000 if t % 2 else -1
        costs[sizes < 0] = -1.0          # tempting: the cheapest option of its item
        W = 12
        allowed = np.where(sizes < 0, W + 1000, sizes)   # out of every budget
        ref = brute(allowed, costs, W)
        st, choice, budget, size, cost, best = oracle.mckp_search(sizes, costs, W, np.inf, True)
        fin = np.isfinite(ref)
        np.testing.assert_allclose(best[fin], ref[fin], rtol=0, atol=1e-12)
        assert np.array_equal(np.isinf(best), np.isinf(ref))
        if st != 2:
            assert all(sizes[l, j] >= 0 for l, j in enumerate(choice))
