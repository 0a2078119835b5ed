"""Pins for oracle/budgets.py (TopK-Guided section 2.2 and Appendix D), host only.

* Table 4's toy block (tests/golden/budget_table4.json): the walk reaches P = 0.3 at
  pA = 0.5, pB = 0.25 after switching from B to A, and the compute-weighted sparsity of that
  allocation is (100 * 0.5 + 400 * 0.25) / 500 = 0.3.
* Every increment moves P by the same amount (the step is inversely proportional to the
  parameter count).
* On separable convex errors the greedy walk is optimal: brute force over every allocation
  on the step grid with the same P finds no smaller error.
* Block targets: hand-worked cases, the global budget conserved, the clamp, monotonicity in
  the sensitivity and the degenerate strengths.
"""

import itertools
import json
import os

import numpy as np
import pytest

from oracle import budgets

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_table4_toy_block():
    g = json.load(open(os.path.join(GOLDEN, "budget_table4.json")))
    f = g["f"]
    # closed form of the page's compute-weighted sparsity
    assert budgets.compute_weighted(f, g["p_at_P"]) == pytest.approx(g["P"], abs=1e-15)

    # an error model under which B is free up to 0.25 and costly past it, A costly from the
    # start: the walk steps B until it would pass 0.25, then A
    def err(p):
        return p[0] + (0.0 if p[1] <= 0.25 + 1e-12 else 10.0 + p[1])

    rows = budgets.greedy_allocation(f, g["alpha"], err, g["P"])
    order = [int(np.argmax(b[1] - a[1])) for a, b in zip(rows, rows[1:])]
    assert order[0] == g["first_matrix_stepped"]
    assert order[-1] == g["then"]
    assert order == sorted(order, reverse=True)        # all B steps, then all A steps
    P, p = rows[-1]
    assert P == pytest.approx(g["P"], abs=1e-12)
    assert np.allclose(p, g["p_at_P"], rtol=0, atol=1e-12)
    assert np.allclose(budgets.allocation_at(rows, g["P"]), g["p_at_P"], rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(10))
def test_every_increment_moves_P_equally(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 7))
    f = rng.integers(1, 50, n) * 1000
    alpha = float(rng.choice([0.025, 0.05, 0.1]))
    w = rng.uniform(0.1, 3, n)
    rows = budgets.greedy_allocation(f, alpha, lambda p: float((w * p ** 2).sum()), 0.8)
    dP = np.diff([P for P, _ in rows])
    assert np.allclose(dP, alpha / n, rtol=1e-12, atol=1e-15)
    for (_, a), (_, b) in zip(rows, rows[1:]):   # one matrix per round
        assert np.count_nonzero(b != a) == 1


@pytest.mark.parametrize("seed", range(12))
def test_greedy_is_optimal_on_separable_convex_errors(seed):
    """Brute force: every allocation of K increments over the matrices (same P) has at least
    the error of the greedy walk's K-th allocation."""
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(2, 4))
    f = rng.integers(1, 6, n) * 100
    alpha = 0.1
    st = budgets.steps(f, alpha)
    w = rng.uniform(0.2, 2.0, n)
    k = rng.uniform(1.2, 3.0, n)

    def err(p):
        return float((w * np.asarray(p) ** k).sum())

    rows = budgets.greedy_allocation(f, alpha, err, 0.6)
    kmax = [int(np.floor(1.0 / s + 1e-9)) for s in st]
    for K, (P, p) in enumerate(rows):
        best = min(err(np.array(c) * st) for c in itertools.product(*[range(m + 1) for m in kmax])
                   if sum(c) == K)
        assert err(p) <= best + 1e-12, (K, err(p), best)


def test_block_sparsity_hand_worked():
    # sensitivities 1, 2, 3 (mean 2), s = 0.5, lambda = 0.5: 0.5 + 0.5 (2 - sigma) / 2
    assert np.allclose(budgets.block_sparsity([1, 2, 3], 0.5, 0.5), [0.75, 0.5, 0.25], atol=1e-12)
    # lambda = 2: raw 1.5, 0.5, -0.5; clamped to 0.95, 0.5, 0.05, whose mean is already 0.5
    assert np.allclose(budgets.block_sparsity([1, 2, 3], 0.5, 2.0), [0.95, 0.5, 0.05], atol=1e-12)
    # 1, 1, 4 (mean 2), s = 0.3, lambda = 1: raw 0.8, 0.8, -0.7; the third clamps at 0.05 and
    # the other two shift by c: (2 (0.8 + c) + 0.05) / 3 = 0.3 gives c = -0.375
    assert np.allclose(budgets.block_sparsity([1, 1, 4], 0.3, 1.0), [0.425, 0.425, 0.05],
                       atol=1e-12)


@pytest.mark.parametrize("seed", range(20))
def test_block_sparsity_properties(seed):
    rng = np.random.default_rng(200 + seed)
    nb = int(rng.integers(1, 40))
    sig = rng.lognormal(0, 1, nb) * (1 + 5 * np.exp(-np.arange(nb) / 4))
    s = float(rng.choice([0.3, 0.5, 0.7, rng.uniform(0.05, 0.95)]))
    lam = float(rng.choice([0.0, 0.2, 0.4, 0.8, 3.0]))
    t = budgets.block_sparsity(sig, s, lam)
    assert t.mean() == pytest.approx(s, abs=1e-9)                    # budget conserved
    assert np.all(t >= 0.05 - 1e-15) and np.all(t <= 0.95 + 1e-15)  # clamp
    order = np.argsort(sig)
    assert np.all(np.diff(t[order]) <= 1e-12)                        # more sensitive, less sparse
    if lam == 0:
        assert np.allclose(t, s, atol=1e-12)
    assert np.allclose(budgets.block_sparsity(np.full(nb, 2.5), s, lam), s, atol=1e-12)
    inner = (t > 0.05 + 1e-9) & (t < 0.95 - 1e-9)
    if inner.sum() >= 2:  # unclamped targets keep their raw differences
        i, j = np.flatnonzero(inner)[:2]
        assert t[i] - t[j] == pytest.approx(lam * (sig[j] - sig[i]) / sig.mean(), abs=1e-9)


def test_allocation_lookup_and_errors():
    rows = [(0.0, np.zeros(2)), (0.1, np.array([0.0, 0.125])), (0.2, np.array([0.0, 0.25])),
            (0.3, np.array([0.5, 0.25]))]
    assert np.array_equal(budgets.allocation_at(rows, 0.0), [0, 0])
    assert np.array_equal(budgets.allocation_at(rows, 0.15), [0.0, 0.25])
    assert np.array_equal(budgets.allocation_at(rows, 0.3), [0.5, 0.25])
    assert np.array_equal(budgets.allocation_at(rows, 0.9), [0.5, 0.25])
    with pytest.raises(ValueError):
        budgets.block_sparsity([1, -1], 0.5, 0.5)
    with pytest.raises(ValueError):
        budgets.block_sparsity([1, 2], 0.99, 0.5)
