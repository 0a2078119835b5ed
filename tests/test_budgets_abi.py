"""The host-side budget helpers of the C ABI (spax_block_sparsity, spax_greedy_allocation,
spax_allocation_at) against oracle/budgets.py, and their error handling.  Host only."""

import json
import os

import numpy as np
import pytest

import activation_sparse_tiered_amd as spax
from activation_sparse_tiered_amd import _lib
from oracle import budgets

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("seed", range(20))
def test_block_sparsity_matches_oracle(seed):
    rng = np.random.default_rng(300 + seed)
    nb = int(rng.integers(1, 64))
    sig = rng.lognormal(0, 1, nb) * (1 + 4 * np.exp(-np.arange(nb) / 3))
    s = float(rng.uniform(0.05, 0.95))
    lam = float(rng.choice([0.0, 0.2, 0.4, 0.6, 0.8, 2.0]))
    got = spax.spax_block_sparsity(sig, s, lam)
    assert np.allclose(got, budgets.block_sparsity(sig, s, lam), rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(12))
def test_greedy_allocation_matches_oracle(seed):
    rng = np.random.default_rng(400 + seed)
    n = int(rng.integers(1, 8))
    f = (rng.integers(1, 60, n) * 4096).astype(np.float64)
    alpha = float(rng.choice([0.025, 0.05, 0.1]))
    w = rng.uniform(0.1, 4, n)
    k = rng.uniform(1.0, 3.0, n)

    def err(p):
        return float((w * np.asarray(p) ** k).sum())

    P_max = float(rng.uniform(0.1, 0.9))
    got = spax.spax_greedy_allocation(f, alpha, P_max, err)
    want = budgets.greedy_allocation(f, alpha, err, P_max)
    assert got.shape == (len(want), 1 + n)
    for r, (P, p) in zip(got, want):
        assert r[0] == pytest.approx(P, abs=1e-12)
        assert np.allclose(r[1:], p, rtol=0, atol=1e-12)
    for t in (0.0, P_max / 3, P_max, 2.0):
        assert np.allclose(spax.spax_allocation_at(got, t), budgets.allocation_at(want, t),
                           rtol=0, atol=1e-12)


def test_table4_through_the_abi():
    g = json.load(open(os.path.join(GOLDEN, "budget_table4.json")))
    rows = spax.spax_greedy_allocation(
        g["f"], g["alpha"], g["P"], lambda p: p[0] + (0.0 if p[1] <= 0.25 + 1e-12 else 10 + p[1]))
    assert rows[-1][0] == pytest.approx(g["P"], abs=1e-12)
    assert np.allclose(spax.spax_allocation_at(rows, g["P"]), g["p_at_P"], rtol=0, atol=1e-12)


def test_budget_errors():
    with pytest.raises(spax.SpaxError) as e:
        spax.spax_block_sparsity([1.0, 0.0], 0.5, 0.4)
    assert e.value.status == _lib.SPAX_ERR_PARAM
    with pytest.raises(spax.SpaxError):
        spax.spax_block_sparsity([1.0, 2.0], 0.99, 0.4)
    with pytest.raises(spax.SpaxError):
        spax.spax_block_sparsity([1.0, 2.0], 0.5, -0.1)
    with pytest.raises(spax.SpaxError):
        spax.spax_greedy_allocation([100.0, -1.0], 0.1, 0.3, lambda p: 0.0)
    with pytest.raises(spax.SpaxError):
        spax.spax_greedy_allocation([100.0], 0.0, 0.3, lambda p: 0.0)
    # too few rows: SPAX_ERR_WORKSPACE with the count needed (the binding then retries)
    import ctypes as C
    f = np.array([100.0, 400.0])
    rows = np.zeros((2, 3))
    nr = C.c_int32()
    cb = _lib.BLOCK_ERROR_FN(lambda p, n, u: 0.0)
    st = _lib.lib.spax_greedy_allocation(f.ctypes.data, 2, 0.1, 0.3, cb, None, rows.ctypes.data,
                                         2, C.byref(nr))
    assert st == _lib.SPAX_ERR_WORKSPACE and nr.value == 7


def test_greedy_rejects_tiny_alpha_and_nonfinite_errors():
    with pytest.raises(spax.SpaxError) as e:  # 2e8 increments to take both matrices to 1
        spax.spax_greedy_allocation([100.0, 100.0], 1e-8, 0.3, lambda p: 0.0)
    assert e.value.status == _lib.SPAX_ERR_PARAM and "too small" in str(e.value)
    with pytest.raises(spax.SpaxError) as e:
        spax.spax_greedy_allocation([100.0, 400.0], 0.1, 0.3,
                                    lambda p: float("nan") if p[1] > 0 else 0.0)
    assert e.value.status == _lib.SPAX_ERR_PARAM and "block_error" in str(e.value)
