"""Pins for the oracle's tiered GEMV, decode step and range ledger (host only).

Pinned against exact rational sums (fractions.Fraction) on tiny inputs, special cases
whose answers follow from the three-option definition (SpAx Abstract: all read in full
is the dense product, all skipped is zero), linearity in the tier sets, the error bound
that small activations place on the approximation (SpAx Abstract: small activations
attenuate approximation error), and closed-form byte counts.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import decode, gemv, pack, quant, ranges, tiers


def _rand_case(seed, d_in=None, d_out=None, G=64, base=pack.FMT_FP16):
    rng = np.random.default_rng(seed)
    d_in = d_in or int(rng.integers(1, 24))
    d_out = d_out or [G * int(rng.integers(1, 3)) for _ in range(int(rng.integers(1, 3)))]
    L = pack.Layout(d_in, d_out, base, 128, G)
    Ws = [(rng.standard_normal((d_in, r)) * 0.02).astype(np.float16) for r in d_out]
    x = rng.laplace(size=d_in).astype(np.float16)
    return rng, L, Ws, x


def _exact_sum(cols, x16, sel):
    """Exact rational y_r = sum_j x_j * cols[j][r] (cols float64 values, exact)."""
    T = cols.shape[1]
    y = [Fraction(0)] * T
    for j in sel:
        xj = Fraction(float(x16[j]))
        for r in range(T):
            y[r] += xj * Fraction(float(cols[j, r]))
    return y


@pytest.mark.parametrize("seed", range(8))
def test_gemv_exact_rational(seed):
    """float64 oracle within float64 summation error of the exact rational result, for
    non-square fused matrices (a transposed operand or a wrong index fails)."""
    rng, L, Ws, x = _rand_case(seed)
    nf = int(rng.integers(0, L.d_in + 1))
    na = int(rng.integers(0, L.d_in - nf + 1))
    _, f, a, _ = tiers.build_tiers(x, tiers.MODE_TOPK, n_full=nf, n_approx=na)
    y = gemv.tiered_gemv(L, Ws, x, f, a)
    cat = np.concatenate(Ws, axis=1).astype(np.float64)
    # approximations re-derived per column through the public quantizer
    ap = np.zeros_like(cat)
    for j in range(L.d_in):
        for g0 in range(0, L.d_out_total, L.approx_group):
            s16, z16, q = quant.quantize_group(np.concatenate(Ws, axis=1)[j, g0:g0 + L.approx_group], 2)
            ap[j, g0:g0 + L.approx_group] = quant.dequant(s16, z16, q)
    exact = [a_ + b_ for a_, b_ in zip(_exact_sum(cat, x, f), _exact_sum(ap, x, a))]
    mag = np.abs(cat[f].T @ np.abs(x[f].astype(np.float64))) if len(f) else 0
    for r in range(L.d_out_total):
        bound = 1e-14 * (1 + (mag[r] if len(f) else 0) + 10)
        assert abs(float(exact[r]) - y[r]) <= bound
    # the pure-Python loop version agrees too
    yl = gemv.tiered_gemv_loops(cat.tolist(), ap.tolist(), x.astype(np.float64), f, a)
    assert np.allclose(yl, y, rtol=0, atol=1e-13)


@pytest.mark.parametrize("seed", range(6))
def test_all_full_is_dense_and_all_skip_is_zero(seed):
    rng, L, Ws, x = _rand_case(100 + seed, d_in=int(np.random.default_rng(seed).integers(2, 30)))
    d = L.d_in
    _, f, a, _ = tiers.build_tiers(x, tiers.MODE_TOPK, n_full=d, n_approx=0)
    y = gemv.tiered_gemv(L, Ws, x, f, a)
    cat = np.concatenate(Ws, axis=1)
    exact = _exact_sum(cat.astype(np.float64), x, range(d))
    assert np.allclose([float(v) for v in exact], y, rtol=1e-13, atol=1e-15)
    _, f, a, _ = tiers.build_tiers(x, tiers.MODE_TOPK, n_full=0, n_approx=0)
    y0 = gemv.tiered_gemv(L, Ws, x, f, a)
    assert np.array_equal(y0, np.zeros(L.d_out_total))
    assert not np.signbit(y0).any()


def test_all_approx_on_exact_levels_is_dense():
    """Columns whose groups sit exactly on four power-of-two-spaced levels approximate
    without error, so all-APPROX equals the dense product."""
    rng = np.random.default_rng(7)
    d_in, T, G = 9, 128, 64
    cols = np.zeros((d_in, T))
    for j in range(d_in):
        for g0 in range(0, T, G):
            s = 2.0 ** int(rng.integers(-10, -4))
            z = -(2.0 ** int(rng.integers(-8, -3)))
            k = rng.integers(0, 4, G)
            k[:4] = [0, 1, 2, 3]
            cols[j, g0:g0 + G] = z + k * s
    W = cols.astype(np.float16)
    L = pack.Layout(d_in, [T], pack.FMT_FP16, 128, G)
    x = rng.laplace(size=d_in).astype(np.float16)
    idx = np.arange(d_in)
    ya = gemv.tiered_gemv(L, [W], x, [], idx)
    yf = gemv.tiered_gemv(L, [W], x, idx, [])
    exact = _exact_sum(W.astype(np.float64), x, idx)
    assert np.allclose(ya, yf, rtol=0, atol=1e-15)
    assert np.allclose([float(v) for v in exact], ya, rtol=0, atol=1e-15)


@pytest.mark.parametrize("seed", range(6))
def test_linearity_in_tier_sets(seed):
    rng, L, Ws, x = _rand_case(200 + seed, d_in=40)
    _, f, a, _ = tiers.build_tiers(x, tiers.MODE_TOPK, n_full=10, n_approx=15)
    y = gemv.tiered_gemv(L, Ws, x, f, a)
    yf = gemv.tiered_gemv(L, Ws, x, f, [])
    ya = gemv.tiered_gemv(L, Ws, x, [], a)
    assert np.allclose(y, yf + ya, rtol=0, atol=1e-14)


@pytest.mark.parametrize("seed", range(6))
def test_attenuation_bound(seed):
    """|y_tiered - y_dense| <= sum_A |x_j| s_max(j)/2 (1+2^-9) + sum_S |x_j| max|W[:,j]|."""
    rng, L, Ws, x = _rand_case(300 + seed, d_in=64, d_out=[128, 64], G=64)
    _, f, a, cnt = tiers.build_tiers(x, tiers.MODE_TOPK, n_full=16, n_approx=24)
    skip = [j for j in range(L.d_in) if j not in set(f) | set(a)]
    y = gemv.tiered_gemv(L, Ws, x, f, a)
    cat = np.concatenate(Ws, axis=1)
    y_dense = cat.astype(np.float64).T @ x.astype(np.float64)
    s16, _, _ = quant.quantize_column_groups(cat, L.approx_group, 2)
    smax = s16.astype(np.float64).max(axis=1)
    ax = np.abs(x.astype(np.float64))
    bound = sum(ax[j] * smax[j] / 2 * (1 + 2.0**-9) for j in a) + sum(
        ax[j] * np.abs(cat[j].astype(np.float64)).max() for j in skip)
    assert np.max(np.abs(y - y_dense)) <= bound + 1e-12
    # the bound is not vacuous: the approximate tier's own error is below its share
    y_fa = gemv.tiered_gemv(L, Ws, x, np.concatenate([f, a]).astype(np.int64), [])
    err_a = np.max(np.abs(y - y_fa))
    assert err_a <= sum(ax[j] * smax[j] / 2 * (1 + 2.0**-9) for j in a) + 1e-12


@pytest.mark.parametrize("base", [pack.FMT_FP16, pack.FMT_INT4])
def test_blob_path_equals_definition(base):
    rng, L, Ws, x = _rand_case(400 + base, d_in=33, d_out=[256, 128], G=128, base=base)
    _, f, a, _ = tiers.build_tiers(x, tiers.MODE_TOPK, n_full=9, n_approx=11)
    blob = pack.pack_columns(L, Ws)
    assert np.array_equal(gemv.tiered_gemv_blob(L, blob, x, f, a),
                          gemv.tiered_gemv_values(pack.full_values(L, Ws), pack.approx_values(L, Ws),
                                                  x, f, a))
    assert np.allclose(gemv.tiered_gemv_blob(L, blob, x, f, a), gemv.tiered_gemv(L, Ws, x, f, a),
                       rtol=0, atol=1e-14)


def test_byte_ledger_and_ranges():
    rng = np.random.default_rng(5)
    d = 200
    L = pack.Layout(d, [4096], pack.FMT_FP16, 128, 128)
    x = rng.laplace(size=d).astype(np.float16)
    _, f, a, cnt = tiers.build_tiers(x, tiers.MODE_TOPK, n_full=40, n_approx=60)
    assert decode.selected_bytes(L, cnt) == 40 * 8192 + 60 * 1152
    led = ranges.ledger(f, a, L.stride_F, L.stride_A, gap=0)
    assert led["selected_bytes"] == led["moved_bytes"] == decode.selected_bytes(L, cnt)
    covered = [j for first, c in led["ranges_full"] for j in range(first, first + c)]
    assert covered == list(f)
    # merging with a gap never moves fewer bytes and never makes more ranges
    prev = led
    for g in [1, 2, 5, 1000]:
        cur = ranges.ledger(f, a, L.stride_F, L.stride_A, gap=g)
        assert cur["moved_bytes"] >= prev["moved_bytes"]
        assert cur["n_ranges"] <= prev["n_ranges"]
        prev = cur
    assert prev["n_ranges"] == 2
    assert ranges.runs([3, 4, 5, 9, 10, 20], gap=0) == [(3, 3), (9, 2), (20, 1)]
    assert ranges.runs([3, 4, 5, 9, 10, 20], gap=3) == [(3, 8), (20, 1)]
    assert ranges.compact_positions([(3, 2), (9, 1)]) == [(3, 0), (4, 1), (9, 2)]


@pytest.mark.parametrize("gap", [0, 1, 3, 7])
def test_ranges_characterised_by_their_gaps(gap):
    """Gap merging pinned by what it must produce, not by how: the ranges are disjoint and
    ascending, cover every selected channel and start and end on one, no range holds a run of
    unselected channels longer than the gap, and the channels between two ranges are a run of
    more than gap unselected channels."""
    rng = np.random.default_rng(100 + gap)
    for _ in range(200):
        d = int(rng.integers(1, 60))
        sel = sorted(rng.choice(d, size=int(rng.integers(0, d + 1)), replace=False).tolist())
        rs = ranges.runs(sel, gap)
        chosen = set(sel)
        covered = [j for first, c in rs for j in range(first, first + c)]
        assert covered == sorted(set(covered))                      # disjoint, ascending
        assert chosen <= set(covered)
        for first, c in rs:
            assert first in chosen and first + c - 1 in chosen
            run = 0
            for j in range(first, first + c):
                run = 0 if j in chosen else run + 1
                assert run <= gap
        for (f0, c0), (f1, _) in zip(rs, rs[1:]):
            assert f1 - (f0 + c0) > gap


def _exact_level_matrix(rng, d_in, d_out, G):
    """Column-major fp16 (d_in, d_out) whose every group of G rows holds only the values
    z, z + s, z + 2s, z + 3s, both ends present, with s a power of two and z a multiple of
    s: the two-bit quantizer then recovers s and z exactly and reconstructs every value."""
    W = np.empty((d_in, d_out), dtype=np.float16)
    for j in range(d_in):
        for g0 in range(0, d_out, G):
            s = 2.0 ** int(rng.integers(-9, -5))
            z = s * int(rng.integers(-6, 3))
            q = rng.integers(0, 4, G)
            q[int(rng.integers(0, G))] = 0
            q[int(rng.integers(0, G))] = 3
            W[j, g0:g0 + G] = (z + s * q).astype(np.float16)
    return W


def test_decode_step_pinned_by_brute_force():
    """O5: each phase's mask comes from its own x and parameters, and its y from its own
    weights.  Three phases, two with the same d_in but different x, so a step that crossed
    the phases' inputs fails.  Expected masks: brute-force sort by (|x| descending, index)
    for TopK, float comparison for the threshold, and TopK-Guided with a one-count band
    (delta = 0), which must equal TopK at that count (TopK-Guided section 2.1).  Expected y:
    NumPy's dense float64 product over the kept columns; the weights take exact two-bit
    levels, so the approximation reconstructs them and FULL and APPROX columns contribute
    their plain values."""
    rng = np.random.default_rng(77)
    vals = np.array([0, 0.25, -0.25, 0.5, -1, 1.5, 2, -2, 3], np.float16)
    specs = [
        (6, [64], dict(mode=tiers.MODE_TOPK, n_full=2, n_approx=2)),
        (9, [64, 64], dict(mode=tiers.MODE_THRESHOLD, tau_skip=0.5, tau_full=1.5)),
        (6, [128], dict(mode=tiers.MODE_TOPK_GUIDED, tau=0.3, n_lo=3, n_hi=3, num=1, den=3)),
    ]
    phases = []
    for d_in, d_out, targs in specs:
        L = pack.Layout(d_in, d_out, pack.FMT_FP16, 128, 64)
        Ws = [_exact_level_matrix(rng, d_in, r, 64) for r in d_out]
        x = rng.choice(vals, d_in)
        phases.append(dict(layout=L, Ws=Ws, x=x, tier_args=targs))
    assert not np.array_equal(phases[0]["x"], phases[2]["x"])
    out = decode.decode_step(phases)
    assert len(out) == len(phases)
    for ph, (tier, f, a, c, y) in zip(phases, out):
        x = ph["x"].astype(np.float64)
        d = x.size
        order = sorted(range(d), key=lambda j: (-abs(x[j]), j))
        t = ph["tier_args"]
        if t["mode"] == tiers.MODE_THRESHOLD:
            want_f = [j for j in range(d) if abs(x[j]) >= 1.5]
            want_a = [j for j in range(d) if 0.5 <= abs(x[j]) < 1.5]
        elif t["mode"] == tiers.MODE_TOPK:
            want_f, want_a = sorted(order[:2]), sorted(order[2:4])
        else:  # band [3, 3]: 3 kept, 1 of them APPROX (round-half-up of 3/3 = 1)
            want_f, want_a = sorted(order[:2]), sorted(order[2:3])
        assert list(f) == want_f and list(a) == want_a
        assert list(c) == [len(want_f), len(want_a), d - len(want_f) - len(want_a)]
        assert [int(v) for v in tier] == [2 if j in want_f else 1 if j in want_a else 0
                                          for j in range(d)]
        W = np.concatenate(ph["Ws"], axis=1).astype(np.float64)      # (d_in, T)
        kept = sorted(want_f + want_a)
        ref = W[kept].T @ x[kept] if kept else np.zeros(W.shape[1])
        assert np.array_equal(y, ref) or np.allclose(y, ref, rtol=0, atol=1e-15)
