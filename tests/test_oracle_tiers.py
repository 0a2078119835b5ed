"""Pins for the oracle's tier masks (host only).

Each pin checks the oracle against something other than itself: hand-worked fixtures,
brute force over Python floats, or invariants the pages state (realised sparsity within
+-delta, TopK-Guided section 2.1 / section 3; tiers nested by magnitude, SpAx Abstract).
"""

import math
import random

import numpy as np
import pytest

from oracle import tiers
from tests.conftest import load_golden


def _f16(vals):
    return np.array([float(v) for v in vals], dtype=np.float64).astype(np.float16)


def _magnitude_rank_bruteforce(x16):
    """Rank by Python float magnitude (NaN above everything), ties by lower index."""
    def mag(v):
        f = float(v)
        return math.inf if math.isnan(f) else abs(f)

    def is_nan(v):
        return math.isnan(float(v))
    return sorted(range(len(x16)), key=lambda j: (-int(is_nan(x16[j])), -mag(x16[j]), j))


# ---------------------------------------------------------------------- fixtures

def test_key_threshold_golden():
    g = load_golden("key_thresholds.json")
    for c in g["cases"]:
        assert tiers.key_threshold(float(c["tau"])) == c["key"], c


def test_counts_golden():
    g = load_golden("counts_bounds.json")
    for c in g["fractions"]:
        assert tiers.counts_from_fractions(c["d"], c["p_full"], c["p_approx"]) == (
            c["n_full"], c["n_approx"]), c
    for c in g["guided_bounds"]:
        assert tiers.guided_bounds(c["d"], c["s"], c["delta"]) == (c["n_lo"], c["n_hi"]), c


def test_tiers_golden():
    g = load_golden("tiers_tiny.json")
    vecs = {k: _f16(v) for k, v in g["vectors"].items()}
    assert list(tiers.rank_order(tiers.keys_of(vecs["v10"]))) == g["rank_v10"]
    for c in g["cases"]:
        x = vecs[c["x"]]
        if c["mode"] == "topk":
            out = tiers.build_tiers(x, tiers.MODE_TOPK, n_full=c["n_full"], n_approx=c["n_approx"])
        elif c["mode"] == "threshold":
            out = tiers.build_tiers(x, tiers.MODE_THRESHOLD, tau_skip=c["tau_skip"],
                                    tau_full=c["tau_full"])
        else:
            out = tiers.build_tiers(x, tiers.MODE_TOPK_GUIDED, tau=c["tau"], n_lo=c["n_lo"],
                                    n_hi=c["n_hi"], num=c["num"], den=c["den"])
        tier, f, a, cnt = out
        assert list(tier) == c["tier"], c
        assert list(f) == c["full"] and list(a) == c["approx"] and list(cnt) == c["counts"], c


# ---------------------------------------------------------------------- brute force

SMALL_SET = [0.0, -0.0, 0.5, -0.5, 1.0, -1.0, 2.0, float("inf"), -float("inf"), 0.25,
             6e-8, -6e-8, 65504.0]


@pytest.mark.parametrize("seed", range(40))
def test_rank_bruteforce_small(seed):
    r = random.Random(seed)
    d = r.randint(1, 12)
    vals = [r.choice(SMALL_SET + ([float("nan")] if seed % 4 == 0 else [])) for _ in range(d)]
    x = _f16(vals)
    assert list(tiers.rank_order(tiers.keys_of(x))) == _magnitude_rank_bruteforce(x)


@pytest.mark.parametrize("seed", range(20))
def test_key_threshold_matches_float_compare(seed):
    """|x| >= tau  <=>  key >= K(tau), checked with Python floats on every finite half."""
    r = random.Random(seed)
    tau = r.choice([r.uniform(0, 4), r.uniform(0, 1e-4), r.uniform(0, 70000), 0.0,
                    r.uniform(-1, 0)])
    k = tiers.key_threshold(tau)
    allh = np.arange(0x7C01, dtype=np.uint16).view(np.float16)
    mags = np.abs(allh.astype(np.float64))
    keys = tiers.keys_of(allh)
    assert np.array_equal(mags >= tau, keys >= k)


def _check_partition(x, tier, f, a, cnt):
    d = x.size
    assert tier.shape == (d,)
    sets = [set(np.flatnonzero(tier == t)) for t in (tiers.SKIP, tiers.APPROX, tiers.FULL)]
    assert set().union(*sets) == set(range(d))
    assert sum(len(s) for s in sets) == d
    assert list(f) == sorted(sets[2]) and list(a) == sorted(sets[1])
    assert list(cnt) == [len(sets[2]), len(sets[1]), len(sets[0])]
    # monotone in magnitude: every FULL channel outranks every APPROX, which outranks SKIP
    order = _magnitude_rank_bruteforce(x)
    pos = {j: i for i, j in enumerate(order)}
    if sets[2] and sets[1]:
        assert max(pos[j] for j in sets[2]) < min(pos[j] for j in sets[1])
    if sets[1] and sets[0]:
        assert max(pos[j] for j in sets[1]) < min(pos[j] for j in sets[0])
    if sets[2] and sets[0]:
        assert max(pos[j] for j in sets[2]) < min(pos[j] for j in sets[0])


@pytest.mark.parametrize("seed", range(30))
def test_topk_partition_and_order(seed):
    rng = np.random.default_rng(seed)
    d = int(rng.integers(1, 300))
    x = (rng.laplace(size=d) * rng.choice([1, 0.01, 100])).astype(np.float16)
    if seed % 3 == 0:   # many ties
        x = np.round(x).astype(np.float16)
    nf = int(rng.integers(0, d + 1))
    na = int(rng.integers(0, d - nf + 1))
    tier, f, a, cnt = tiers.build_tiers(x, tiers.MODE_TOPK, n_full=nf, n_approx=na)
    _check_partition(x, tier, f, a, cnt)
    assert list(cnt[:2]) == [nf, na]


@pytest.mark.parametrize("seed", range(30))
def test_threshold_matches_float_compare(seed):
    rng = np.random.default_rng(100 + seed)
    d = int(rng.integers(1, 400))
    x = rng.laplace(size=d).astype(np.float16)
    t1, t2 = sorted(rng.uniform(0, 3, 2))
    tier, f, a, cnt = tiers.build_tiers(x, tiers.MODE_THRESHOLD, tau_skip=t1, tau_full=t2)
    mag = np.abs(x.astype(np.float64))
    assert np.array_equal(tier == tiers.FULL, mag >= t2)
    assert np.array_equal(tier == tiers.APPROX, (mag >= t1) & (mag < t2))
    _check_partition(x, tier, f, a, cnt)


# ---------------------------------------------------------------------- TopK-Guided

@pytest.mark.parametrize("seed", range(60))
def test_guided_realised_sparsity_within_delta(seed):
    """TopK-Guided section 2.1 / section 3: realised per-token sparsity within +-delta."""
    rng = np.random.default_rng(1000 + seed)
    d = int(rng.choice([7, 64, 100, 512, 1000, 4096]))
    s = float(rng.choice([0.3, 0.5, 0.7, rng.uniform(0.05, 0.95)]))
    delta = float(rng.choice([0.01, 0.0, 0.05]))
    n_lo, n_hi = tiers.guided_bounds(d, s, delta)
    x = (rng.laplace(size=d) * rng.lognormal(0, 0.7)).astype(np.float16)
    tau = -math.log(1 - s)
    if n_lo > n_hi:
        # An empty integer band: no skip count n has n/d within +-delta of s (brute force
        # over every count), and the mask refuses the band.  Then delta = 1/d, whose band
        # always holds an integer, is checked instead.
        assert not any(s - delta - 1e-12 <= n / d <= s + delta + 1e-12 for n in range(d + 1))
        with pytest.raises(ValueError):
            tiers.build_tiers(x, tiers.MODE_TOPK_GUIDED, tau=tau, n_lo=n_lo, n_hi=n_hi,
                              num=3, den=10)
        delta = 1.0 / d
        n_lo, n_hi = tiers.guided_bounds(d, s, delta)
        assert n_lo <= n_hi
    tier, f, a, cnt = tiers.build_tiers(x, tiers.MODE_TOPK_GUIDED, tau=tau, n_lo=n_lo,
                                        n_hi=n_hi, num=3, den=10)
    n_skip = int(cnt[2])
    assert s - delta - 1e-12 <= n_skip / d <= s + delta + 1e-12
    _check_partition(x, tier, f, a, cnt)
    kept = d - n_skip
    assert int(cnt[1]) == (3 * kept + 5) // 10


@pytest.mark.parametrize("seed", range(30))
def test_guided_inside_band_equals_threshold(seed):
    """If the natural count lies in the band, SKIP is exactly {|x| < tau} (the threshold
    mask, TopK-Guided Abstract / section 1)."""
    rng = np.random.default_rng(2000 + seed)
    d = 2000
    x = rng.laplace(size=d).astype(np.float16)
    tau = float(rng.uniform(0.3, 1.0))
    nat = int(np.count_nonzero(np.abs(x.astype(np.float64)) < tau))
    n_lo, n_hi = max(0, nat - int(rng.integers(0, 20))), min(d, nat + int(rng.integers(0, 20)))
    tier, *_ = tiers.build_tiers(x, tiers.MODE_TOPK_GUIDED, tau=tau, n_lo=n_lo, n_hi=n_hi,
                                 num=1, den=3)
    assert np.array_equal(tier == tiers.SKIP, np.abs(x.astype(np.float64)) < tau)


@pytest.mark.parametrize("seed", range(10))
def test_guided_special_cases(seed):
    rng = np.random.default_rng(3000 + seed)
    d = 1000
    x = rng.laplace(size=d).astype(np.float16)
    # delta = 0 with s*d an integer: pure TopK with n_skip = s*d
    tier, f, a, cnt = tiers.build_tiers(x, tiers.MODE_TOPK_GUIDED, tau=0.7, n_lo=400, n_hi=400,
                                        num=3, den=10)
    ref = tiers.build_tiers(x, tiers.MODE_TOPK, n_full=420, n_approx=180)
    assert np.array_equal(tier, ref[0])
    # band = [0, d]: pure threshold estimate
    tier, *_ = tiers.build_tiers(x, tiers.MODE_TOPK_GUIDED, tau=0.7, n_lo=0, n_hi=d, num=0, den=1)
    assert np.array_equal(tier == tiers.SKIP, np.abs(x.astype(np.float64)) < 0.7)
    # tau = 0 -> natural count 0 -> n_lo ; tau = +inf -> natural count d -> n_hi
    *_, cnt = tiers.build_tiers(x, tiers.MODE_TOPK_GUIDED, tau=0.0, n_lo=123, n_hi=456, num=1, den=2)
    assert cnt[2] == 123
    *_, cnt = tiers.build_tiers(x, tiers.MODE_TOPK_GUIDED, tau=math.inf, n_lo=123, n_hi=456,
                                num=1, den=2)
    assert cnt[2] == 456


def test_guided_bad_params():
    x = np.zeros(10, dtype=np.float16)
    with pytest.raises(ValueError):
        tiers.build_tiers(x, tiers.MODE_TOPK_GUIDED, tau=1.0, n_lo=6, n_hi=5, num=1, den=2)
    with pytest.raises(ValueError):
        tiers.build_tiers(x, tiers.MODE_TOPK_GUIDED, tau=1.0, n_lo=1, n_hi=5, num=1, den=0)
    with pytest.raises(ValueError):
        tiers.build_tiers(x, tiers.MODE_TOPK, n_full=6, n_approx=5)
    with pytest.raises(ValueError):
        tiers.build_tiers(x, tiers.MODE_THRESHOLD, tau_skip=2.0, tau_full=1.0)
