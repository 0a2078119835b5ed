"""Host-side sparsity budgets: per-block targets from measured sensitivity, and a greedy
split of a block's target over the projections of the block.

Oracle (test infrastructure only; see ``oracle/__init__.py``).

TopK-Guided (arXiv:2610.01763), section 2.2 "Sensitivity-Aware Block Sparsity": a calibration
pass measures how much each block's output changes when the block is sparsified at a probe
sparsity; blocks more sensitive than average get less sparsity, the global budget moves to the
robust blocks, a strength lambda controls how much moves, and every block target is clamped
to [0.05, 0.95].

TopK-Guided, Appendix D "Block-wise Greedy Sparsity Allocation" (Table 4): the block target
is split over the block's matrices greedily: from zero, each round tries one sparsity
increment on each matrix, keeps the increment whose trial allocation gives the least block
output error, and records the allocation against the block's compute-weighted sparsity
P = sum_m f_m p_m / sum_m f_m (f_m: parameter count).  A matrix's increment is inversely
proportional to its parameter count, so every increment moves P by the same amount.

Readings taken where the pages are silent:

1. Block targets: u_b = s + lambda * (mean(sigma) - sigma_b) / mean(sigma), then
   s_b = clamp(u_b + c, lo, hi) with the one shift c that makes the mean of the s_b equal
   the global target s (the blocks of a decoder stack have equal parameter counts, so the
   mean is the global budget).  c = 0 whenever no target is clamped.
2. Increment of matrix m: alpha * mean(f) / f_m, so a matrix of average size steps by alpha
   and every increment moves P by alpha / n_mats.
3. A matrix is not stepped past sparsity 1.  Ties in the error go to the lower matrix index.
   The walk stops once P reaches the largest budget asked for (or no matrix can step).
4. The allocation for a block target t is the first recorded allocation whose P >= t (all
   zeros for t <= 0).
5. Matrices that multiply one activation vector share one tier mask, so in a decoder layer
   the allocation units are the projection groups (q|k|v, o, gate|up, down), each with the
   summed parameter count of its matrices.
"""

from __future__ import annotations

import numpy as np

CLAMP_LO, CLAMP_HI = 0.05, 0.95


def block_sparsity(sens, s: float, lam: float, lo: float = CLAMP_LO, hi: float = CLAMP_HI):
    """Per-block sparsity targets (reading 1).  ``sens``: positive sensitivities, one per
    block.  Returns a float64 array with mean s (s must lie in [lo, hi])."""
    sig = np.asarray(sens, dtype=np.float64)
    if sig.ndim != 1 or sig.size == 0 or not np.all(sig > 0) or not np.all(np.isfinite(sig)):
        raise ValueError("sensitivities must be finite and positive")
    if not (lo <= s <= hi) or lam < 0 or lo > hi:
        raise ValueError("bad target, strength or clamp")
    mean = sig.mean()
    u = s + lam * (mean - sig) / mean

    def mean_at(c):
        return np.clip(u + c, lo, hi).mean()

    # mean_at is continuous and non-decreasing in c, from lo (c small) to hi (c large):
    # bisection for the shift that gives mean s.
    a, b = lo - u.max() - 1.0, hi - u.min() + 1.0
    for _ in range(200):
        m = 0.5 * (a + b)
        if mean_at(m) < s:
            a = m
        else:
            b = m
    return np.clip(u + 0.5 * (a + b), lo, hi)


def steps(params, alpha: float):
    """Sparsity increment of each matrix (reading 2)."""
    f = np.asarray(params, dtype=np.float64)
    return alpha * f.mean() / f


def compute_weighted(params, p) -> float:
    f = np.asarray(params, dtype=np.float64)
    return float((f * np.asarray(p, dtype=np.float64)).sum() / f.sum())


def greedy_allocation(params, alpha: float, block_error, P_max: float):
    """The recorded trajectory: a list of (P, p) after each committed increment, starting
    with (0, zeros).  ``block_error(p)`` returns the block output error of a trial
    allocation ``p`` (a float64 array)."""
    f = np.asarray(params, dtype=np.float64)
    n = f.size
    st = steps(f, alpha)
    p = np.zeros(n)
    rows = [(0.0, p.copy())]
    while compute_weighted(f, p) < P_max:
        best, best_err = -1, None
        for m in range(n):
            if p[m] + st[m] > 1.0 + 1e-12:
                continue
            trial = p.copy()
            trial[m] += st[m]
            e = float(block_error(trial))
            if best_err is None or e < best_err:
                best, best_err = m, e
        if best < 0:
            break
        p[best] += st[best]
        rows.append((compute_weighted(f, p), p.copy()))
    return rows


def allocation_at(rows, target: float):
    """Reading 4: the first recorded allocation whose P reaches the target."""
    if target <= 0:
        return np.zeros_like(rows[0][1])
    for P, p in rows:
        if P >= target - 1e-12:
            return p.copy()
    return rows[-1][1].copy()
