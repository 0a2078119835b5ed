"""Tier masks: which weight columns are read in full, read approximately, or skipped.

Oracle (test infrastructure only; see ``oracle/__init__.py``).

Definitions followed:

* SpAx Abstract (arXiv:2610.02598): activations closest to zero skip their weights,
  smaller-magnitude activations read approximate weights, the largest-magnitude
  activations read original weights.  So tiers are a function of ``|x_j|`` alone, and
  the three sets are nested by magnitude.
* eigenradar commentary on SpAx, "The route outside GPU memory", first paragraph: the
  unit of choice is one weight column per input channel.
* TopK-Guided (arXiv:2610.01763), Abstract and section 1: a threshold mask adapts the
  count per token; a TopK mask fixes the count per token.
* TopK-Guided section 2.1: the natural sparsity of a token is estimated from the
  calibrated threshold, clipped to a band of +-delta around the target, and TopK is
  then applied with that count; realised sparsity stays within +-delta.

Readings taken where the pages are silent:

1. Magnitude is compared on fp16 bit patterns: ``key = bits(x) & 0x7FFF``.  For
   non-NaN values this order equals the order of ``|x|``; NaN keys (0x7C01..0x7FFF)
   rank above +Inf (0x7C00).
2. Ties: channel j outranks channel k iff ``key_j > key_k`` or
   (``key_j == key_k`` and ``j < k``).  This makes the ranking a total order, so every
   mask has exactly one correct value.
3. A float threshold tau becomes the key threshold K(tau) = the smallest key k in
   [0, 0x7C00] whose half value is >= tau (compared in float64), else 0x7C01.  Then
   ``|x| >= tau`` is ``key >= K(tau)`` for every non-NaN x.
4. Fixed fractions become counts by cumulative round-half-up:
   n_full = floor(p_full*d + 0.5), n_keep = floor((p_full + p_approx)*d + 0.5).
5. TopK-Guided: the natural skip count is c = #{key < K(tau)} (strict), the clip acts
   on the skip count, n_skip = min(max(c, n_lo), n_hi) with
   n_lo = max(0, ceil(d*(s - delta) - 1e-9)), n_hi = min(d, floor(d*(s + delta) + 1e-9)),
   and the kept set is split FULL/APPROX by a fixed ratio num/den of the kept count,
   n_approx = floor((num*kept + floor(den/2)) / den).
"""

from __future__ import annotations

import math

import numpy as np

SKIP, APPROX, FULL = 0, 1, 2
MODE_TOPK, MODE_THRESHOLD, MODE_TOPK_GUIDED = 0, 1, 2

KEY_INF = 0x7C00
KEY_ABOVE_FINITE = 0x7C01


def keys_of(x_f16: np.ndarray) -> np.ndarray:
    """Magnitude key of each fp16 activation: the bit pattern with the sign cleared."""
    x = np.ascontiguousarray(x_f16, dtype=np.float16)
    return (x.view(np.uint16) & np.uint16(0x7FFF)).astype(np.int64)


def key_threshold(tau: float) -> int:
    """K(tau): smallest key in [0, 0x7C00] whose fp16 value is >= tau, else 0x7C01.

    Written as the definition: walk the non-negative finite halves and +Inf in key
    order (which is value order) and return the first one that reaches tau.
    """
    if math.isnan(tau):
        raise ValueError("tau is NaN")
    halves = np.arange(KEY_INF + 1, dtype=np.uint16).view(np.float16).astype(np.float64)
    hits = np.flatnonzero(halves >= float(tau))
    return int(hits[0]) if hits.size else KEY_ABOVE_FINITE


def rank_order(keys: np.ndarray) -> np.ndarray:
    """Channels from highest to lowest rank: key descending, then index ascending."""
    keys = np.asarray(keys, dtype=np.int64)
    idx = np.arange(keys.size, dtype=np.int64)
    # np.lexsort sorts by the last key first.
    return np.lexsort((idx, -keys))


def counts_from_fractions(d: int, p_full: float, p_approx: float) -> tuple[int, int]:
    """Fixed keep fractions -> (n_full, n_approx) by cumulative round-half-up."""
    n_full = int(math.floor(p_full * d + 0.5))
    n_keep = int(math.floor((p_full + p_approx) * d + 0.5))
    n_full = min(max(n_full, 0), d)
    n_keep = min(max(n_keep, n_full), d)
    return n_full, n_keep - n_full


def guided_bounds(d: int, s: float, delta: float) -> tuple[int, int]:
    """Integer skip-count band [n_lo, n_hi] with n_lo/d >= s - delta and n_hi/d <= s + delta."""
    n_lo = max(0, int(math.ceil(d * (s - delta) - 1e-9)))
    n_hi = min(d, int(math.floor(d * (s + delta) + 1e-9)))
    return n_lo, n_hi


def guided_counts(keys: np.ndarray, k_tau: int, n_lo: int, n_hi: int,
                  num: int, den: int) -> tuple[int, int, int]:
    """TopK-Guided section 2.1: natural skip count, clipped, then the FULL/APPROX split.

    Returns (n_full, n_approx, natural_count).
    """
    keys = np.asarray(keys, dtype=np.int64)
    d = keys.size
    natural = int(np.count_nonzero(keys < k_tau))
    n_skip = min(max(natural, n_lo), n_hi)
    kept = d - n_skip
    n_approx = (num * kept + den // 2) // den
    n_approx = min(max(n_approx, 0), kept)
    return kept - n_approx, n_approx, natural


def tiers_topk(keys: np.ndarray, n_full: int, n_approx: int) -> np.ndarray:
    """Ranks 0..n_full-1 -> FULL, the next n_approx -> APPROX, the rest -> SKIP."""
    keys = np.asarray(keys, dtype=np.int64)
    d = keys.size
    if not (0 <= n_full and 0 <= n_approx and n_full + n_approx <= d):
        raise ValueError("counts out of range")
    order = rank_order(keys)
    tier = np.full(d, SKIP, dtype=np.uint8)
    tier[order[:n_full]] = FULL
    tier[order[n_full:n_full + n_approx]] = APPROX
    return tier


def tiers_threshold(keys: np.ndarray, k_skip: int, k_full: int) -> np.ndarray:
    """FULL if key >= K(tau_full); else APPROX if key >= K(tau_skip); else SKIP."""
    keys = np.asarray(keys, dtype=np.int64)
    if k_skip > k_full:
        raise ValueError("skip threshold above full threshold")
    tier = np.full(keys.size, SKIP, dtype=np.uint8)
    tier[keys >= k_skip] = APPROX
    tier[keys >= k_full] = FULL
    return tier


def lists_of(tier: np.ndarray):
    """Ascending index lists of the FULL and APPROX tiers and the counts [F, A, S]."""
    tier = np.asarray(tier)
    full_idx = np.flatnonzero(tier == FULL).astype(np.int32)
    approx_idx = np.flatnonzero(tier == APPROX).astype(np.int32)
    counts = np.array([full_idx.size, approx_idx.size,
                       tier.size - full_idx.size - approx_idx.size], dtype=np.int32)
    return full_idx, approx_idx, counts


def build_tiers(x_f16: np.ndarray, mode: int, *, n_full: int = 0, n_approx: int = 0,
                tau_skip: float = 0.0, tau_full: float = 0.0, tau: float = 0.0,
                n_lo: int = 0, n_hi: int = 0, num: int = 0, den: int = 1):
    """One tier mask for one activation vector.

    Returns (tier u8[d], full_idx i32[], approx_idx i32[], counts i32[3]).
    """
    keys = keys_of(x_f16)
    d = keys.size
    if mode == MODE_TOPK:
        tier = tiers_topk(keys, n_full, n_approx)
    elif mode == MODE_THRESHOLD:
        tier = tiers_threshold(keys, key_threshold(tau_skip), key_threshold(tau_full))
    elif mode == MODE_TOPK_GUIDED:
        if not (0 <= n_lo <= n_hi <= d) or den <= 0 or not (0 <= num <= den):
            raise ValueError("bad guided parameters")
        nf, na, _ = guided_counts(keys, key_threshold(tau), n_lo, n_hi, num, den)
        tier = tiers_topk(keys, nf, na)
    else:
        raise ValueError("unknown mode")
    full_idx, approx_idx, counts = lists_of(tier)
    return tier, full_idx, approx_idx, counts
