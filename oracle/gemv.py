"""float64 three-tier GEMV at batch one.

Oracle (test infrastructure only; see ``oracle/__init__.py``).

SpAx Abstract (arXiv:2610.02598) and the eigenradar commentary, "The route outside GPU
memory", first paragraph: per input channel j, the weight column W[:, j] is read in its
original form (FULL), read as its two-bit approximation (APPROX) or not read (SKIP).
The product is therefore

    y_r = sum_{j in FULL} x_j * W[r, j]  +  sum_{j in APPROX} x_j * W_hat[r, j]

with W_hat the reconstruction of the approximation.  Skipped channels contribute
nothing.  Computed in float64; the fp16 activations and the fp16 / reconstructed weights
are exact in float64, so the only rounding is the float64 summation.
"""

from __future__ import annotations

import numpy as np

from . import pack


def tiered_gemv_values(full_vals: np.ndarray, approx_vals: np.ndarray, x_f16: np.ndarray,
                       full_idx, approx_idx) -> np.ndarray:
    """``full_vals`` / ``approx_vals``: (d_in, d_out) float64 per-channel columns."""
    x = np.asarray(x_f16, dtype=np.float16).astype(np.float64)
    f = np.asarray(full_idx, dtype=np.int64)
    a = np.asarray(approx_idx, dtype=np.int64)
    d_out = full_vals.shape[1]
    y = np.zeros(d_out, dtype=np.float64)
    if f.size:
        y += full_vals[f].T @ x[f]
    if a.size:
        y += approx_vals[a].T @ x[a]
    return y


def tiered_gemv(layout: pack.Layout, Ws, x_f16, full_idx, approx_idx) -> np.ndarray:
    """From the fp16 master matrices, by the definition (no blob)."""
    f = np.asarray(full_idx, dtype=np.int64)
    a = np.asarray(approx_idx, dtype=np.int64)
    x = np.asarray(x_f16, dtype=np.float16).astype(np.float64)
    y = np.zeros(layout.d_out_total, dtype=np.float64)
    if f.size:
        y += pack.full_values(layout, Ws, f).T @ x[f]
    if a.size:
        y += pack.approx_values(layout, Ws, a).T @ x[a]
    return y


def tiered_gemv_blob(layout: pack.Layout, blob, x_f16, full_idx, approx_idx) -> np.ndarray:
    """From a packed blob, decoded by the oracle's own decoder."""
    return tiered_gemv_values(pack.decode_full_region(layout, blob),
                              pack.decode_approx_region(layout, blob),
                              x_f16, full_idx, approx_idx)


def tiered_gemv_loops(full_cols, approx_cols, x, full_idx, approx_idx):
    """Pure-Python loops over channels and rows, for tiny cases only.

    ``full_cols[j][r]`` and ``approx_cols[j][r]`` are Python floats.
    """
    d_out = len(full_cols[0]) if len(full_cols) else 0
    y = [0.0] * d_out
    for j in full_idx:
        for r in range(d_out):
            y[r] += float(x[j]) * full_cols[j][r]
    for j in approx_idx:
        for r in range(d_out):
            y[r] += float(x[j]) * approx_cols[j][r]
    return y

