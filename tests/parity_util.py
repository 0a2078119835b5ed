"""Comparison of a device y with the oracle's, shared by the GPU parity tests.

Three checks, all asserted:

* every element of y is finite (the tests fill y with NaN before a call);
* relative L2 over the whole vector <= 1e-3, the tolerance the tiered GEMV is held to for
  fp32 accumulation;
* per row r, |y_gpu[r] - y_ref[r]| <= 1e-5 * sum_{j kept} |x_j| |w_hat[r, j]| + 1e-30, with
  w_hat the value the tier reads (the fp16 weight, or its int4 / two-bit reconstruction).
  This catches a wrong or missing contribution in a few rows that the vector norm would
  hide.  Margin: every kernel sums a row in fp32 with fused multiply-adds along chains of at
  most a few hundred columns per lane, then 16 cross-wave adds and one atomic add per
  column chunk; a quantized column enters as (2^b x s)(1 + q / 2^b) plus x (z - 2^b s), terms
  up to about 15 times |x w_hat|.  Independent roundings of 2^-24 over such chains give
  errors near 1e-7 of the magnitude sum (the measured rel-L2 is about 1e-7), two orders of
  magnitude inside the bound, while a contribution missing or wrong by 1% in a row exceeds
  it (the magnitude sum is 30 to 50 times |y_r| at these sizes).
"""

from __future__ import annotations

import numpy as np

from oracle import pack as opack

REL_L2 = 1e-3
ROW_REL = 1e-5


def rel_l2(got, ref):
    ref = np.asarray(ref, dtype=np.float64)
    num = np.linalg.norm(np.asarray(got, dtype=np.float64) - ref)
    den = np.linalg.norm(ref)
    return num / den if den > 0 else num


def magnitude_sum(O: opack.Layout, Ws, x16, full_idx, approx_idx):
    """sum_{j kept} |x_j| |w_hat[r, j]| per row r."""
    x = np.abs(np.asarray(x16, dtype=np.float16).astype(np.float64))
    f = np.asarray(full_idx, dtype=np.int64)
    a = np.asarray(approx_idx, dtype=np.int64)
    out = np.zeros(O.d_out_total, dtype=np.float64)
    if f.size:
        out += np.abs(opack.full_values(O, Ws, f)).T @ x[f]
    if a.size:
        out += np.abs(opack.approx_values(O, Ws, a)).T @ x[a]
    return out


def row_bound(O: opack.Layout, Ws, x16, full_idx, approx_idx):
    return ROW_REL * magnitude_sum(O, Ws, x16, full_idx, approx_idx) + 1e-30


def check_y(got, ref, bound, what=""):
    """Assert every element finite, rel-L2 <= 1e-3 and |got - ref| <= bound per row.
    Returns (rel-L2, largest |got - ref| / bound)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), (what, "non-finite y", int(np.count_nonzero(~np.isfinite(got))))
    err = rel_l2(got, ref)
    assert err <= REL_L2, (what, "rel-L2", err)
    diff = np.abs(got - ref)
    ratio = diff / bound
    worst = int(np.argmax(ratio))
    assert ratio[worst] <= 1.0, (what, "row", worst, float(diff[worst]), float(bound[worst]))
    return err, float(ratio[worst])


def check_y_oracle(got, O: opack.Layout, Ws, x16, full_idx, approx_idx, what=""):
    """check_y against the oracle's float64 tiered GEMV of these inputs."""
    from oracle import gemv as ogemv
    ref = ogemv.tiered_gemv(O, Ws, x16, full_idx, approx_idx)
    return check_y(got, ref, row_bound(O, Ws, x16, full_idx, approx_idx), what)
