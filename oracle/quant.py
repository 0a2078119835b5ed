"""Group quantizer for the compressed column approximation (and the int4 base format).

Oracle (test infrastructure only; see ``oracle/__init__.py``).

The pages fix that the approximate tier reads a two-bit form of each weight column
(eigenradar commentary on SpAx, "The route outside GPU memory": first and third
paragraphs) and that it needs fewer bytes than the original (SpAx Abstract).  They do
not give the quantizer.  Reading taken: asymmetric min-max
round-to-nearest per group of G consecutive rows of one column, reconstructed as
w_hat = s*q + z with z = the group minimum and fp16 s, z.  With L = 2**bits - 1 levels:

1. w (fp16) -> float32 (exact); lo = min w, hi = max w; z32 = lo + 0.0 (turns -0 into +0).
2. s32 = fl32(fl32(hi - lo) / L) with a correctly rounded division; s16 = fp16(s32)
   rounded to nearest even; z16 = fp16(z32), which is exact because lo is an fp16 value.
3. If s16 == 0 every code is 0.  Otherwise
   q = clamp(round_half_even(fl32(fl32(w - z16) / s16)), 0, L).

The same 4-bit quantizer (L = 15, G = 128) is the int4 base format of the original
tier: the SpAx Abstract reports results for 4-bit weights without giving the format.

Every step that decides a code runs in float32, as the device does, so that codes
compare bit for bit.  Dequantization is float64 and exact: s16*q + z16.
"""

from __future__ import annotations

import numpy as np


def levels(bits: int) -> int:
    if bits not in (2, 4):
        raise ValueError("bits must be 2 or 4")
    return (1 << bits) - 1


def quantize_groups(w_f16: np.ndarray, bits: int):
    """Quantize groups along the last axis.

    ``w_f16``: float16 array of shape (..., G).  Returns (s16, z16, q) with s16 and z16
    float16 of shape (...) and q uint8 of shape (..., G).
    """
    L = levels(bits)
    w16 = np.asarray(w_f16, dtype=np.float16)
    if not np.all(np.isfinite(w16)):
        raise ValueError("non-finite weight")
    w = w16.astype(np.float32)
    lo = w.min(axis=-1)
    hi = w.max(axis=-1)
    z32 = (lo + np.float32(0.0)).astype(np.float32)
    rng = (hi - lo).astype(np.float32)
    s32 = (rng / np.float32(L)).astype(np.float32)
    s16 = s32.astype(np.float16)
    z16 = z32.astype(np.float16)
    s_f = s16.astype(np.float32)[..., None]
    z_f = z16.astype(np.float32)[..., None]
    diff = (w - z_f).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (diff / np.where(s_f == 0, np.float32(1.0), s_f)).astype(np.float32)
    q = np.clip(np.rint(t), 0, L)
    q = np.where(s_f == 0, 0, q).astype(np.uint8)
    return s16, z16, q


def quantize_group(w_f16: np.ndarray, bits: int):
    """One group (1-D) -> (s16, z16, q).  Scalar version of :func:`quantize_groups`."""
    s16, z16, q = quantize_groups(np.asarray(w_f16, dtype=np.float16)[None, :], bits)
    return np.float16(s16[0]), np.float16(z16[0]), q[0]


def dequant(s16, z16, q) -> np.ndarray:
    """float64 reconstruction s*q + z (exact in float64)."""
    s = np.asarray(s16, dtype=np.float16).astype(np.float64)
    z = np.asarray(z16, dtype=np.float16).astype(np.float64)
    return s[..., None] * np.asarray(q, dtype=np.float64) + z[..., None]


def quantize_column_groups(col_f16: np.ndarray, group: int, bits: int):
    """Quantize one column (or a stack of columns along axis 0) in groups of rows.

    ``col_f16``: (..., d_out) float16 with d_out % group == 0.
    Returns (s16 (..., d_out/group), z16 (..., d_out/group), q (..., d_out)).
    """
    c = np.asarray(col_f16, dtype=np.float16)
    d_out = c.shape[-1]
    if d_out % group:
        raise ValueError("rows not a multiple of the group size")
    g = c.reshape(c.shape[:-1] + (d_out // group, group))
    s16, z16, q = quantize_groups(g, bits)
    return s16, z16, q.reshape(c.shape)


def dequant_column_groups(s16, z16, q, group: int) -> np.ndarray:
    """Inverse of :func:`quantize_column_groups` in float64."""
    q = np.asarray(q)
    d_out = q.shape[-1]
    g = q.reshape(q.shape[:-1] + (d_out // group, group))
    return dequant(s16, z16, g).reshape(q.shape)
