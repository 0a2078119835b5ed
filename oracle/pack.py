"""Byte-exact packed weight blob: original columns and co-located two-bit approximations.

Oracle (test infrastructure only; see ``oracle/__init__.py``).

Pages: the eigenradar commentary on SpAx, "The route outside GPU memory", third
paragraph (jointly accessed columns are placed together; adjacent read ranges are
merged), first paragraph (each weight column has an original and a two-bit approximate
form).  The pages give no byte format.  Reading taken:

* Matrices that multiply the same activation vector (q|k|v; gate|up) are fused: each
  column record holds that column of every matrix, concatenated along rows.  One read
  per selected column then serves all of them ("jointly accessed columns together").
* Column-major, one record per input channel j, records in channel order, every record
  zero-padded to a multiple of 128 bytes (one cache line).
* Region F (offset 0): the original column.  fp16: the d_out_total halves, little
  endian.  int4: codes (two rows per byte, row 2k in bits [3:0], row 2k+1 in bits [7:4]),
  then one u32 per group of ``base_group`` rows holding fp16 s in bits [15:0] and fp16 z
  in bits [31:16].
* Region A (offset d_in * stride_F): the two-bit approximation.  Codes four rows per byte
  (row 4k+i in bits [2i+1:2i]), then one u32 (s, z) per group of ``approx_group`` rows.
* The approximation is always quantized from the fp16 master column, also when the
  original tier is int4.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import quant

FMT_FP16, FMT_INT4 = 0, 1
RECORD_ALIGN = 128


def _roundup(v: int, a: int) -> int:
    return (v + a - 1) // a * a


@dataclass
class Layout:
    d_in: int
    d_out: list
    base_fmt: int = FMT_FP16
    base_group: int = 128
    approx_group: int = 128
    # derived
    d_out_total: int = field(init=False)
    rec_F: int = field(init=False)
    rec_A: int = field(init=False)
    stride_F: int = field(init=False)
    stride_A: int = field(init=False)
    off_A: int = field(init=False)
    total_bytes: int = field(init=False)

    def __post_init__(self):
        self.d_out = [int(v) for v in self.d_out]
        if not (1 <= len(self.d_out) <= 4) or self.d_in < 1:
            raise ValueError("bad layout")
        for v in self.d_out:
            if v <= 0 or v % self.approx_group or (
                    self.base_fmt == FMT_INT4 and v % self.base_group):
                raise ValueError("rows must be a multiple of every group size")
        t = sum(self.d_out)
        self.d_out_total = t
        if self.base_fmt == FMT_FP16:
            self.rec_F = 2 * t
        elif self.base_fmt == FMT_INT4:
            self.rec_F = t // 2 + 4 * (t // self.base_group)
        else:
            raise ValueError("unknown base format")
        self.rec_A = t // 4 + 4 * (t // self.approx_group)
        self.stride_F = _roundup(self.rec_F, RECORD_ALIGN)
        self.stride_A = _roundup(self.rec_A, RECORD_ALIGN)
        self.off_A = self.d_in * self.stride_F
        self.total_bytes = self.off_A + self.d_in * self.stride_A


def _sz_words(s16: np.ndarray, z16: np.ndarray) -> np.ndarray:
    s_bits = np.asarray(s16, dtype=np.float16).view(np.uint16).astype(np.uint32)
    z_bits = np.asarray(z16, dtype=np.float16).view(np.uint16).astype(np.uint32)
    return (s_bits | (z_bits << np.uint32(16))).astype("<u4")


def pack_codes(q: np.ndarray, bits: int) -> np.ndarray:
    """Pack codes of shape (..., rows) into bytes, little-endian within each byte."""
    q = np.asarray(q, dtype=np.uint8)
    per = 8 // bits
    rows = q.shape[-1]
    g = q.reshape(q.shape[:-1] + (rows // per, per)).astype(np.uint16)
    out = np.zeros(g.shape[:-1], dtype=np.uint16)
    for i in range(per):
        out |= g[..., i] << np.uint16(bits * i)
    return out.astype(np.uint8)


def unpack_codes(b: np.ndarray, bits: int, rows: int) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint8)
    per = 8 // bits
    mask = (1 << bits) - 1
    out = np.empty(b.shape + (per,), dtype=np.uint8)
    for i in range(per):
        out[..., i] = (b >> (bits * i)) & mask
    return out.reshape(b.shape[:-1] + (rows,))


def fuse_columns(layout: Layout, Ws) -> np.ndarray:
    """Column-major fp16 matrices W[m] of shape (d_in, d_out[m]) -> (d_in, d_out_total)."""
    if len(Ws) != len(layout.d_out):
        raise ValueError("matrix count")
    for W, r in zip(Ws, layout.d_out):
        if W.shape != (layout.d_in, r) or W.dtype != np.float16:
            raise ValueError("matrix shape/dtype")
    return np.concatenate([np.asarray(W) for W in Ws], axis=1)


def pack_columns(layout: Layout, Ws) -> np.ndarray:
    """The whole blob as uint8[total_bytes]."""
    cols = fuse_columns(layout, Ws)              # (d_in, T) fp16
    d_in, T = cols.shape
    blob = np.zeros(layout.total_bytes, dtype=np.uint8)

    region_F = blob[:layout.off_A].reshape(d_in, layout.stride_F)
    if layout.base_fmt == FMT_FP16:
        region_F[:, :2 * T] = cols.astype("<f2").view(np.uint8).reshape(d_in, 2 * T)
    else:
        s16, z16, q = quant.quantize_column_groups(cols, layout.base_group, 4)
        codes = pack_codes(q, 4)                  # (d_in, T/2)
        region_F[:, :T // 2] = codes
        sz = _sz_words(s16, z16).view(np.uint8).reshape(d_in, -1)
        region_F[:, T // 2:T // 2 + sz.shape[1]] = sz

    region_A = blob[layout.off_A:].reshape(d_in, layout.stride_A)
    s16, z16, q = quant.quantize_column_groups(cols, layout.approx_group, 2)
    codes = pack_codes(q, 2)                      # (d_in, T/4)
    region_A[:, :T // 4] = codes
    sz = _sz_words(s16, z16).view(np.uint8).reshape(d_in, -1)
    region_A[:, T // 4:T // 4 + sz.shape[1]] = sz
    return blob


def _decode_quant_region(recs: np.ndarray, T: int, group: int, bits: int) -> np.ndarray:
    per = 8 // bits
    code_bytes = T // per
    q = unpack_codes(recs[:, :code_bytes], bits, T)
    ngroups = T // group
    words = np.ascontiguousarray(recs[:, code_bytes:code_bytes + 4 * ngroups]).view("<u4")
    s16 = (words & 0xFFFF).astype(np.uint16).view(np.float16)
    z16 = (words >> 16).astype(np.uint16).view(np.float16)
    return quant.dequant_column_groups(s16, z16, q, group)


def decode_full_region(layout: Layout, blob: np.ndarray) -> np.ndarray:
    """float64 values of the original tier, shape (d_in, d_out_total)."""
    T, d_in = layout.d_out_total, layout.d_in
    recs = np.asarray(blob, dtype=np.uint8)[:layout.off_A].reshape(d_in, layout.stride_F)
    if layout.base_fmt == FMT_FP16:
        return np.ascontiguousarray(recs[:, :2 * T]).view("<f2").astype(np.float64)
    return _decode_quant_region(recs, T, layout.base_group, 4)


def decode_approx_region(layout: Layout, blob: np.ndarray) -> np.ndarray:
    """float64 values of the two-bit approximation, shape (d_in, d_out_total)."""
    T, d_in = layout.d_out_total, layout.d_in
    recs = np.asarray(blob, dtype=np.uint8)[layout.off_A:layout.total_bytes].reshape(
        d_in, layout.stride_A)
    return _decode_quant_region(recs, T, layout.approx_group, 2)


def full_values(layout: Layout, Ws, cols_sel=None) -> np.ndarray:
    """Original-tier values straight from the definition (no blob): fp16 master, or the
    int4 reconstruction of it.  Shape (d_in, d_out_total) float64, or only the rows of
    the channels in ``cols_sel``."""
    cols = fuse_columns(layout, Ws)
    if cols_sel is not None:
        cols = cols[np.asarray(cols_sel, dtype=np.int64)]
    if layout.base_fmt == FMT_FP16:
        return cols.astype(np.float64)
    s16, z16, q = quant.quantize_column_groups(cols, layout.base_group, 4)
    return quant.dequant_column_groups(s16, z16, q, layout.base_group)


def approx_values(layout: Layout, Ws, cols_sel=None) -> np.ndarray:
    """Two-bit reconstruction straight from the definition (no blob), float64; all
    channels, or only those in ``cols_sel``."""
    cols = fuse_columns(layout, Ws)
    if cols_sel is not None:
        cols = cols[np.asarray(cols_sel, dtype=np.int64)]
    s16, z16, q = quant.quantize_column_groups(cols, layout.approx_group, 2)
    return quant.dequant_column_groups(s16, z16, q, layout.approx_group)
