"""Merged read ranges for the host-resident path.

Oracle (test infrastructure only; see ``oracle/__init__.py``).

eigenradar commentary on SpAx, "The route outside GPU memory", third paragraph: jointly
accessed columns are placed together and adjacent read ranges are merged, and coarse
granularity can move more bytes than the selected columns need; the last paragraph asks
that bytes selected and bytes physically moved be counted apart.

Reading: a range is a maximal run of consecutive selected channels
of one tier, in the packed (channel) order; two runs whose gap is at most ``gap``
unselected channels are merged, and the gap columns are moved too.

Storage granularity (same paragraph: coarse storage granularity can move more bytes than a
selected column needs; last paragraph: for NVMe, selected bytes and bytes physically read
are separate entries).  Reading: the blob sits on a device read in
blocks of ``block`` bytes, the blob starting on a block boundary; each merged range is one
read request, and a request reads every block its bytes touch.  Two requests that touch one
block each read it.
"""

from __future__ import annotations

import numpy as np


def runs(sel_idx, gap: int = 0):
    """Ascending channel indices -> list of (first, count) ranges after gap merging."""
    idx = [int(v) for v in sel_idx]
    out = []
    for j in idx:
        if out and j - (out[-1][0] + out[-1][1]) <= gap:
            first, _ = out[-1]
            out[-1] = (first, j - first + 1)
        else:
            out.append((j, 1))
    return out


def ledger(full_idx, approx_idx, stride_F: int, stride_A: int, gap: int = 0):
    """Selected bytes, moved bytes and range counts for one projection."""
    rf = runs(full_idx, gap)
    ra = runs(approx_idx, gap)
    selected = len(full_idx) * stride_F + len(approx_idx) * stride_A
    moved = sum(c for _, c in rf) * stride_F + sum(c for _, c in ra) * stride_A
    return {"ranges_full": rf, "ranges_approx": ra, "selected_bytes": selected,
            "moved_bytes": moved, "n_ranges": len(rf) + len(ra)}


def compact_positions(ranges):
    """Where each moved column lands in a compacted staging buffer, in range order:
    a list of (channel, slot)."""
    out, slot = [], 0
    for first, count in ranges:
        for k in range(count):
            out.append((first + k, slot))
            slot += 1
    return out


def storage_ledger(full_idx, approx_idx, stride_F: int, stride_A: int, off_A: int,
                   block: int, gap: int = 0):
    """Bytes selected, bytes of the merged record ranges, and bytes physically read at a
    storage granularity of ``block`` bytes, with the counts of ranges and blocks."""
    if block < 1:
        raise ValueError("block must be >= 1")
    reads = []
    for idx, stride, off in ((full_idx, stride_F, 0), (approx_idx, stride_A, off_A)):
        for first, count in runs(idx, gap):
            begin = off + first * stride
            end = begin + count * stride
            reads.append((begin // block, -(-end // block)))   # blocks [b0, b1)
    led = ledger(full_idx, approx_idx, stride_F, stride_A, gap)
    n_blocks = sum(b1 - b0 for b0, b1 in reads)
    return {"selected_bytes": led["selected_bytes"], "moved_bytes": led["moved_bytes"],
            "read_bytes": n_blocks * block, "n_ranges": led["n_ranges"],
            "n_blocks": n_blocks}


def placement_order(calib_tiers, stride_F: int, stride_A: int):
    """Offline placement of the column records (same paragraph: jointly accessed columns are
    placed together).  Reading: from calibration masks (one tier array
    per calibration token: 2 FULL, 1 APPROX, 0 SKIP), each channel scores the bytes it made
    selected (stride_F per FULL, stride_A per APPROX); records are placed by descending score,
    equal scores by channel index.  Returns ``order``: position p of the placed blob holds
    channel order[p]."""
    t = np.asarray(calib_tiers)
    if t.ndim != 2:
        raise ValueError("calibration tiers must be (tokens, d)")
    score = ((t == 2).sum(axis=0).astype(np.int64) * stride_F +
             (t == 1).sum(axis=0).astype(np.int64) * stride_A)
    return np.lexsort((np.arange(t.shape[1]), -score)).astype(np.int32)
