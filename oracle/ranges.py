"""Merged read ranges for the host-resident path.

Oracle (test infrastructure only; see ``oracle/__init__.py``).

eigenradar commentary on SpAx, "The route outside GPU memory", third paragraph: jointly
accessed columns are placed together and adjacent read ranges are merged, and coarse
granularity can move more bytes than the selected columns need; the last paragraph asks
that bytes selected and bytes physically moved be counted apart.

Reading (listed in the design doc): a range is a maximal run of consecutive selected channels
of one tier, in the packed (channel) order; two runs whose gap is at most ``gap``
unselected channels are merged, and the gap columns are moved too.
"""

from __future__ import annotations

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

