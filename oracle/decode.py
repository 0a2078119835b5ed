"""One batch-one decode step over the projections of a decoder stack.

Oracle (test infrastructure only; see ``oracle/__init__.py``).

eigenradar commentary on SpAx, "The route outside GPU memory", second and last
paragraphs: selection applies per generated token during batch-one decoding; the
measured unit is bytes moved per token.  A 7B-shaped decoder layer has four groups of
projections that each share one input vector: q|k|v, o, gate|up, down.

Reading: the step is, for each layer and each group in that order,
one tier mask from that group's activation vector followed by one tiered GEMV of the
fused group.  Attention and norms are not part of the path; each group's activation
vector is an independent seeded input.
"""

from __future__ import annotations

from . import gemv, pack, tiers


def decode_step(phases):
    """``phases``: list of dicts with keys ``layout`` (pack.Layout), ``Ws`` (fp16
    column-major matrices), ``x`` (fp16 activations) and ``tier_args`` (keyword
    arguments of :func:`oracle.tiers.build_tiers`, including ``mode``).

    Returns a list of (tier, full_idx, approx_idx, counts, y) per phase.
    """
    out = []
    for ph in phases:
        args = dict(ph["tier_args"])
        mode = args.pop("mode")
        tier, f, a, c = tiers.build_tiers(ph["x"], mode, **args)
        y = gemv.tiered_gemv(ph["layout"], ph["Ws"], ph["x"], f, a)
        out.append((tier, f, a, c, y))
    return out


def selected_bytes(layout: pack.Layout, counts) -> int:
    """Bytes of the column records a mask selects (the per-token byte ledger)."""
    return int(counts[0]) * layout.stride_F + int(counts[1]) * layout.stride_A
