"""Plain CPU oracle for three-tier activation-sparse decoding GEMV.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (``activation_sparse_tiered_amd``) never imports it, and this package
never imports the product path: the two share no code, no constants and no helpers.

What it computes, and where that is defined:

* SpAx, "Activation Sparsity with Weight Approximation for Faster LLM Decoding on
  Offloaded Weights" (arXiv:2610.02598), Abstract: every weight is either read in its
  original form, read from a compressed approximation, or not read at all; the choice
  follows the magnitude of the activation it multiplies (largest -> original, smaller ->
  approximation, closest to zero -> skipped).
* The eigenradar commentary on SpAx, section "The route outside GPU memory": the
  choice is made per weight *column*, the approximation is two-bit, jointly accessed
  columns are stored together and adjacent read ranges are merged.
* "TopK-Guided: Adaptive, Budget-Aware Activation Sparsity for Efficient LLM
  Inference" (arXiv:2610.01763), section 2.1 "TopK-Guided Masking": a per-token
  natural sparsity estimated from a calibrated threshold, clipped to +-delta around the
  target, then TopK; section 2.2 and Appendix D: per-block targets from measured
  sensitivity and a greedy split of a block's target over its projections.

Modules:

* :mod:`oracle.tiers`  -- magnitude keys, ranking, TOPK / THRESHOLD / TOPK_GUIDED masks,
  host-side conversions (float threshold -> key threshold, fractions -> counts,
  guided clip bounds).
* :mod:`oracle.quant`  -- min-max round-to-nearest group quantizer (2-bit and 4-bit).
* :mod:`oracle.pack`   -- byte-exact column-major packed blob and its decoder.
* :mod:`oracle.gemv`   -- float64 tiered GEMV, from the fp16 master and from a blob.
* :mod:`oracle.ranges` -- merged column ranges for the host-resident path, and the bytes
  physically read from block storage.
* :mod:`oracle.budgets` -- sensitivity-aware block targets and the greedy per-projection
  allocation that produce the per-phase TopK-Guided targets.
* :mod:`oracle.decode` -- one decode step over several projections.

Floating point: the GEMV is float64.  Where floating point decides an integer (a
quantized code, a scale rounded to fp16) the oracle takes the decision in float32 with
round-to-nearest-even, the precision the device kernels use, so that codes can be
compared bit for bit.  Everything else (keys, ranks, counts, byte layout) is integer.

Parity pins live in ``tests/test_oracle_*.py``.  Parity unpinned: whether min-max
round-to-nearest is the quantizer the SpAx authors used (the pages do not say; only the
quantizer's internal consistency and its error bound are pinned), and model quality.
"""

from . import tiers, quant, pack, gemv, ranges, decode, budgets  # noqa: F401
