"""Seeded synthetic inputs (weights and activations) for tests, smoke and bench.

This module holds input recipes only: it draws random numbers and describes workload
shapes.  It contains none of the method's arithmetic (no keys, ranks, counts, quantizer
or packing), so both the oracle side and the device side can take their inputs from it.

Recipes (shapes of the 7B / 8B decoder projections; values are synthetic because no
trained weights or datasets are used):

* weights: W = fp16(0.02 * N(0, 1)), stored column-major as an array of shape
  (d_in, d_out) whose row j is weight column j.
* activations: fp16(Laplace(0, 1)) per token; the "channel-scaled" variant multiplies
  each channel by a per-channel LogNormal(0, 0.5) factor drawn once per seed.

Host arrays come from ``numpy.random.Generator(PCG64(SeedSequence(...)))``; large device
weight sets come from torch's seeded device generator (Philox) so that several GB can be
drawn without a host round trip.  Tests read device-drawn weights back when they need
them on the host.
"""

from __future__ import annotations

import numpy as np

# Stream tags inside one seed.
TAG_WEIGHT, TAG_ACT, TAG_CHANNEL = 1, 2, 3


def rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def weights(seed: int, d_in: int, d_out: int, *tag) -> np.ndarray:
    """fp16 column-major weights (d_in, d_out): row j is column j of W."""
    g = rng(seed, TAG_WEIGHT, d_in, d_out, *tag)
    w = g.standard_normal((d_in, d_out), dtype=np.float32) * np.float32(0.02)
    return w.astype(np.float16)


def channel_scales(seed: int, d: int) -> np.ndarray:
    return rng(seed, TAG_CHANNEL, d).lognormal(0.0, 0.5, d)


def activations(seed: int, d: int, *tag, channel_scaled: bool = False,
                token_scale: float | None = None) -> np.ndarray:
    """fp16 activation vector of length d."""
    g = rng(seed, TAG_ACT, d, *tag)
    v = g.laplace(0.0, 1.0, d)
    if channel_scaled:
        v = v * channel_scales(seed, d)
    if token_scale is not None:
        v = v * token_scale
    return v.astype(np.float16)


def token_scale(seed: int, *tag) -> float:
    """Per-token LogNormal(0, 0.5) scale (pushes a threshold estimate to either side)."""
    return float(rng(seed, 4, *tag).lognormal(0.0, 0.5))


def weights_device(seed: int, d_in: int, d_out: int, device, *tag):
    """Same recipe drawn on the device with torch's seeded generator (fp16, (d_in, d_out))."""
    import torch
    g = torch.Generator(device=device)
    s = int(rng(seed, TAG_WEIGHT, d_in, d_out, *tag).integers(0, 2**62))
    g.manual_seed(s)
    w = torch.randn((d_in, d_out), generator=g, device=device, dtype=torch.float32)
    return (w * 0.02).to(torch.float16)


# --------------------------------------------------------------------------------------
# Workload shapes.  Each phase is a group of matrices that multiply one activation vector.

def decoder_phases_7b():
    """7B-shaped decoder layer: q|k|v, o, gate|up, down (hidden 4096, MLP 11008)."""
    h, m = 4096, 11008
    return [("qkv", h, [h, h, h]), ("o", h, [h]), ("gateup", h, [m, m]), ("down", m, [h])]


def decoder_phases_8b():
    """Llama-3-8B-shaped layer: GQA q|k|v (4096, 1024, 1024), o, gate|up 14336, down."""
    h, m, kv = 4096, 14336, 1024
    return [("qkv", h, [h, kv, kv]), ("o", h, [h]), ("gateup", h, [m, m]), ("down", m, [h])]


def mlp_phases_7b():
    """7B MLP only: gate|up 4096 -> 11008 (fused, shared input), down 11008 -> 4096."""
    h, m = 4096, 11008
    return [("gateup", h, [m, m]), ("down", m, [h])]


WORKLOADS = {
    # name: description used in reports; tiers are given as the workload states them.
    "linear512": dict(phases=[("linear", 512, [512])], layers=1, approx_group=64,
                      tiers=dict(kind="fractions", p_full=0.2, p_approx=0.3),
                      channel_scaled=False),
    "mlp7b": dict(phases=mlp_phases_7b(), layers=1, approx_group=128,
                  tiers=dict(kind="fractions", p_full=0.3, p_approx=0.3),
                  channel_scaled=True),
    "decode7b": dict(phases=decoder_phases_7b(), layers=32, approx_group=128,
                     tiers=dict(kind="guided", s=0.5, delta=0.01, num=3, den=10),
                     channel_scaled=False),
    "decode7b_int4": dict(phases=decoder_phases_7b(), layers=32, approx_group=128,
                          base_fmt="int4",
                          tiers=dict(kind="fractions", p_full=0.25, p_approx=0.35),
                          channel_scaled=False),
    "decode8b_host": dict(phases=decoder_phases_8b(), layers=32, approx_group=128,
                          tiers=dict(kind="fractions", p_full=0.2, p_approx=0.3),
                          channel_scaled=True),
}
