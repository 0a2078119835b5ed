"""A decode step whose per-phase TopK-Guided targets come from the library's budget helpers
(TopK-Guided section 2.2 block targets, Appendix D greedy split), against the oracle.

The sensitivities and the block error the greedy walk minimises are synthetic (no trained
weights here): sensitivities fall with depth (early blocks more sensitive) times a seeded
LogNormal(0, 0.2) factor; a block's error for a trial allocation is sum_m w_m p_m^2 with
seeded weights per layer.  Four 7B-shaped layers, global target s = 0.5, lambda = 0.4,
alpha = 0.025 over the four projection groups of a layer (their parameter counts).  The
per-phase targets from the C helpers equal the oracle's; each phase's mask uses its target
with delta = 0.01 (tau = -ln(1 - target), the Laplace(0, 1) calibration); masks, lists and
counts bit for bit and y within the parity bar against the oracle, and every phase's
realised sparsity within +-delta of its own target.
"""

import math

import numpy as np
import pytest

import synth
from oracle import budgets
from oracle import pack as opack
from oracle import tiers as otiers
from tests.parity_util import check_y_oracle

pytestmark = pytest.mark.gpu
SEED = 8128
LAYERS = 4


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import activation_sparse_tiered_amd as spax
    return torch, spax, torch.device("cuda:0")


def _synthetic(layers):
    rng = np.random.default_rng(SEED)
    sens = (1 + 4 * np.exp(-np.arange(layers) / 1.5)) * rng.lognormal(0, 0.2, layers)
    w = rng.uniform(0.5, 3.0, (layers, 4))
    return sens, w


@pytest.mark.parametrize("flags", [0, 2])
def test_step_with_budget_targets(env, flags):
    torch, spax, dev = env
    shapes = synth.decoder_phases_7b()
    params = np.array([d_in * sum(d_out) for _, d_in, d_out in shapes], dtype=np.float64)
    sens, w = _synthetic(LAYERS)
    s, lam, alpha, delta = 0.5, 0.4, 0.025, 0.01

    # the library's producers
    s_block = spax.spax_block_sparsity(sens, s, lam)
    targets = []
    for l in range(LAYERS):
        rows = spax.spax_greedy_allocation(params, alpha, float(s_block.max()),
                                           lambda p, wl=w[l]: float((wl * p ** 2).sum()))
        targets.append(spax.spax_allocation_at(rows, float(s_block[l])))
    # the oracle's
    o_block = budgets.block_sparsity(sens, s, lam)
    assert np.allclose(s_block, o_block, rtol=0, atol=1e-12)
    for l in range(LAYERS):
        orows = budgets.greedy_allocation(params, alpha,
                                          lambda p, wl=w[l]: float((wl * p ** 2).sum()),
                                          float(o_block.max()))
        assert np.allclose(targets[l], budgets.allocation_at(orows, float(o_block[l])),
                           rtol=0, atol=1e-12)
    # more sensitive layers are given less sparsity, on the compute-weighted average
    weighted = [budgets.compute_weighted(params, targets[l]) for l in np.argsort(-sens)]
    assert all(a <= b + 1e-12 for a, b in zip(weighted, weighted[1:])), weighted

    phases, keep = [], []
    for l in range(LAYERS):
        for k, (name, d_in, d_out) in enumerate(shapes):
            t = float(targets[l][k])
            L = spax.spax_layout_init(d_in, d_out, 0, 128, 128)
            packed = torch.empty(int(L.total_bytes), dtype=torch.uint8, device=dev)
            Ws = [synth.weights_device(SEED, d_in, r, dev, l, k, m) for m, r in enumerate(d_out)]
            spax.spax_pack_columns(L, Ws, packed)
            x16 = synth.activations(SEED, d_in, l, k)
            lo, hi = spax.spax_guided_bounds(d_in, t, delta)
            olo, ohi = otiers.guided_bounds(d_in, t, delta)
            assert (lo, hi) == (olo, ohi)
            tau = -math.log(1.0 - t)
            b = dict(x=torch.from_numpy(x16).to(dev),
                     tier=torch.empty(d_in, dtype=torch.uint8, device=dev),
                     f=torch.empty(d_in, dtype=torch.int32, device=dev),
                     a=torch.empty(d_in, dtype=torch.int32, device=dev),
                     c=torch.full((3,), -7, dtype=torch.int32, device=dev),
                     y=torch.full((int(L.d_out_total),), float("nan"), dtype=torch.float32,
                                  device=dev))
            phases.append(spax.make_phase(L, packed, b["x"], spax.guided_params(tau, lo, hi, 3, 10),
                                          b["tier"], b["f"], b["a"], b["c"], b["y"]))
            keep.append((l, name, d_in, d_out, Ws, x16, t, tau, lo, hi, b))
    arr = spax.phase_array(phases)
    ws = torch.zeros(max(1, spax.spax_step_workspace_bytes(arr)), dtype=torch.uint8, device=dev)
    print(f"[budgets] flags {flags}: targets {np.round(np.array(targets), 4).tolist()}", flush=True)
    spax.spax_decode_step_projections(arr, ws, flags=flags)
    torch.cuda.synchronize()
    for l, name, d_in, d_out, Ws, x16, t, tau, lo, hi, b in keep:
        wt, wf, wa, wc = otiers.build_tiers(x16, otiers.MODE_TOPK_GUIDED, tau=tau, n_lo=lo,
                                            n_hi=hi, num=3, den=10)
        c = b["c"].cpu().numpy()
        assert list(c) == list(wc), (l, name)
        assert np.array_equal(b["tier"].cpu().numpy(), wt), (l, name)
        assert np.array_equal(b["f"].cpu().numpy()[:c[0]], wf), (l, name)
        assert np.array_equal(b["a"].cpu().numpy()[:c[1]], wa), (l, name)
        assert abs(c[2] / d_in - t) <= delta + 1e-12, (l, name, c[2] / d_in, t)
        Wh = [w_.cpu().numpy() for w_ in Ws]
        check_y_oracle(b["y"].cpu().numpy(), opack.Layout(d_in, d_out, 0, 128, 128), Wh, x16,
                       wf, wa, f"layer {l} {name}")
