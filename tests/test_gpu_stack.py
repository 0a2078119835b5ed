"""One decode step over the whole 32-layer 7B-shaped stack the benchmark times, on the GPU.

Every layer holds its own weights (drawn on the device from a seed, as the benchmark draws
them) and its own activations; the step runs all 128 projection groups in order through
spax_decode_step_projections in each launch form (fused layer-serial, two launches per group,
batched, fused with the deterministic reduction).  Checked: the masks, lists and
counts of all 128 groups bit for bit against the oracle, every element of every y finite, and
y of every group of the first and the last layer against the oracle (relative L2 1e-3 and the
per-row fp32 bound of tests/parity_util.py; those two layers' weights are copied back to the
host).  fp16 base with TopK-Guided masks at s = 0.5 +- 0.01, and int4 base with TopK
25% / 35% / 40%.
"""

import math

import numpy as np
import pytest

import synth
from oracle import pack as opack
from oracle import tiers as otiers
from tests.parity_util import check_y_oracle

pytestmark = pytest.mark.gpu
SEED = 20240607
LAYERS = 32
CHECKED_LAYERS = (0, LAYERS - 1)


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import activation_sparse_tiered_amd as spax
    return torch, spax, torch.device("cuda:0")


def _rule_args(rule, d_in):
    if rule[0] == "guided":
        _, s, delta = rule
        lo, hi = otiers.guided_bounds(d_in, s, delta)
        return dict(mode=otiers.MODE_TOPK_GUIDED, tau=-math.log(1.0 - s), n_lo=lo, n_hi=hi,
                    num=3, den=10)
    nf, na = otiers.counts_from_fractions(d_in, rule[1], rule[2])
    return dict(mode=otiers.MODE_TOPK, n_full=nf, n_approx=na)


def _params(spax, ra):
    if ra["mode"] == otiers.MODE_TOPK:
        return spax.topk_params(ra["n_full"], ra["n_approx"])
    return spax.guided_params(ra["tau"], ra["n_lo"], ra["n_hi"], ra["num"], ra["den"])


FORMS = [(0, "fused"), (1, "separate"), (2, "batched"), (4, "deterministic")]


@pytest.mark.parametrize("flags", [f for f, _ in FORMS], ids=[n for _, n in FORMS])
@pytest.mark.parametrize("fmt,rule", [(0, ("guided", 0.5, 0.01)), (1, ("topk", 0.25, 0.35))],
                         ids=["fp16-guided-s0.5", "int4-topk-25-35"])
def test_decode_step_32_layers(env, fmt, rule, flags):
    torch, spax, dev = env
    shapes = synth.decoder_phases_7b()
    phases, keep, host_w = [], [], {}
    for l in range(LAYERS):
        for k, (name, d_in, d_out) in enumerate(shapes):
            L = spax.spax_layout_init(d_in, d_out, fmt, 128, 128)
            Ws = [synth.weights_device(SEED, d_in, r, dev, l, k, m) for m, r in enumerate(d_out)]
            packed = torch.empty(int(L.total_bytes), dtype=torch.uint8, device=dev)
            spax.spax_pack_columns(L, Ws, packed)
            if l in CHECKED_LAYERS:
                host_w[(l, k)] = [w.cpu().numpy() for w in Ws]
            del Ws
            x16 = synth.activations(SEED, d_in, l, k)
            ra = _rule_args(rule, d_in)
            b = dict(x=torch.from_numpy(x16).to(dev),
                     tier=torch.full((d_in,), 0xAB, dtype=torch.uint8, device=dev),
                     f=torch.full((d_in,), -7, dtype=torch.int32, device=dev),
                     a=torch.full((d_in,), -7, dtype=torch.int32, device=dev),
                     c=torch.full((3,), -7, dtype=torch.int32, device=dev),
                     y=torch.full((int(L.d_out_total),), float("nan"), dtype=torch.float32,
                                  device=dev))
            phases.append(spax.make_phase(L, packed, b["x"], _params(spax, ra), b["tier"],
                                          b["f"], b["a"], b["c"], b["y"]))
            keep.append((l, k, name, d_in, d_out, x16, ra, b, packed))
    arr = spax.phase_array(phases)
    ws = torch.zeros(max(1, spax.spax_step_workspace_bytes(arr)), dtype=torch.uint8, device=dev)
    print(f"[stack] fmt {fmt} flags {flags}: {len(phases)} groups packed, step enqueued",
          flush=True)
    spax.spax_decode_step_projections(arr, ws, flags=flags)
    torch.cuda.synchronize()
    for l, k, name, d_in, d_out, x16, ra, b, _ in keep:
        args = dict(ra)
        mode = args.pop("mode")
        wt, wf, wa, wc = otiers.build_tiers(x16, mode, **args)
        c = b["c"].cpu().numpy()
        assert list(c) == list(wc), (l, name, c, wc)
        assert np.array_equal(b["tier"].cpu().numpy(), wt), (l, name)
        assert np.array_equal(b["f"].cpu().numpy()[:c[0]], wf), (l, name)
        assert np.array_equal(b["a"].cpu().numpy()[:c[1]], wa), (l, name)
        y = b["y"].cpu().numpy()
        assert np.all(np.isfinite(y)), (l, name)
        if l in CHECKED_LAYERS:
            O = opack.Layout(d_in, d_out, fmt, 128, 128)
            err, worst = check_y_oracle(y, O, host_w[(l, k)], x16, wf, wa,
                                        f"fmt {fmt} flags {flags} layer {l} {name}")
            print(f"[stack] fmt {fmt} flags {flags} layer {l} {name}: rel-L2 {err:.2e}, "
                  f"worst row at {worst:.2e} of its bound", flush=True)
