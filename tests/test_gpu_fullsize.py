"""GPU parity at the full sizes the benchmark runs.

* One layer of the 7B-shaped decoder (q|k|v 4096 -> 3 x 4096, o 4096 -> 4096, gate|up 4096 ->
  2 x 11008, down 11008 -> 4096) through spax_decode_step_projections in the launch forms the
  benchmark times (fused layer-serial and batched): fp16 base with TopK-Guided masks
  (s = 0.5 +- 0.01, approximate tier 3/10 of the kept channels), and int4 base with TopK
  25% FULL / 35% APPROX / 40% skipped.
* Llama-3-8B-shaped projections (q|k|v 4096 -> 4096 + 1024 + 1024, gate|up 4096 -> 2 x 14336,
  down 14336 -> 4096) with the blob in pinned host memory, TopK 20% / 30% / 50% of
  channel-scaled Laplace activations, through spax_tiered_gemv_pinned in all three transfer
  modes.

Masks, lists and counts are compared with the oracle bit for bit over every channel; y over
every row, against relative L2 1e-3 and the per-row fp32 rounding bound of
tests/parity_util.py, and every element of y must be finite (y starts as NaN).  The byte
account of the pinned path equals the oracle's range ledger.
"""

import math

import numpy as np
import pytest

import synth
from oracle import pack as opack
from oracle import ranges as orng
from oracle import tiers as otiers
from tests.parity_util import check_y_oracle

pytestmark = pytest.mark.gpu
SEED = 424242
GROUP = 128

# (label, base format, tier rule)
LAYER_CASES = [("fp16-guided-s0.5", 0, ("guided", 0.5, 0.01)),
               ("int4-topk-25-35", 1, ("topk", 0.25, 0.35))]


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import activation_sparse_tiered_amd as spax
    return torch, spax, torch.device("cuda:0")


def _tier_args(rule, d_in):
    if rule[0] == "guided":
        _, s, delta = rule
        lo, hi = otiers.guided_bounds(d_in, s, delta)
        return dict(mode=otiers.MODE_TOPK_GUIDED, tau=-math.log(1.0 - s), n_lo=lo, n_hi=hi,
                    num=3, den=10)
    nf, na = otiers.counts_from_fractions(d_in, rule[1], rule[2])
    return dict(mode=otiers.MODE_TOPK, n_full=nf, n_approx=na)


def _params(spax, ta):
    if ta["mode"] == otiers.MODE_TOPK:
        return spax.topk_params(ta["n_full"], ta["n_approx"])
    return spax.guided_params(ta["tau"], ta["n_lo"], ta["n_hi"], ta["num"], ta["den"])


@pytest.mark.parametrize("flags", [0, 2])
@pytest.mark.parametrize("case", LAYER_CASES, ids=[c[0] for c in LAYER_CASES])
def test_decode_layer_7b_full_size(env, case, flags):
    torch, spax, dev = env
    label, fmt, rule = case
    phases, keep = [], []
    for k, (name, d_in, d_out) in enumerate(synth.decoder_phases_7b()):
        L = spax.spax_layout_init(d_in, d_out, fmt, GROUP, GROUP)
        Ws = [synth.weights(SEED, d_in, r, k, m) for m, r in enumerate(d_out)]
        packed = torch.empty(int(L.total_bytes), dtype=torch.uint8, device=dev)
        spax.spax_pack_columns(L, [torch.from_numpy(w).to(dev) for w in Ws], packed)
        x16 = synth.activations(SEED, d_in, k)
        ta = _tier_args(rule, d_in)
        b = dict(x=torch.from_numpy(x16).to(dev),
                 tier=torch.full((d_in,), 0xAB, dtype=torch.uint8, device=dev),
                 f=torch.full((d_in,), -7, dtype=torch.int32, device=dev),
                 a=torch.full((d_in,), -7, dtype=torch.int32, device=dev),
                 c=torch.full((3,), -7, dtype=torch.int32, device=dev),
                 y=torch.full((int(L.d_out_total),), float("nan"), dtype=torch.float32,
                              device=dev))
        phases.append(spax.make_phase(L, packed, b["x"], _params(spax, ta), b["tier"], b["f"],
                                      b["a"], b["c"], b["y"]))
        keep.append((name, d_in, d_out, Ws, x16, ta, b, packed))  # the phase holds raw pointers
    arr = spax.phase_array(phases)
    ws = torch.zeros(max(1, spax.spax_step_workspace_bytes(arr)), dtype=torch.uint8, device=dev)
    print(f"[fullsize] {label} flags {flags}: step enqueued", flush=True)
    spax.spax_decode_step_projections(arr, ws, flags=flags)
    torch.cuda.synchronize()

    for name, d_in, d_out, Ws, x16, ta, b, _ in keep:
        args = dict(ta)
        mode = args.pop("mode")
        wt, wf, wa, wc = otiers.build_tiers(x16, mode, **args)
        c = b["c"].cpu().numpy()
        assert list(c) == list(wc), (name, c, wc)
        assert np.array_equal(b["tier"].cpu().numpy(), wt), name
        assert np.array_equal(b["f"].cpu().numpy()[:c[0]], wf), name
        assert np.array_equal(b["a"].cpu().numpy()[:c[1]], wa), name
        O = opack.Layout(d_in, d_out, fmt, GROUP, GROUP)
        err, worst = check_y_oracle(b["y"].cpu().numpy(), O, Ws, x16, wf, wa,
                                    f"{label} flags {flags} {name}")
        print(f"[fullsize] {label} flags {flags} {name}: rel-L2 {err:.2e}, "
              f"worst row at {worst:.2e} of its bound", flush=True)


PINNED_PHASES = [(name, d_in, d_out) for name, d_in, d_out in synth.decoder_phases_8b()
                 if name in ("qkv", "gateup", "down")]


@pytest.mark.parametrize("transfer", [0, 1, 2])
@pytest.mark.parametrize("phase", PINNED_PHASES, ids=[p[0] for p in PINNED_PHASES])
def test_pinned_projection_8b_full_size(env, phase, transfer):
    """A Llama-3-8B projection group through the pinned-host path: y over every row against
    the oracle, the byte account against the oracle's range ledger."""
    torch, spax, dev = env
    name, d_in, d_out = phase
    L = spax.spax_layout_init(d_in, d_out, 0, GROUP, GROUP)
    O = opack.Layout(d_in, d_out, 0, GROUP, GROUP)
    Ws = [synth.weights(SEED, d_in, r, 8, m) for m, r in enumerate(d_out)]
    packed = torch.empty(int(L.total_bytes), dtype=torch.uint8, device=dev)
    spax.spax_pack_columns(L, [torch.from_numpy(w).to(dev) for w in Ws], packed)
    host = torch.empty(int(L.total_bytes), dtype=torch.uint8, pin_memory=True)
    host.copy_(packed)
    del packed
    x16 = synth.activations(SEED, d_in, 8, channel_scaled=True)
    nF, nA = spax.spax_counts_from_fractions(d_in, 0.2, 0.3)
    x = torch.from_numpy(x16).to(dev)
    f = torch.empty(d_in, dtype=torch.int32, device=dev)
    a = torch.empty(d_in, dtype=torch.int32, device=dev)
    c = torch.zeros(3, dtype=torch.int32, device=dev)
    spax.spax_build_tiers(x, d_in, spax.topk_params(nF, nA), None, f, a, c)
    y = torch.full((int(L.d_out_total),), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty(spax.spax_pinned_workspace_bytes(L), dtype=torch.uint8, device=dev)
    print(f"[fullsize] pinned {name} transfer {transfer}", flush=True)
    st = spax.spax_tiered_gemv_pinned(L, host, x, f, a, c, y, 0, ws, transfer=transfer)
    torch.cuda.synchronize()
    _, wf, wa, wc = otiers.build_tiers(x16, otiers.MODE_TOPK, n_full=nF, n_approx=nA)
    assert list(c.cpu().numpy()) == list(wc)
    check_y_oracle(y.cpu().numpy(), O, Ws, x16, wf, wa, f"pinned {name} transfer {transfer}")
    led = orng.ledger(wf, wa, O.stride_F, O.stride_A, 0)
    assert st.selected_bytes == led["selected_bytes"] and st.moved_bytes == led["moved_bytes"]
    assert st.n_ranges == led["n_ranges"]
