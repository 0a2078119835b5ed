"""spax_decode_step_projections_noalloc: the decode step with no workspace (the batched form's
descriptor tables in the library's static device scratch), through the C ABI, against
spax_decode_step_projections on the same phases: masks, lists and counts bit for bit, y
within the parity bar of the oracle and within fp32 reordering of the other entry point's.
Two calls in a row, the second over fewer and smaller phases, so stale tables of the first
call sit past the second's in the scratch."""

import math

import numpy as np
import pytest

import synth
from oracle import pack as opack
from oracle import tiers as otiers
from tests.parity_util import check_y_oracle, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import activation_sparse_tiered_amd as spax
    return torch, spax, torch.device("cuda:0")


def _args(rule, d):
    kind = rule[0]
    if kind == "topk":
        nf, na = otiers.counts_from_fractions(d, rule[1], rule[2])
        return dict(mode=otiers.MODE_TOPK, n_full=nf, n_approx=na)
    if kind == "threshold":
        return dict(mode=otiers.MODE_THRESHOLD, tau_skip=rule[1], tau_full=rule[2])
    lo, hi = otiers.guided_bounds(d, rule[1], rule[2])
    return dict(mode=otiers.MODE_TOPK_GUIDED, tau=-math.log(1 - rule[1]), n_lo=lo, n_hi=hi,
                num=3, den=10)


def _params(spax, a):
    if a["mode"] == otiers.MODE_TOPK:
        return spax.topk_params(a["n_full"], a["n_approx"])
    if a["mode"] == otiers.MODE_THRESHOLD:
        return spax.threshold_params(a["tau_skip"], a["tau_full"])
    return spax.guided_params(a["tau"], a["n_lo"], a["n_hi"], a["num"], a["den"])


def _build(env, specs, seed):
    torch, spax, dev = env
    keep = []
    for i, (d_in, d_out, fmt, G, rule) in enumerate(specs):
        L = spax.spax_layout_init(d_in, d_out, fmt, 128, G)
        O = opack.Layout(d_in, d_out, fmt, 128, G)
        Ws = [synth.weights(seed + i, d_in, r, m) for m, r in enumerate(d_out)]
        packed = torch.empty(int(L.total_bytes), dtype=torch.uint8, device=dev)
        spax.spax_pack_columns(L, [torch.from_numpy(w).to(dev) for w in Ws], packed)
        x16 = synth.activations(seed, d_in, i)
        a = _args(rule, d_in)
        b = dict(x=torch.from_numpy(x16).to(dev),
                 tier=torch.empty(d_in, dtype=torch.uint8, device=dev),
                 f=torch.empty(d_in, dtype=torch.int32, device=dev),
                 a=torch.empty(d_in, dtype=torch.int32, device=dev),
                 c=torch.empty(3, dtype=torch.int32, device=dev),
                 y=torch.empty(int(L.d_out_total), dtype=torch.float32, device=dev))
        keep.append((L, O, Ws, x16, a, packed, b))
    phases = [spax.make_phase(L, packed, b["x"], _params(spax, a), b["tier"], b["f"], b["a"],
                              b["c"], b["y"]) for (L, O, Ws, x16, a, packed, b) in keep]
    return keep, spax.phase_array(phases)


def _clobber(keep):
    for *_, b in keep:
        b["tier"].fill_(0xAB)
        b["f"].fill_(-7)
        b["a"].fill_(-7)
        b["c"].fill_(-7)
        b["y"].fill_(float("nan"))


def _snapshot(keep):
    return [{k: b[k].clone() for k in ("tier", "f", "a", "c", "y")} for *_, b in keep]


def _compare(env, keep, arr, flags, what):
    torch, spax, dev = env
    ws = torch.zeros(max(1, spax.spax_step_workspace_bytes(arr)), dtype=torch.uint8, device=dev)
    _clobber(keep)
    spax.spax_decode_step_projections(arr, ws, flags=flags)
    torch.cuda.synchronize()
    want = _snapshot(keep)
    _clobber(keep)
    print(f"[no-alloc] {what}: flags {flags}, {len(keep)} phases", flush=True)
    spax.spax_decode_step_projections_noalloc(arr, flags=flags)
    torch.cuda.synchronize()
    for i, ((L, O, Ws, x16, a, packed, b), w) in enumerate(zip(keep, want)):
        c = w["c"].cpu().numpy()
        args = dict(a)
        mode = args.pop("mode")
        wt, wf, wa, wc = otiers.build_tiers(x16, mode, **args)
        assert list(c) == list(wc), (what, i)
        assert torch.equal(b["c"], w["c"]), (what, i)
        assert torch.equal(b["tier"], w["tier"]), (what, i)
        assert torch.equal(b["f"][:c[0]], w["f"][:c[0]]), (what, i)
        assert torch.equal(b["a"][:c[1]], w["a"][:c[1]]), (what, i)
        y = b["y"].cpu().numpy()
        check_y_oracle(y, O, Ws, x16, wf, wa, f"{what} phase {i}")
        assert rel_l2(y, w["y"].cpu().numpy()) <= 1e-6, (what, i)


@pytest.mark.parametrize("flags", [2, 0])
def test_noalloc_matches_step_with_workspace(env, flags):
    big = [(4096, [4096, 1024, 1024], 0, 128, ("guided", 0.5, 0.01)),
           (4096, [4096], 0, 128, ("topk", 0.2, 0.3)),
           (4096, [2816, 2816], 1, 128, ("topk", 0.25, 0.35)),
           (2816, [4096], 0, 64, ("threshold", 0.5, 1.5)),
           (11008, [512], 0, 128, ("guided", 0.7, 0.01)),
           (20000, [256], 0, 128, ("guided", 0.3, 0.01))]
    small = [(1536, [1024], 1, 128, ("topk", 0.3, 0.3)),
             (640, [512], 0, 64, ("guided", 0.5, 0.02))]
    keep1, arr1 = _build(env, big, 61)
    _compare(env, keep1, arr1, flags, "first call")
    keep2, arr2 = _build(env, small, 62)
    _compare(env, keep2, arr2, flags, "second, smaller call")


def test_noalloc_rejects_too_many_phases(env):
    """More phases than the static scratch holds tables for: SPAX_ERR_WORKSPACE before
    anything is enqueued (outputs untouched)."""
    torch, spax, dev = env
    keep, _ = _build(env, [(256, [256], 0, 128, ("topk", 0.2, 0.3))], 63)
    L, O, Ws, x16, a, packed, b = keep[0]
    # 1300 phases over disjoint outputs (about 208 bytes of tables each: past 256 KiB)
    outs = [dict(tier=torch.empty(256, dtype=torch.uint8, device=dev),
                 f=torch.empty(256, dtype=torch.int32, device=dev),
                 a=torch.empty(256, dtype=torch.int32, device=dev),
                 c=torch.full((3,), -7, dtype=torch.int32, device=dev),
                 y=torch.empty(256, dtype=torch.float32, device=dev)) for _ in range(1300)]
    phases = [spax.make_phase(L, packed, b["x"], _params(spax, a), o["tier"], o["f"], o["a"],
                              o["c"], o["y"]) for o in outs]
    with pytest.raises(spax.SpaxError) as e:
        spax.spax_decode_step_projections_noalloc(phases, flags=2)
    assert "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert all(int(o["c"][0]) == -7 for o in outs[:4])
