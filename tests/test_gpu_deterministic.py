"""Deterministic reduction of the decode step (SPAX_STEP_DETERMINISTIC) on the GPU.

A 7B-shaped decoder layer (q|k|v, o, gate|up, down) plus one projection wider than the fused
kernel takes (24576 -> 4096, so the stand-alone mask + GEMV launches run it) goes through
spax_decode_step_projections eight times with the flag, in the default and in the
SPAX_STEP_SEPARATE form.  y must be identical bit for bit from run to run (it is set to NaN
before every run, so every row must also be written), the masks equal the oracle's bit for
bit, and y meets the oracle's product at relative L2 1e-3 and the per-row fp32 rounding bound.
The same step without the flag (fp32 atomics) is checked against the same bound.
"""

import numpy as np
import pytest

import synth
from oracle import pack as opack
from oracle import tiers as otiers
from tests.parity_util import check_y_oracle
from tests.test_gpu_fullsize import _params, _tier_args

pytestmark = pytest.mark.gpu
SEED = 90210
GROUP = 128
RUNS = 8


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import activation_sparse_tiered_amd as spax
    return torch, spax, torch.device("cuda:0")


def _shapes():
    return synth.decoder_phases_7b() + [("wide", 24576, [4096])]


@pytest.mark.parametrize("fmt,rule", [(0, ("guided", 0.5, 0.01)), (1, ("topk", 0.25, 0.35))],
                         ids=["fp16-guided", "int4-topk"])
def test_deterministic_step_is_bit_stable(env, fmt, rule):
    torch, spax, dev = env
    phases, keep = [], []
    for k, (name, d_in, d_out) in enumerate(_shapes()):
        L = spax.spax_layout_init(d_in, d_out, fmt, GROUP, GROUP)
        Ws = [synth.weights(SEED, d_in, r, k, m) for m, r in enumerate(d_out)]
        packed = torch.empty(int(L.total_bytes), dtype=torch.uint8, device=dev)
        spax.spax_pack_columns(L, [torch.from_numpy(w).to(dev) for w in Ws], packed)
        x16 = synth.activations(SEED, d_in, k)
        ta = _tier_args(rule, d_in)
        b = dict(x=torch.from_numpy(x16).to(dev),
                 tier=torch.empty(d_in, dtype=torch.uint8, device=dev),
                 f=torch.empty(d_in, dtype=torch.int32, device=dev),
                 a=torch.empty(d_in, dtype=torch.int32, device=dev),
                 c=torch.empty(3, dtype=torch.int32, device=dev),
                 y=torch.empty(int(L.d_out_total), dtype=torch.float32, device=dev))
        phases.append(spax.make_phase(L, packed, b["x"], _params(spax, ta), b["tier"], b["f"],
                                      b["a"], b["c"], b["y"]))
        keep.append((name, d_in, d_out, Ws, x16, ta, b, packed))
    arr = spax.phase_array(phases)
    ws = torch.zeros(spax.spax_step_workspace_bytes(arr), dtype=torch.uint8, device=dev)

    def run(flags):
        for *_, b, _p in keep:
            b["y"].fill_(float("nan"))
        spax.spax_decode_step_projections(arr, ws, flags=flags)
        torch.cuda.synchronize()
        return [b["y"].cpu().numpy().copy() for *_, b, _p in keep]

    refs = {}
    for name, d_in, d_out, Ws, x16, ta, b, _ in keep:
        args = dict(ta)
        mode = args.pop("mode")
        refs[name] = otiers.build_tiers(x16, mode, **args)
    for flags in (spax.STEP_DETERMINISTIC, spax.STEP_DETERMINISTIC | spax.STEP_SEPARATE):
        print(f"[deterministic] fmt {fmt} flags {flags}: {RUNS} runs", flush=True)
        first = run(flags)
        for r in range(1, RUNS):
            again = run(flags)
            for (name, *_), y0, y1 in zip(keep, first, again):
                assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32)), \
                    f"{name}: run {r} differs from run 0 (flags {flags})"
        for (name, d_in, d_out, Ws, x16, ta, b, _), y0 in zip(keep, first):
            wt, wf, wa, wc = refs[name]
            assert list(b["c"].cpu().numpy()) == list(wc), name
            assert np.array_equal(b["tier"].cpu().numpy(), wt), name
            O = opack.Layout(d_in, d_out, fmt, GROUP, GROUP)
            err, worst = check_y_oracle(y0, O, Ws, x16, wf, wa, f"fmt {fmt} flags {flags} {name}")
            print(f"[deterministic] fmt {fmt} flags {flags} {name}: rel-L2 {err:.2e}, worst row "
                  f"at {worst:.2e} of its bound", flush=True)
    # the atomic form: same bound; whether its runs differ is only reported
    ya, yb = run(0), run(0)
    same = all(np.array_equal(u.view(np.uint32), v.view(np.uint32)) for u, v in zip(ya, yb))
    print(f"[deterministic] fmt {fmt} atomics: two runs identical: {same}", flush=True)
    for (name, d_in, d_out, Ws, x16, ta, b, _), y0 in zip(keep, ya):
        _, wf, wa, _ = refs[name]
        O = opack.Layout(d_in, d_out, fmt, GROUP, GROUP)
        check_y_oracle(y0, O, Ws, x16, wf, wa, f"fmt {fmt} atomics {name}")
