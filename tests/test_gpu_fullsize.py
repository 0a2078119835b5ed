"""GPU parity at the full sizes the benchmark runs: one layer of the 7B-shaped decoder (q|k|v
4096 -> 3 x 4096, o 4096 -> 4096, gate|up 4096 -> 2 x 11008, down 11008 -> 4096) through
spax_decode_step_projections in the launch forms the benchmark times (fused layer-serial and
batched), fp16 and int4 bases, TopK-Guided masks; and the pinned-host path at the
Llama-3-8B down projection (14336 -> 4096) in both transfer modes.

Masks, lists and counts are compared with the oracle bit for bit over every channel.  The
oracle GEMV over whole matrices of this size is slow, so y is checked on sampled rows: whole
quantisation groups of rows (the first, a middle and the last group of every matrix), for
which the oracle runs on the sub-matrix of those rows; a group quantises its rows on its own,
so the sub-matrix packs exactly as the rows of the full one do.  Bound: rel-L2 <= 1e-3.
"""

import math

import numpy as np
import pytest

import synth
from oracle import gemv as ogemv
from oracle import pack as opack
from oracle import tiers as otiers

pytestmark = pytest.mark.gpu
REL_L2 = 1e-3
SEED = 424242
GROUP = 128


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import activation_sparse_tiered_amd as spax
    return torch, spax, torch.device("cuda:0")


def rel_l2(got, ref):
    ref = np.asarray(ref, dtype=np.float64)
    num = np.linalg.norm(np.asarray(got, dtype=np.float64) - ref)
    den = np.linalg.norm(ref)
    return num / den if den > 0 else num


def sampled_groups(d_out):
    n = d_out // GROUP
    return sorted({0, n // 2, n - 1})


@pytest.mark.parametrize("flags", [0, 2])
@pytest.mark.parametrize("fmt", [0, 1])
def test_decode_layer_7b_full_size(env, fmt, flags):
    torch, spax, dev = env
    phases, keep = [], []
    s, delta = 0.5, 0.01
    for k, (name, d_in, d_out) in enumerate(synth.decoder_phases_7b()):
        L = spax.spax_layout_init(d_in, d_out, fmt, GROUP, GROUP)
        Ws = [synth.weights(SEED, d_in, r, k, m) for m, r in enumerate(d_out)]
        packed = torch.empty(int(L.total_bytes), dtype=torch.uint8, device=dev)
        spax.spax_pack_columns(L, [torch.from_numpy(w).to(dev) for w in Ws], packed)
        x16 = synth.activations(SEED, d_in, k)
        lo, hi = spax.spax_guided_bounds(d_in, s, delta)
        params = spax.guided_params(-math.log(1.0 - s), lo, hi, 3, 10)
        b = dict(x=torch.from_numpy(x16).to(dev),
                 tier=torch.full((d_in,), 0xAB, dtype=torch.uint8, device=dev),
                 f=torch.full((d_in,), -7, dtype=torch.int32, device=dev),
                 a=torch.full((d_in,), -7, dtype=torch.int32, device=dev),
                 c=torch.full((3,), -7, dtype=torch.int32, device=dev),
                 y=torch.full((int(L.d_out_total),), float("nan"), dtype=torch.float32,
                              device=dev))
        phases.append(spax.make_phase(L, packed, b["x"], params, b["tier"], b["f"], b["a"],
                                      b["c"], b["y"]))
        keep.append((d_in, d_out, Ws, x16, lo, hi, b, packed))  # the phase holds raw pointers
    arr = spax.phase_array(phases)
    ws = torch.zeros(max(1, spax.spax_step_workspace_bytes(arr)), dtype=torch.uint8, device=dev)
    spax.spax_decode_step_projections(arr, ws, flags=flags)
    torch.cuda.synchronize()

    for k, (d_in, d_out, Ws, x16, lo, hi, b, _) in enumerate(keep):
        wt, wf, wa, wc = otiers.build_tiers(x16, otiers.MODE_TOPK_GUIDED, tau=-math.log(1 - s),
                                            n_lo=lo, n_hi=hi, num=3, den=10)
        c = b["c"].cpu().numpy()
        assert list(c) == list(wc), (k, c, wc)
        assert np.array_equal(b["tier"].cpu().numpy(), wt), k
        assert np.array_equal(b["f"].cpu().numpy()[:c[0]], wf), k
        assert np.array_equal(b["a"].cpu().numpy()[:c[1]], wa), k
        y = b["y"].cpu().numpy()
        off = 0
        for m, r in enumerate(d_out):
            rows = np.concatenate([np.arange(g * GROUP, (g + 1) * GROUP)
                                   for g in sampled_groups(r)])
            sub = [np.ascontiguousarray(Ws[m][:, rows])]
            O = opack.Layout(d_in, [len(rows)], fmt, GROUP, GROUP)
            ref = ogemv.tiered_gemv(O, sub, x16, wf, wa)
            err = rel_l2(y[off + rows], ref)
            assert err <= REL_L2, (k, m, err)
            off += r


@pytest.mark.parametrize("transfer", [0, 1])
def test_pinned_down_projection_8b_full_size(env, transfer):
    """The pinned-host path at the Llama-3-8B down projection (14336 -> 4096): y on sampled
    row groups against the oracle, the byte account against the oracle's range ledger."""
    from oracle import ranges as orng
    torch, spax, dev = env
    d_in, d_out = 14336, [4096]
    L = spax.spax_layout_init(d_in, d_out, 0, GROUP, GROUP)
    O = opack.Layout(d_in, d_out, 0, GROUP, GROUP)
    Ws = [synth.weights(SEED, d_in, d_out[0], 7)]
    packed = torch.empty(int(L.total_bytes), dtype=torch.uint8, device=dev)
    spax.spax_pack_columns(L, [torch.from_numpy(Ws[0]).to(dev)], packed)
    host = torch.empty(int(L.total_bytes), dtype=torch.uint8, pin_memory=True)
    host.copy_(packed)
    del packed
    x16 = synth.activations(SEED, d_in, 7, channel_scaled=True)
    nF, nA = spax.spax_counts_from_fractions(d_in, 0.2, 0.3)
    x = torch.from_numpy(x16).to(dev)
    f = torch.empty(d_in, dtype=torch.int32, device=dev)
    a = torch.empty(d_in, dtype=torch.int32, device=dev)
    c = torch.zeros(3, dtype=torch.int32, device=dev)
    spax.spax_build_tiers(x, d_in, spax.topk_params(nF, nA), None, f, a, c)
    y = torch.full((d_out[0],), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty(spax.spax_pinned_workspace_bytes(L), dtype=torch.uint8, device=dev)
    st = spax.spax_tiered_gemv_pinned(L, host, x, f, a, c, y, 0, ws, transfer=transfer)
    torch.cuda.synchronize()
    _, wf, wa, _ = otiers.build_tiers(x16, otiers.MODE_TOPK, n_full=nF, n_approx=nA)
    rows = np.concatenate([np.arange(g * GROUP, (g + 1) * GROUP) for g in sampled_groups(4096)])
    ref = ogemv.tiered_gemv(opack.Layout(d_in, [len(rows)], 0, GROUP, GROUP),
                            [np.ascontiguousarray(Ws[0][:, rows])], x16, wf, wa)
    assert rel_l2(y.cpu().numpy()[rows], ref) <= REL_L2
    led = orng.ledger(wf, wa, O.stride_F, O.stride_A, 0)
    assert st.selected_bytes == led["selected_bytes"] and st.moved_bytes == led["moved_bytes"]
    assert st.n_ranges == led["n_ranges"]
