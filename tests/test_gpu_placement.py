"""Co-access placement (eigenradar commentary on SpAx, "The route outside GPU memory", third
paragraph) on the GPU.

Calibration masks of 16 channel-scaled Laplace tokens come from spax_build_tiers;
spax_placement_order turns them into a record order (equal to the oracle's); the blob is
packed in that order with spax_pack_columns_placed (bit for bit the oracle's pack of the
permuted weights); a timed token's activations are permuted alike.  The placed product --
device path, and the pinned-host path with all three transfers -- equals the oracle's
product of the unpermuted weights over the same channels (the masks are built on the placed
vector, so ties between equal magnitudes follow positions; the oracle builds its mask on the
same vector and maps positions back to channels).
"""

import numpy as np
import pytest

import synth
from oracle import pack as opack
from oracle import ranges as orng
from oracle import tiers as otiers
from tests.parity_util import check_y_oracle

pytestmark = pytest.mark.gpu
SEED = 4711


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import activation_sparse_tiered_amd as spax
    return torch, spax, torch.device("cuda:0")


@pytest.mark.parametrize("fmt", [0, 1])
def test_placed_pack_and_product(env, fmt):
    torch, spax, dev = env
    d_in, d_out = 4096, [4096, 1024, 1024]
    L = spax.spax_layout_init(d_in, d_out, fmt, 128, 128)
    O = opack.Layout(d_in, d_out, fmt, 128, 128)
    nF, nA = spax.spax_counts_from_fractions(d_in, 0.2, 0.3)
    params = spax.topk_params(nF, nA)
    # calibration masks on the device
    tier = torch.empty(d_in, dtype=torch.uint8, device=dev)
    f = torch.empty(d_in, dtype=torch.int32, device=dev)
    a = torch.empty(d_in, dtype=torch.int32, device=dev)
    c = torch.zeros(3, dtype=torch.int32, device=dev)
    calib, ocalib = [], []
    for t in range(16):
        xc = synth.activations(SEED, d_in, 1000 + t, channel_scaled=True)
        spax.spax_build_tiers(torch.from_numpy(xc).to(dev), d_in, params, tier, f, a, c)
        calib.append(tier.cpu().numpy().copy())
        ocalib.append(otiers.build_tiers(xc, otiers.MODE_TOPK, n_full=nF, n_approx=nA)[0])
    calib = np.stack(calib)
    assert np.array_equal(calib, np.stack(ocalib))
    order = spax.spax_placement_order(L, calib)
    assert np.array_equal(order, orng.placement_order(calib, O.stride_F, O.stride_A))
    # calibration tokens read fewer ranges from the placed blob
    before = sum(orng.ledger(np.flatnonzero(t == 2), np.flatnonzero(t == 1), 1, 1)["n_ranges"]
                 for t in calib)
    after = sum(orng.ledger(np.flatnonzero(t[order] == 2), np.flatnonzero(t[order] == 1), 1,
                            1)["n_ranges"] for t in calib)
    print(f"[placement] calibration ranges {before} -> {after}", flush=True)
    assert after <= before

    Ws = [synth.weights(SEED, d_in, r, m) for m, r in enumerate(d_out)]
    packed = torch.empty(int(L.total_bytes), dtype=torch.uint8, device=dev)
    perm = torch.from_numpy(order).to(dev)
    spax.spax_pack_columns_placed(L, [torch.from_numpy(w).to(dev) for w in Ws], perm, packed)
    placed_blob = packed.cpu().numpy()
    assert np.array_equal(placed_blob, opack.pack_columns(O, [w[order] for w in Ws]))

    x16 = synth.activations(SEED, d_in, 7, channel_scaled=True)
    xp16 = np.ascontiguousarray(x16[order])
    xp = torch.from_numpy(xp16).to(dev)
    spax.spax_build_tiers(xp, d_in, params, None, f, a, c)
    _, pf, pa, pc = otiers.build_tiers(xp16, otiers.MODE_TOPK, n_full=nF, n_approx=nA)
    cc = c.cpu().numpy()
    assert list(cc) == list(pc)
    assert np.array_equal(f.cpu().numpy()[:cc[0]], pf)
    assert np.array_equal(a.cpu().numpy()[:cc[1]], pa)
    ch_f, ch_a = np.sort(order[pf]), np.sort(order[pa])   # the channels those positions hold

    y = torch.full((int(L.d_out_total),), float("nan"), dtype=torch.float32, device=dev)
    spax.spax_tiered_gemv(L, packed, xp, f, a, c, y, None, ws_bytes=0)
    torch.cuda.synchronize()
    check_y_oracle(y.cpu().numpy(), O, Ws, x16, ch_f, ch_a, f"placed device fmt {fmt}")

    host = torch.empty(int(L.total_bytes), dtype=torch.uint8, pin_memory=True)
    host.copy_(packed)
    ws = torch.empty(spax.spax_pinned_workspace_bytes(L), dtype=torch.uint8, device=dev)
    led = orng.ledger(pf, pa, O.stride_F, O.stride_A, 0)
    for transfer in (0, 1, 2):
        y.fill_(float("nan"))
        st = spax.spax_tiered_gemv_pinned(L, host, xp, f, a, c, y, 0, ws, transfer=transfer)
        torch.cuda.synchronize()
        check_y_oracle(y.cpu().numpy(), O, Ws, x16, ch_f, ch_a,
                       f"placed pinned fmt {fmt} transfer {transfer}")
        assert st.moved_bytes == led["moved_bytes"] and st.n_ranges == led["n_ranges"]
