"""Blobs with a region of 2 GiB or more, on the GPU.

The GEMV kernels address a column record through one buffer descriptor per blob region with a
32-bit offset while both regions are below 2 GiB, and through a descriptor built per record
on its 64-bit base otherwise.  Every other GPU test runs the first form; this one runs the
second: one fp16 layer with d_in = 4096 and 262144 rows, whose FULL region is exactly 2 GiB,
through the decode step in the fused, two-launch and batched forms and through the pinned-host
path with the device gather (its compacted staging copy has the blob's layout).  TopK 30% FULL
/ 30% APPROX / 40% skipped.  Masks, lists and counts are compared with the oracle bit for bit;
y must be finite everywhere and match the oracle on three whole 128-row groups (the first, one
in the middle, the last), which the oracle computes from those rows of W alone: the two-bit
quantization of a column is per row group, so a group's values do not depend on other rows.
"""

import numpy as np
import pytest

import synth
from oracle import pack as opack
from oracle import tiers as otiers
from tests.parity_util import check_y_oracle

pytestmark = pytest.mark.gpu
SEED = 7070
D_IN, ROWS, GROUP = 4096, 262144, 128
CHECK_ROWS = np.concatenate([np.arange(0, 128), np.arange(ROWS // 2, ROWS // 2 + 128),
                             np.arange(ROWS - 128, ROWS)])


@pytest.fixture(scope="module")
def wide():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import activation_sparse_tiered_amd as spax
    dev = torch.device("cuda:0")
    L = spax.spax_layout_init(D_IN, [ROWS], 0, GROUP, GROUP)
    assert L.off_A >= 1 << 31, L.off_A  # the FULL region is at least 2 GiB
    W = synth.weights_device(SEED, D_IN, ROWS, dev, 1)
    packed = torch.empty(int(L.total_bytes), dtype=torch.uint8, device=dev)
    spax.spax_pack_columns(L, [W], packed)
    W_rows = W[:, torch.from_numpy(CHECK_ROWS).to(dev)].cpu().numpy()
    del W
    torch.cuda.synchronize()
    x16 = synth.activations(SEED, D_IN, 1)
    nF, nA = otiers.counts_from_fractions(D_IN, 0.3, 0.3)
    want = otiers.build_tiers(x16, otiers.MODE_TOPK, n_full=nF, n_approx=nA)
    return dict(torch=torch, spax=spax, dev=dev, L=L, packed=packed, W_rows=W_rows, x16=x16,
                nF=nF, nA=nA, want=want)


def _check(e, y, f, a, c, tier, what):
    wt, wf, wa, wc = e["want"]
    cc = c.cpu().numpy()
    assert list(cc) == list(wc), (what, cc, wc)
    if tier is not None:
        assert np.array_equal(tier.cpu().numpy(), wt), what
    assert np.array_equal(f.cpu().numpy()[:cc[0]], wf), what
    assert np.array_equal(a.cpu().numpy()[:cc[1]], wa), what
    yy = y.cpu().numpy()
    assert np.isfinite(yy).all(), (what, int(np.count_nonzero(~np.isfinite(yy))))
    O = opack.Layout(D_IN, [len(CHECK_ROWS)], 0, GROUP, GROUP)
    err, worst = check_y_oracle(yy[CHECK_ROWS], O, [e["W_rows"]], e["x16"], wf, wa, what)
    print(f"[wide] {what}: rel-L2 {err:.2e}, worst row at {worst:.2e} of its bound", flush=True)


@pytest.mark.parametrize("flags", [0, 1, 2], ids=["fused", "separate", "batched"])
def test_wide_blob_decode_step(wide, flags):
    e = wide
    torch, spax, dev = e["torch"], e["spax"], e["dev"]
    x = torch.from_numpy(e["x16"]).to(dev)
    tier = torch.full((D_IN,), 0xAB, dtype=torch.uint8, device=dev)
    f = torch.full((D_IN,), -7, dtype=torch.int32, device=dev)
    a = torch.full((D_IN,), -7, dtype=torch.int32, device=dev)
    c = torch.full((3,), -7, dtype=torch.int32, device=dev)
    y = torch.full((ROWS,), float("nan"), dtype=torch.float32, device=dev)
    arr = spax.phase_array([spax.make_phase(e["L"], e["packed"], x,
                                            spax.topk_params(e["nF"], e["nA"]), tier, f, a, c, y)])
    ws = torch.zeros(max(1, spax.spax_step_workspace_bytes(arr)), dtype=torch.uint8, device=dev)
    print(f"[wide] decode step flags {flags}", flush=True)
    spax.spax_decode_step_projections(arr, ws, flags=flags)
    torch.cuda.synchronize()
    _check(e, y, f, a, c, tier, f"decode step flags {flags}")


def test_wide_blob_pinned_gather(wide):
    e = wide
    torch, spax, dev = e["torch"], e["spax"], e["dev"]
    L = e["L"]
    host = torch.empty(int(L.total_bytes), dtype=torch.uint8, pin_memory=True)
    host.copy_(e["packed"])
    x = torch.from_numpy(e["x16"]).to(dev)
    f = torch.empty(D_IN, dtype=torch.int32, device=dev)
    a = torch.empty(D_IN, dtype=torch.int32, device=dev)
    c = torch.zeros(3, dtype=torch.int32, device=dev)
    spax.spax_build_tiers(x, D_IN, spax.topk_params(e["nF"], e["nA"]), None, f, a, c)
    y = torch.full((ROWS,), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty(spax.spax_pinned_workspace_bytes(L), dtype=torch.uint8, device=dev)
    print("[wide] pinned gather", flush=True)
    spax.spax_tiered_gemv_pinned(L, host, x, f, a, c, y, 0, ws, transfer=1)
    torch.cuda.synchronize()
    _check(e, y, f, a, c, None, "pinned gather")
