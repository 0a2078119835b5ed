"""GPU parity of the pinned-host path (spax_tiered_gemv_pinned): the blob in pinned host
memory, merged record ranges copied over PCIe into a compacted staging area (one copy per
range, a copy kernel reading the mapped blob, or host threads gathering the ranges into one
pinned buffer moved by one copy), then the GEMV.

y against the oracle (rel-L2 <= 1e-3 and the per-row fp32 bound of tests/parity_util.py) and
against spax_tiered_gemv on the device copy of the
same blob; the byte account (selected / moved bytes, number of ranges) against
oracle/ranges.py exactly.
"""

import math

import numpy as np
import pytest

import synth
from oracle import pack as opack
from oracle import ranges as orng
from oracle import tiers as otiers
from tests.parity_util import check_y, check_y_oracle, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import activation_sparse_tiered_amd as spax
    return torch, spax, torch.device("cuda:0")


def setup(env, d_in, d_out, fmt, G, seed, n_full, n_approx, x16=None):
    torch, spax, dev = env
    L = spax.spax_layout_init(d_in, d_out, fmt, 128, G)
    O = opack.Layout(d_in, d_out, fmt, 128, G)
    Ws = [synth.weights(seed, d_in, r, m) for m, r in enumerate(d_out)]
    packed = torch.empty(int(L.total_bytes), dtype=torch.uint8, device=dev)
    spax.spax_pack_columns(L, [torch.from_numpy(w).to(dev) for w in Ws], packed)
    host = torch.empty(int(L.total_bytes), dtype=torch.uint8, pin_memory=True)
    host.copy_(packed)
    if x16 is None:
        x16 = synth.activations(seed, d_in, 7, channel_scaled=True)
    b = dict(x=torch.from_numpy(x16).to(dev),
             f=torch.full((d_in,), -1, dtype=torch.int32, device=dev),
             a=torch.full((d_in,), -1, dtype=torch.int32, device=dev),
             c=torch.zeros(3, dtype=torch.int32, device=dev))
    spax.spax_build_tiers(b["x"], d_in, spax.topk_params(n_full, n_approx), None, b["f"], b["a"],
                          b["c"])
    torch.cuda.synchronize()
    return L, O, Ws, x16, packed, host, b


def run_pinned(env, L, host, b, gap, transfer=0):
    torch, spax, dev = env
    y = torch.full((int(L.d_out_total),), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty(spax.spax_pinned_workspace_bytes(L), dtype=torch.uint8, device=dev)
    st = spax.spax_tiered_gemv_pinned(L, host, b["x"], b["f"], b["a"], b["c"], y, gap, ws,
                                      transfer=transfer)
    torch.cuda.synchronize()
    return y.cpu().numpy(), st


@pytest.mark.parametrize("transfer", [0, 1, 2])
@pytest.mark.parametrize("fmt,G", [(0, 128), (1, 128), (0, 64)])
@pytest.mark.parametrize("gap", [0, 3])
def test_pinned_matches_oracle_and_device_path(env, fmt, G, gap, transfer):
    torch, spax, dev = env
    d_in, d_out = 2048, [1024, 512, 512]
    nF, nA = spax.spax_counts_from_fractions(d_in, 0.2, 0.3)
    L, O, Ws, x16, packed, host, b = setup(env, d_in, d_out, fmt, G, 31 + fmt, nF, nA)
    y_pin, st = run_pinned(env, L, host, b, gap, transfer)
    # the device path on the same blob
    y_dev = torch.empty(int(L.d_out_total), dtype=torch.float32, device=dev)
    spax.spax_tiered_gemv(L, packed, b["x"], b["f"], b["a"], b["c"], y_dev, None, ws_bytes=0)
    torch.cuda.synchronize()
    _, wf, wa, _ = otiers.build_tiers(x16, otiers.MODE_TOPK, n_full=nF, n_approx=nA)
    check_y_oracle(y_pin, O, Ws, x16, wf, wa, f"transfer {transfer} gap {gap}")
    assert rel_l2(y_pin, y_dev.cpu().numpy()) <= 1e-6
    led = orng.ledger(wf, wa, O.stride_F, O.stride_A, gap)
    led["n_full"], led["n_approx"] = len(wf), len(wa)
    assert st.n_full == len(wf) and st.n_approx == len(wa)
    assert st.selected_bytes == led["selected_bytes"]
    assert st.moved_bytes == led["moved_bytes"]
    assert st.n_ranges == led["n_ranges"]
    assert st.list_bytes == expected_upload(d_in, led, transfer)


def expected_upload(d, led, transfer):
    """Bytes of list data sent host -> device: none for the gather transfer (the ranges are
    merged on the device); for the memcpy and host-gather transfers one upload of the two
    compacted host lists
    (d entries each) up to the last one in use."""
    if transfer == 1:
        return 0
    lf, la = led["n_full"], led["n_approx"]
    return 4 * (d + la if la else lf)


@pytest.mark.parametrize("transfer", [0, 1, 2])
def test_pinned_all_skip_and_all_full(env, transfer):
    torch, spax, dev = env
    d_in, d_out = 1000, [768]
    L, O, Ws, x16, packed, host, b = setup(env, d_in, d_out, 0, 128, 5, 0, 0)
    y, st = run_pinned(env, L, host, b, 0, transfer)
    assert np.all(y == 0) and st.n_ranges == 0 and st.moved_bytes == 0
    L, O, Ws, x16, packed, host, b = setup(env, d_in, d_out, 0, 128, 6, d_in, 0)
    y, st = run_pinned(env, L, host, b, 0, transfer)
    dense = Ws[0].astype(np.float64).T @ x16.astype(np.float64)
    check_y_oracle(y, O, Ws, x16, np.arange(d_in), [], "all FULL")
    assert rel_l2(y, dense) <= 1e-5
    assert st.n_ranges == 1 and st.moved_bytes == d_in * O.stride_F   # one range: every column


@pytest.mark.parametrize("transfer", [0, 1, 2])
def test_pinned_repeated_calls_and_wide_gap(env, transfer):
    torch, spax, dev = env
    d_in, d_out = 4096, [1024]
    nF, nA = spax.spax_counts_from_fractions(d_in, 0.2, 0.3)
    L, O, Ws, x16, packed, host, b = setup(env, d_in, d_out, 0, 128, 9, nF, nA)
    y0, st0 = run_pinned(env, L, host, b, 0, transfer)
    for _ in range(3):
        y1, st1 = run_pinned(env, L, host, b, 0, transfer)
        assert rel_l2(y1, y0) <= 1e-6 and st1.moved_bytes == st0.moved_bytes
    y2, st2 = run_pinned(env, L, host, b, d_in, transfer)   # everything merged
    assert rel_l2(y2, y0) <= 1e-6
    assert st2.n_ranges <= 2 and st2.moved_bytes >= st0.moved_bytes


def test_pinned_rejects_device_blob(env):
    torch, spax, dev = env
    L, O, Ws, x16, packed, host, b = setup(env, 256, [256], 0, 128, 11, 32, 32)
    ws = torch.empty(spax.spax_pinned_workspace_bytes(L), dtype=torch.uint8, device=dev)
    y = torch.empty(int(L.d_out_total), dtype=torch.float32, device=dev)
    with pytest.raises(spax.SpaxError) as e:
        spax.spax_tiered_gemv_pinned(L, packed, b["x"], b["f"], b["a"], b["c"], y, 0, ws)
    assert "pinned" in str(e.value)


def test_pinned_gather_without_account_and_in_a_graph(env):
    """The gather transfer merges the ranges on the device, so a call without the byte account
    waits for nothing and can be captured into a HIP graph: y from replays (outputs clobbered
    in between) equals y from the eager call with the account."""
    torch, spax, dev = env
    d_in, d_out = 3000, [1024, 512]
    nF, nA = spax.spax_counts_from_fractions(d_in, 0.2, 0.3)
    L, O, Ws, x16, packed, host, b = setup(env, d_in, d_out, 0, 64, 21, nF, nA)
    y_ref, st = run_pinned(env, L, host, b, 2, transfer=1)
    assert st.n_full == nF and st.n_approx == nA and st.list_bytes == 0
    ws = torch.empty(spax.spax_pinned_workspace_bytes(L), dtype=torch.uint8, device=dev)
    y = torch.full((int(L.d_out_total),), float("nan"), dtype=torch.float32, device=dev)
    assert spax.spax_tiered_gemv_pinned(L, host, b["x"], b["f"], b["a"], b["c"], y, 2, ws,
                                        transfer=1, stats=False) is None
    torch.cuda.synchronize()
    assert rel_l2(y.cpu().numpy(), y_ref) <= 1e-6
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream
        spax.spax_tiered_gemv_pinned(L, host, b["x"], b["f"], b["a"], b["c"], y, 2, ws,
                                     transfer=1, stats=False)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        spax.spax_tiered_gemv_pinned(L, host, b["x"], b["f"], b["a"], b["c"], y, 2, ws,
                                     transfer=1, stats=False)
    for _ in range(3):
        y.fill_(float("nan"))
        ws.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert rel_l2(y.cpu().numpy(), y_ref) <= 1e-6


def test_pinned_gather_malformed_lists_stay_inside(env):
    """Lists that are not ascending and hold out-of-range channels (the device merge cannot
    return an error): the call completes, every access stays inside the blob and the
    workspace (indices and slots are clamped on the device), and y is finite."""
    torch, spax, dev = env
    d_in, d_out = 1000, [512]
    L, O, Ws, x16, packed, host, b = setup(env, d_in, d_out, 0, 128, 23, 40, 60)
    rng = np.random.default_rng(5)
    bad_f = rng.integers(-50, d_in + 50, size=d_in).astype(np.int32)   # unordered, out of range
    bad_a = np.concatenate([np.arange(d_in - 1, -1, -1)]).astype(np.int32)  # descending
    b["f"].copy_(torch.from_numpy(bad_f))
    b["a"].copy_(torch.from_numpy(bad_a))
    b["c"].copy_(torch.tensor([700, 900, 0], dtype=torch.int32))
    for gap in (0, 5, d_in):
        y, st = run_pinned(env, L, host, b, gap, transfer=1)
        assert np.isfinite(y).all()
        assert 0 <= st.moved_bytes <= d_in * (L.stride_F + L.stride_A)


def test_pinned_calls_from_several_host_threads(env):
    """Four host threads, each with its own stream, workspace and output, call the pinned path
    at once on one shared blob in all three transfers (the host-merged transfers share the
    library's per-device pinned scratch and the host-gather thread pool): every call gives the
    single-threaded result, and the byte accounts agree."""
    import threading
    torch, spax, dev = env
    d_in, d_out = 4096, [2048, 1024]
    nF, nA = spax.spax_counts_from_fractions(d_in, 0.2, 0.3)
    L, O, Ws, x16, packed, host, b = setup(env, d_in, d_out, 0, 128, 77, nF, nA)
    want = {t: run_pinned(env, L, host, b, 2, t) for t in (0, 1, 2)}
    _, wf, wa, _ = otiers.build_tiers(x16, otiers.MODE_TOPK, n_full=nF, n_approx=nA)
    for t, (y, _) in want.items():
        check_y_oracle(y, O, Ws, x16, wf, wa, f"single-threaded transfer {t}")
    errors = []

    def worker(k):
        try:
            s = torch.cuda.Stream(device=dev)
            y = torch.empty(int(L.d_out_total), dtype=torch.float32, device=dev)
            ws = torch.empty(spax.spax_pinned_workspace_bytes(L), dtype=torch.uint8, device=dev)
            for rep in range(6):
                t = (k + rep) % 3
                y.fill_(float("nan"))
                s.wait_stream(torch.cuda.current_stream(dev))
                st = spax.spax_tiered_gemv_pinned(L, host, b["x"], b["f"], b["a"], b["c"], y, 2,
                                                  ws, transfer=t, stream=s)
                s.synchronize()
                got = y.cpu().numpy()
                if rel_l2(got, want[t][0]) > 1e-6 or not np.all(np.isfinite(got)):
                    errors.append((k, rep, t, "y"))
                if st.moved_bytes != want[t][1].moved_bytes or st.n_ranges != want[t][1].n_ranges:
                    errors.append((k, rep, t, "account"))
        except Exception as e:  # reported below
            errors.append((k, repr(e)))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a host thread did not finish"
    assert not errors, errors
