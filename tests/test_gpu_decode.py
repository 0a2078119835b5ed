"""GPU parity of spax_decode_step_projections: every path the step can take.

flags 0 (fused launches), 1 (mask launch + GEMV launch per phase), 2 (batched: all masks in
one launch, all GEMVs in one launch) wherever the phases are independent.
* fused mask+GEMV launches (d_in <= 16384), fp16 and int4 base formats;
* the two-kernel fallback (d_in > 16384) mixed into the same step;
* a single column chunk (tiny d_in: plain stores instead of atomics);
* consecutive phases writing the same y buffer (the early clearing must not fire);
* TOPK, THRESHOLD and TOPK_GUIDED masks in one step;
* selections concentrated in one wave's channel range per workgroup (the fused kernel's
  waves then stream columns from each other's lists);
* the default step captured into a HIP graph and replayed.
Masks, lists and counts bit-exact against the oracle; y within relative L2 1e-3 and the
per-row fp32 rounding bound (tests/parity_util.py).
"""

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


def _oracle_args(mode_spec, d):
    kind = mode_spec[0]
    if kind == "topk":
        nf, na = otiers.counts_from_fractions(d, mode_spec[1], mode_spec[2])
        return dict(mode=otiers.MODE_TOPK, n_full=nf, n_approx=na)
    if kind == "threshold":
        return dict(mode=otiers.MODE_THRESHOLD, tau_skip=mode_spec[1], tau_full=mode_spec[2])
    s, delta = mode_spec[1], mode_spec[2]
    lo, hi = otiers.guided_bounds(d, s, delta)
    return dict(mode=otiers.MODE_TOPK_GUIDED, tau=-math.log(1 - s), n_lo=lo, n_hi=hi, num=3, den=10)


def _params(spax, oa):
    if oa["mode"] == otiers.MODE_TOPK:
        return spax.topk_params(oa["n_full"], oa["n_approx"])
    if oa["mode"] == otiers.MODE_THRESHOLD:
        return spax.threshold_params(oa["tau_skip"], oa["tau_full"])
    return spax.guided_params(oa["tau"], oa["n_lo"], oa["n_hi"], oa["num"], oa["den"])


def run_step(env, specs, seed, share_y=None, flags=0, xs=None):
    """specs: list of (d_in, d_out list, base_fmt, G, mode_spec).  share_y: set of phase
    indices whose y buffer is the same tensor as the previous phase's (same size).  xs: optional
    {phase: fp16 activations} replacing the synthetic ones."""
    torch, spax, dev = env
    phases, keep = [], []
    share_y = share_y or set()
    prev_y = None
    for i, (d_in, d_out, fmt, G, mspec) in enumerate(specs):
        L = spax.spax_layout_init(d_in, d_out, fmt, 128, G)
        O = opack.Layout(d_in, d_out, fmt, 128, G)
        Ws = [synth.weights(seed + i, d_in, r, m) for m, r in enumerate(d_out)]
        packed = torch.empty(int(L.total_bytes), dtype=torch.uint8, device=dev)
        spax.spax_pack_columns(L, [torch.from_numpy(w).to(dev) for w in Ws], packed)
        x16 = synth.activations(seed, d_in, i, token_scale=synth.token_scale(seed, i))
        if xs and i in xs:
            x16 = np.ascontiguousarray(xs[i], dtype=np.float16)
            assert x16.shape == (d_in,)
        oa = _oracle_args(mspec, d_in)
        if i in share_y:
            y = prev_y
        else:
            y = torch.full((int(L.d_out_total),), float("nan"), dtype=torch.float32, device=dev)
        b = dict(x=torch.from_numpy(x16).to(dev),
                 tier=torch.full((d_in,), 0xAB, dtype=torch.uint8, device=dev),
                 f=torch.full((d_in,), -7, dtype=torch.int32, device=dev),
                 a=torch.full((d_in,), -7, dtype=torch.int32, device=dev),
                 c=torch.full((3,), -7, dtype=torch.int32, device=dev), y=y)
        phases.append(spax.make_phase(L, packed, b["x"], _params(spax, oa), b["tier"], b["f"],
                                      b["a"], b["c"], b["y"]))
        keep.append((L, O, Ws, x16, oa, packed, b))
        prev_y = y
    arr = spax.phase_array(phases)
    ws = torch.zeros(max(1, spax.spax_step_workspace_bytes(arr)), dtype=torch.uint8, device=dev)
    spax.spax_decode_step_projections(arr, ws, flags=flags)
    torch.cuda.synchronize()
    return keep


def check(keep, skip_y=()):
    for i, (L, O, Ws, x16, oa, packed, b) in enumerate(keep):
        args = dict(oa)
        mode = args.pop("mode")
        wt, wf, wa, wc = otiers.build_tiers(x16, mode, **args)
        c = b["c"].cpu().numpy()
        assert list(c) == list(wc), (i, c, wc)
        assert np.array_equal(b["tier"].cpu().numpy(), wt), i
        assert np.array_equal(b["f"].cpu().numpy()[:c[0]], wf), i
        assert np.array_equal(b["a"].cpu().numpy()[:c[1]], wa), i
        if i in skip_y:
            continue
        check_y_oracle(b["y"].cpu().numpy(), O, Ws, x16, wf, wa, f"phase {i}")


@pytest.mark.parametrize("flags", [0, 1, 2])
def test_step_fp16_and_int4(env, flags):
    specs = [(1024, [1024, 512, 512], 0, 128, ("guided", 0.5, 0.01)),
             (1024, [1024], 0, 128, ("guided", 0.3, 0.01)),
             (1024, [2816, 2816], 1, 128, ("topk", 0.25, 0.35)),
             (2816, [1024], 1, 64, ("threshold", 0.5, 1.5)),
             (768, [640], 0, 64, ("topk", 0.2, 0.3))]
    check(run_step(env, specs, 101, flags=flags))


@pytest.mark.parametrize("flags", [0, 1, 2])
def test_step_both_paths_same_outputs(env, flags):
    """The separate mask + GEMV launches and the fused launch give the same masks."""
    specs = [(4096, [1024, 512, 512], 0, 128, ("guided", 0.5, 0.01)),
             (2048, [2048], 1, 128, ("topk", 0.25, 0.35)),
             (3000, [1024], 0, 64, ("threshold", 0.6, 1.4))]
    check(run_step(env, specs, 707, flags=flags))


@pytest.mark.parametrize("flags", [0, 1, 2])
def test_step_wide_input(env, flags):
    """Fused phases whose activation vector needs more LDS than the reduction buffer
    (d_in > 8192): the activations, list slices and reduction area must not overlap."""
    specs = [(11008, [512], 0, 128, ("guided", 0.5, 0.01)),
             (16384, [256], 0, 128, ("topk", 0.3, 0.3)),
             (9000, [1024], 1, 128, ("guided", 0.7, 0.01)),
             (8194, [256], 0, 64, ("threshold", 0.5, 1.5))]
    check(run_step(env, specs, 606, flags=flags))


@pytest.mark.parametrize("flags", [0, 1, 2])
def test_step_fallback_large_din(env, flags):
    specs = [(512, [512], 0, 64, ("guided", 0.5, 0.05)),
             (20000, [256], 0, 128, ("guided", 0.7, 0.01)),     # > 16384: two-kernel path
             (256, [1024, 1024], 0, 128, ("topk", 0.3, 0.3)),
             (17000, [384], 1, 128, ("topk", 0.25, 0.35))]
    check(run_step(env, specs, 202, flags=flags))


@pytest.mark.parametrize("flags", [0, 1, 2])
def test_step_single_chunk_phases(env, flags):
    specs = [(8, [4096], 0, 128, ("topk", 0.5, 0.25)),   # d_in < 32: one chunk, plain stores
             (20, [64], 0, 64, ("topk", 1.0, 0.0)),
             (3000, [512], 0, 64, ("guided", 0.5, 0.01))]
    check(run_step(env, specs, 303, flags=flags))


@pytest.mark.parametrize("flags", [0, 1])
def test_step_shared_y_buffers(env, flags):
    """Phases 1 and 2 write the same y: only the last writer's result must remain."""
    specs = [(512, [1024], 0, 128, ("guided", 0.5, 0.05)),
             (640, [1024], 0, 128, ("topk", 0.3, 0.3)),
             (768, [1024], 0, 128, ("topk", 0.2, 0.3)),
             (512, [512], 0, 64, ("threshold", 0.4, 1.2))]
    keep = run_step(env, specs, 404, share_y={2}, flags=flags)
    check(keep, skip_y={1})


@pytest.mark.parametrize("flags", [0, 1, 2])
def test_step_repeated_calls_stable(env, flags):
    torch, spax, dev = env
    specs = [(2048, [1536, 512], 0, 128, ("guided", 0.5, 0.01)), (1536, [2048], 0, 128, ("topk", 0.3, 0.3))]
    keep = run_step(env, specs, 505, flags=flags)
    first = [b["y"].cpu().numpy().copy() for *_, b in keep]
    # run the same phases again through a fresh step call on the same buffers
    phases = [spax.make_phase(L, packed, b["x"], _params(spax, oa), b["tier"], b["f"], b["a"],
                              b["c"], b["y"]) for (L, O, Ws, x16, oa, packed, b) in keep]
    arr = spax.phase_array(phases)
    ws = torch.zeros(max(1, spax.spax_step_workspace_bytes(arr)), dtype=torch.uint8, device=dev)
    for _ in range(5):
        spax.spax_decode_step_projections(arr, ws, flags=flags)
    torch.cuda.synchronize()
    for f0, (*_, b) in zip(first, keep):
        assert rel_l2(b["y"].cpu().numpy(), f0) <= 1e-6
    check(keep)


def _tie_inputs(seed):
    """Activations whose tier boundaries fall inside runs of equal magnitudes."""
    r = np.random.default_rng(seed)
    x0 = r.laplace(0, 1, 4096).astype(np.float16)
    x0[r.random(4096) < 0.6] = 0                     # zeros: the kept boundary splits them
    x1 = r.choice(np.array([-2, -1, -0.5, -0.25, 0.25, 0.5, 1, 2], np.float16), 4096)
    x2 = r.laplace(0, 1, 3000).astype(np.float16)
    x2[r.random(3000) < 0.3] = 0.5                   # exactly at the thresholds
    x2[r.random(3000) < 0.2] = -1.0
    x3 = np.full(2048, 0.75, np.float16)             # one key for every channel
    x3[::7] = -0.75
    x4 = r.laplace(0, 1, 11008).astype(np.float16)
    x4[r.random(11008) < 0.7] = 0
    x4[r.random(11008) < 0.1] = 1.5
    return {0: x0, 1: x1, 2: x2, 3: x3, 4: x4}


@pytest.mark.parametrize("flags", [0, 1, 2])
def test_step_ties(env, flags):
    """Boundaries that keep some but not all channels of one magnitude: ties go by channel
    order in both launch forms."""
    specs = [(4096, [1024], 0, 128, ("guided", 0.5, 0.01)),
             (4096, [2048], 1, 128, ("topk", 0.3, 0.3)),
             (3000, [512], 0, 64, ("threshold", 0.5, 1.0)),
             (2048, [512], 0, 128, ("topk", 0.2, 0.3)),
             (11008, [768], 0, 128, ("guided", 0.5, 0.01))]
    check(run_step(env, specs, 808, flags=flags, xs=_tie_inputs(808)))


@pytest.mark.parametrize("flags", [0, 4], ids=["fused", "deterministic"])
def test_step_ties_speculative(env, flags):
    """Ties at the boundaries in fp16 phases wide enough (12288 and 4096 rows: tens of channels
    per wave) that the fused kernel loads each wave's largest-key FULL columns before the mask
    is known: speculated columns that the mask then puts in APPROX or SKIP (a tie key past the
    boundary's share, one key for every channel) must be dropped, and confirmed ones must not
    be streamed twice."""
    r = np.random.default_rng(4242)
    x0 = r.laplace(0, 1, 4096).astype(np.float16)
    x0[r.random(4096) < 0.6] = 0
    x1 = r.choice(np.array([-2, -1, -0.5, -0.25, 0.25, 0.5, 1, 2], np.float16), 4096)
    x2 = np.full(4096, 0.75, np.float16)
    x2[::7] = -0.75
    x3 = r.laplace(0, 1, 11008).astype(np.float16)
    x3[r.random(11008) < 0.1] = 1.5
    specs = [(4096, [4096, 4096, 4096], 0, 128, ("guided", 0.5, 0.01)),
             (4096, [4096, 4096, 4096], 0, 128, ("topk", 0.3, 0.3)),
             (4096, [4096, 4096, 4096], 0, 128, ("topk", 0.2, 0.3)),
             (11008, [4096], 0, 128, ("guided", 0.5, 0.01))]
    check(run_step(env, specs, 4242, flags=flags, xs={0: x0, 1: x1, 2: x2, 3: x3}))


@pytest.mark.parametrize("flags", [0, 1, 2])
def test_step_special_values(env, flags):
    """-0, subnormals, infinities and NaN order by their key; masks and lists stay exact
    (y is not compared where x holds infinities or NaN)."""
    r = np.random.default_rng(909)
    x0 = r.laplace(0, 1, 4096).astype(np.float16)
    x0[r.integers(0, 4096, 300)] = np.float16(-0.0)
    x0[r.integers(0, 4096, 300)] = np.float16(6e-8)          # subnormal
    x1 = x0.copy()
    x1[r.integers(0, 4096, 20)] = np.inf
    x1[r.integers(0, 4096, 20)] = -np.inf
    x1[r.integers(0, 4096, 20)] = np.nan
    specs = [(4096, [1024], 0, 128, ("guided", 0.5, 0.01)),
             (4096, [1024], 0, 128, ("topk", 0.25, 0.35)),
             (4096, [512], 1, 128, ("threshold", 0.5, 1.5))]
    keep = run_step(env, specs, 909, flags=flags, xs={0: x0, 1: x1, 2: x1})
    check(keep, skip_y={1, 2})


def test_step_batched_rejects_shared_outputs(env):
    torch, spax, dev = env
    specs = [(512, [1024], 0, 128, ("guided", 0.5, 0.05)), (640, [1024], 0, 128, ("topk", 0.3, 0.3))]
    with pytest.raises(spax.SpaxError) as e:
        run_step(env, specs, 405, share_y={1}, flags=2)
    assert "overlap" in str(e.value)


def _concentrated_x(d, period, width, seed):
    """Large activations only on channels j with j % period < width (one wave's range in each
    column chunk of a 12288-row fused phase); tiny ones elsewhere."""
    rng = np.random.default_rng(seed)
    j = np.arange(d)
    hot = (j % period) < width
    mag = np.where(hot, 4.0 + rng.exponential(1.0, d), 0.01 * rng.exponential(1.0, d))
    sign = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    return (sign * mag).astype(np.float16)


@pytest.mark.parametrize("flags", [0, 1, 2])
def test_step_concentrated_selection(env, flags):
    """Every selected column of a workgroup in one wave's channel range: the fused kernel's
    waves then take most of their columns from another wave's list."""
    d = 4096
    xs = {0: _concentrated_x(d, 410, 26, 11), 1: _concentrated_x(d, 410, 26, 12),
          2: _concentrated_x(d, 410, 26, 13)}
    specs = [(d, [4096, 4096, 4096], 0, 128, ("topk", 200 / d, 60 / d)),
             (d, [4096, 4096, 4096], 1, 128, ("topk", 200 / d, 60 / d)),
             (d, [4096, 4096, 4096], 0, 128, ("threshold", 1.0, 4.5))]
    check(run_step(env, specs, 808, flags=flags, xs=xs))


def test_step_graph_capture_replays(env):
    """The default step (fused launches, plus the clearing launch of the first y) captured into
    a HIP graph through torch and replayed several times, with eager work between the replays:
    every replay gives the eager step's masks, lists and counts bit for bit and its y within
    the atomics' reordering (the graph holds no memset and no host copy)."""
    torch, spax, dev = env
    specs = [(4096, [1024, 512, 512], 0, 128, ("guided", 0.5, 0.01)),
             (2048, [2048], 1, 128, ("topk", 0.25, 0.35)),
             (3000, [1024], 0, 64, ("threshold", 0.6, 1.4))]
    keep = run_step(env, specs, 909, flags=0)
    check(keep)
    want = [dict((k, b[k].clone()) for k in ("tier", "f", "a", "c", "y")) for *_, b in keep]
    phases = [spax.make_phase(L, packed, b["x"], _params(spax, oa), b["tier"], b["f"], b["a"],
                              b["c"], b["y"]) for (L, O, Ws, x16, oa, packed, b) in keep]
    arr = spax.phase_array(phases)
    ws = torch.zeros(max(1, spax.spax_step_workspace_bytes(arr)), dtype=torch.uint8, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        spax.spax_decode_step_projections(arr, ws, flags=0)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        spax.spax_decode_step_projections(arr, ws, flags=0)
    torch.cuda.synchronize()
    for rep in range(3):
        for *_, b in keep:  # clobber every output, eagerly, between replays
            b["tier"].fill_(0xAB)
            b["f"].fill_(-7)
            b["a"].fill_(-7)
            b["c"].fill_(-7)
            b["y"].fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, ((*_, b), w) in enumerate(zip(keep, want)):
            c = w["c"].cpu().numpy()
            assert torch.equal(b["c"], w["c"]), (rep, i)
            assert torch.equal(b["tier"], w["tier"]), (rep, i)
            assert torch.equal(b["f"][:c[0]], w["f"][:c[0]]), (rep, i)
            assert torch.equal(b["a"][:c[1]], w["a"][:c[1]]), (rep, i)
            err = rel_l2(b["y"].cpu().numpy(), w["y"].cpu().numpy())
            assert err <= 1e-6, (rep, i, err)


@pytest.mark.parametrize("flags", [0, 1])
@pytest.mark.parametrize("what", ["x", "f", "a", "tier", "c"])
def test_step_next_y_reuses_previous_phase_buffer(env, flags, what):
    """Stream order lets phase 1 reuse phase 0's buffers: here phase 1's y occupies the memory
    of phase 0's x, one of its lists, its tier bytes or its counts.  Phase 0 must still
    compute everything from intact inputs (its y and the outputs that were not reused match
    the oracle), and phase 1's y must start from zero (no clearing of it may overlap phase
    0's launch)."""
    torch, spax, dev = env
    specs = [(4096, [2048, 1024], 0, 128, ("guided", 0.5, 0.01)),
             (2048, [4096], 0, 128, ("topk", 0.3, 0.3)),
             (1024, [1024], 1, 128, ("guided", 0.3, 0.01))]
    shared = torch.zeros(1 << 16, dtype=torch.uint8, device=dev)  # 64 KiB, 256-byte aligned
    keep, phases = [], []
    for i, (d_in, d_out, fmt, G, mspec) in enumerate(specs):
        L = spax.spax_layout_init(d_in, d_out, fmt, 128, G)
        O = opack.Layout(d_in, d_out, fmt, 128, G)
        Ws = [synth.weights(515 + i, d_in, r, m) for m, r in enumerate(d_out)]
        packed = torch.empty(int(L.total_bytes), dtype=torch.uint8, device=dev)
        spax.spax_pack_columns(L, [torch.from_numpy(w).to(dev) for w in Ws], packed)
        x16 = synth.activations(515, d_in, i)
        oa = _oracle_args(mspec, d_in)
        b = dict(x=torch.from_numpy(x16).to(dev),
                 tier=torch.full((d_in,), 0xAB, dtype=torch.uint8, device=dev),
                 f=torch.full((d_in,), -7, dtype=torch.int32, device=dev),
                 a=torch.full((d_in,), -7, dtype=torch.int32, device=dev),
                 c=torch.full((3,), -7, dtype=torch.int32, device=dev),
                 y=torch.full((int(L.d_out_total),), float("nan"), dtype=torch.float32,
                              device=dev))
        if i == 0:  # phase 0's `what` lives at the start of the shared storage
            view = {"x": torch.float16, "f": torch.int32, "a": torch.int32,
                    "tier": torch.uint8, "c": torch.int32}[what]
            n = b[what].numel() * b[what].element_size()
            v = shared[:n].view(view)
            v.copy_(b[what])
            b[what] = v
        if i == 1:  # phase 1's y over the same bytes (NaN: it must be cleared before use)
            n = b["y"].numel() * 4
            b["y"] = shared[:n].view(torch.float32)
        keep.append((L, O, Ws, x16, oa, packed, b))
    for (L, O, Ws, x16, oa, packed, b) in keep:
        phases.append(spax.make_phase(L, packed, b["x"], _params(spax, oa), b["tier"], b["f"],
                                      b["a"], b["c"], b["y"]))
    torch.cuda.synchronize()
    # phase 1's y holds phase 0's data where the two share bytes and NaN past them: either way
    # it must be cleared before phase 1 accumulates into it
    n0 = keep[0][6][what].numel() * keep[0][6][what].element_size()
    keep[1][6]["y"].view(torch.uint8)[n0:].fill_(0xFF)
    arr = spax.phase_array(phases)
    ws = torch.zeros(max(1, spax.spax_step_workspace_bytes(arr)), dtype=torch.uint8, device=dev)
    spax.spax_decode_step_projections(arr, ws, flags=flags)
    torch.cuda.synchronize()
    for i, (L, O, Ws, x16, oa, packed, b) in enumerate(keep):
        args = dict(oa)
        mode = args.pop("mode")
        wt, wf, wa, wc = otiers.build_tiers(x16, mode, **args)
        if not (i == 0 and what == "c"):
            c = b["c"].cpu().numpy()
            assert list(c) == list(wc), (i, c, wc)
        if not (i == 0 and what == "tier"):
            assert np.array_equal(b["tier"].cpu().numpy(), wt), i
        if not (i == 0 and what == "f"):
            assert np.array_equal(b["f"].cpu().numpy()[:wc[0]], wf), i
        if not (i == 0 and what == "a"):
            assert np.array_equal(b["a"].cpu().numpy()[:wc[1]], wa), i
        check_y_oracle(b["y"].cpu().numpy(), O, Ws, x16, wf, wa, f"phase {i} over {what}")


def test_step_from_several_host_threads(env):
    """Four host threads, each with its own stream and its own copy of every output buffer and
    workspace, enqueue decode steps at once in the default, batched and deterministic forms
    (the batched form stages its descriptor tables through the library's pinned ring, shared
    by all callers on a device): every call gives the single-threaded masks bit for bit and
    the same form's single-threaded y within the atomics' reordering (the deterministic form
    bit for bit)."""
    import threading
    torch, spax, dev = env
    specs = [(4096, [1024, 512, 512], 0, 128, ("guided", 0.5, 0.01)),
             (2048, [2048], 1, 128, ("topk", 0.25, 0.35)),
             (3000, [1024], 0, 64, ("threshold", 0.6, 1.4))]
    keep = run_step(env, specs, 4242, flags=0)
    check(keep)
    want = [dict((k, b[k].cpu().numpy().copy()) for k in ("tier", "f", "a", "c"))
            for *_, b in keep]
    # each form's own single-threaded y (the forms sum in different orders)
    arr0 = spax.phase_array([spax.make_phase(L, packed, b["x"], _params(spax, oa), b["tier"],
                                             b["f"], b["a"], b["c"], b["y"])
                             for (L, O, Ws, x16, oa, packed, b) in keep])
    ws0 = torch.zeros(spax.spax_step_workspace_bytes(arr0), dtype=torch.uint8, device=dev)
    forms = (0, spax.STEP_BATCHED, spax.STEP_DETERMINISTIC)
    want_y = {}
    for flags in forms:
        spax.spax_decode_step_projections(arr0, ws0, flags=flags)
        torch.cuda.synchronize()
        want_y[flags] = [b["y"].cpu().numpy().copy() for *_, b in keep]
        for (L, O, Ws, x16, oa, packed, b), yv in zip(keep, want_y[flags]):
            args = dict(oa)
            mode = args.pop("mode")
            _, wf, wa, _ = otiers.build_tiers(x16, mode, **args)
            check_y_oracle(yv, O, Ws, x16, wf, wa, f"single-threaded flags {flags}")
    errors = []

    def worker(k):
        try:
            s = torch.cuda.Stream(device=dev)
            bufs, phases = [], []
            for (L, O, Ws, x16, oa, packed, b) in keep:
                nb = dict(tier=torch.empty_like(b["tier"]), f=torch.empty_like(b["f"]),
                          a=torch.empty_like(b["a"]), c=torch.empty_like(b["c"]),
                          y=torch.empty_like(b["y"]))
                bufs.append(nb)
                phases.append(spax.make_phase(L, packed, b["x"], _params(spax, oa), nb["tier"],
                                              nb["f"], nb["a"], nb["c"], nb["y"]))
            arr = spax.phase_array(phases)
            ws = torch.zeros(spax.spax_step_workspace_bytes(arr), dtype=torch.uint8, device=dev)
            s.wait_stream(torch.cuda.current_stream(dev))
            for rep in range(6):
                flags = forms[(k + rep) % 3]
                spax.spax_decode_step_projections(arr, ws, flags=flags, stream=s)
                s.synchronize()
                for i, (nb, w) in enumerate(zip(bufs, want)):
                    c = w["c"]
                    if not (np.array_equal(nb["c"].cpu().numpy(), c)
                            and np.array_equal(nb["tier"].cpu().numpy(), w["tier"])
                            and np.array_equal(nb["f"].cpu().numpy()[:c[0]], w["f"][:c[0]])
                            and np.array_equal(nb["a"].cpu().numpy()[:c[1]], w["a"][:c[1]])):
                        errors.append((k, rep, flags, i, "mask"))
                    y = nb["y"].cpu().numpy()
                    ref = want_y[flags][i]
                    if flags == spax.STEP_DETERMINISTIC:
                        ok = np.array_equal(y.view(np.uint32), ref.view(np.uint32))
                    else:
                        ok = np.all(np.isfinite(y)) and rel_l2(y, ref) <= 1e-6
                    if not ok:
                        errors.append((k, rep, flags, i, "y", float(rel_l2(y, ref))))
        except Exception as e:  # reported below
            errors.append((k, repr(e)))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a host thread did not finish"
    assert not errors, errors
