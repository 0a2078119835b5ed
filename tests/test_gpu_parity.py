"""GPU parity: the HIP path (through the C ABI) against the oracle on the same seeded inputs.

Bar: packed blob, tier bytes, index lists and counts bit-exact; y within relative L2 error
1e-3 of the float64 oracle (fp32 accumulation) and within the per-row fp32 rounding bound of
tests/parity_util.py, and exactly zero when nothing is selected.
"""

import math
import zlib

import numpy as np
import pytest

import synth
from oracle import gemv as ogemv
from oracle import pack as opack
from oracle import tiers as otiers
from tests.parity_util import check_y, check_y_oracle, rel_l2, row_bound

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def spax():
    import activation_sparse_tiered_amd as m
    return m


def _t(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _np(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _empty(n, dtype, dev):
    import torch
    return torch.empty(max(1, n), dtype=dtype, device=dev)


def _fill_garbage(t):
    import torch
    if t.dtype.is_floating_point:
        t.fill_(float("nan"))
    else:
        t.fill_(-7 if t.dtype != torch.uint8 else 0xAB)
    return t


# ------------------------------------------------------------------ pack

PACK_CASES = [
    # (d_in, d_out list, base_fmt, approx_group)
    (1, [64], 0, 64), (3, [128], 0, 64), (17, [512], 0, 64), (5, [128, 64, 192], 0, 64),
    (9, [128], 0, 128), (33, [4096], 0, 128), (7, [1024, 256, 256], 0, 128),
    (2, [128], 1, 128), (11, [384, 128], 1, 128), (6, [512], 1, 64), (13, [4096, 4096], 1, 128),
]


@pytest.mark.parametrize("case", PACK_CASES)
def test_pack_bit_exact(dev, spax, case):
    d_in, d_out, fmt, G = case
    seed = zlib.crc32(repr(case).encode()) % 1000
    L = spax.spax_layout_init(d_in, d_out, fmt, 128, G)
    O = opack.Layout(d_in, d_out, fmt, 128, G)
    Ws = [synth.weights(seed, d_in, r, m) for m, r in enumerate(d_out)]
    # edge values: a constant group, a group with -0 and +0, subnormals, large magnitudes
    Ws[0][0, :G] = np.float16(0.5)
    if d_in > 1:
        Ws[0][1, :G] = np.float16(0.0)
        Ws[0][1, 3] = np.float16(-0.0)
    if d_in > 2:
        Ws[0][2, :8] = np.array([6e-8, -6e-8, 1e-7, 0, 3e-5, -2e-5, 1e-6, 0], dtype=np.float16)
    if d_in > 3:
        Ws[0][3, :4] = np.array([65504, -65504, 1000, -3], dtype=np.float16)
    dW = [_t(w, dev) for w in Ws]
    packed = _fill_garbage(_empty(L.total_bytes, __import__("torch").uint8, dev))
    spax.spax_pack_columns(L, dW, packed)
    got = _np(packed)[:L.total_bytes]
    want = opack.pack_columns(O, Ws)
    if not np.array_equal(got, want):
        bad = np.flatnonzero(got != want)
        pytest.fail(f"{bad.size} bytes differ, first at {bad[:8]} got {got[bad[:8]]} want {want[bad[:8]]}")


def test_pack_golden_on_gpu(dev, spax, golden):
    import torch
    g = golden("pack_tiny.json")
    for c in g["cases"]:
        fmt = 0 if c["base_fmt"] == "fp16" else 1
        L = spax.spax_layout_init(c["d_in"], c["d_out"], fmt, c["base_group"], c["approx_group"])
        T = int(L.d_out_total)
        cols = []
        for p in c["columns"]:
            vals = [float(v) for v in p]
            cols.append([vals[r % len(vals)] for r in range(T)])
        W = np.array(cols, dtype=np.float64).astype(np.float16)
        packed = _fill_garbage(_empty(L.total_bytes, torch.uint8, dev))
        spax.spax_pack_columns(L, [_t(W, dev)], packed)
        blob = _np(packed)
        for region, stride, base in (("F", L.stride_F, 0), ("A", L.stride_A, L.off_A)):
            for j, parts in enumerate(c[region]):
                want = b"".join(bytes.fromhex(h) * n for h, n in parts)
                want = want + bytes(stride - len(want))
                assert bytes(blob[base + j * stride: base + (j + 1) * stride]) == want, (c["name"], region, j)


# ------------------------------------------------------------------ tiers

def _run_tiers(spax, dev, x16, params):
    import torch
    d = x16.size
    x = _t(x16, dev)
    tier = _fill_garbage(_empty(d, torch.uint8, dev))
    f = _fill_garbage(_empty(d, torch.int32, dev))
    a = _fill_garbage(_empty(d, torch.int32, dev))
    cnt = _fill_garbage(_empty(3, torch.int32, dev))
    spax.spax_build_tiers(x, d, params, tier, f, a, cnt)
    cnt = _np(cnt)
    return _np(tier)[:d], _np(f)[:cnt[0]], _np(a)[:cnt[1]], cnt


def _compare_tiers(got, want):
    tier, f, a, cnt = got
    wt, wf, wa, wc = want
    assert list(cnt) == list(wc)
    assert np.array_equal(tier, wt)
    assert np.array_equal(f, wf) and np.array_equal(a, wa)


def _x_cases():
    out = []
    for d in [1, 2, 3, 63, 64, 65, 127, 1000, 1024, 4096, 11008, 14336, 32768]:
        out.append((d, "laplace"))
    for d in [5, 100, 777, 5000]:
        out.append((d, "ties"))
        out.append((d, "special"))
    return out


def _make_x(d, kind, seed):
    x = synth.activations(seed, d, 7)
    if kind == "ties":
        x = np.round(x.astype(np.float64) * 2).astype(np.float16)
    elif kind == "special":
        r = np.random.default_rng(seed)
        pick = r.integers(0, d, max(1, d // 10))
        x[pick] = r.choice(np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 65504, 6e-8],
                                    dtype=np.float16), pick.size)
    return x


@pytest.mark.parametrize("d,kind", _x_cases())
def test_tiers_topk(dev, spax, d, kind):
    x = _make_x(d, kind, d * 3 + 1)
    for pf, pa in [(0.2, 0.3), (0.3, 0.3), (0.0, 0.0), (1.0, 0.0), (0.0, 1.0), (0.25, 0.35),
                   (0.5, 0.5)]:
        nf, na = otiers.counts_from_fractions(d, pf, pa)
        got = _run_tiers(spax, dev, x, spax.topk_params(nf, na))
        _compare_tiers(got, otiers.build_tiers(x, otiers.MODE_TOPK, n_full=nf, n_approx=na))


@pytest.mark.parametrize("d,kind", _x_cases())
def test_tiers_threshold(dev, spax, d, kind):
    x = _make_x(d, kind, d * 5 + 2)
    for ts, tf in [(0.5, 1.5), (0.0, 0.0), (0.7, 0.7), (1e-9, 1e9), (math.inf, math.inf),
                   (0.356675, 1.203973)]:
        got = _run_tiers(spax, dev, x, spax.threshold_params(ts, tf))
        _compare_tiers(got, otiers.build_tiers(x, otiers.MODE_THRESHOLD, tau_skip=ts, tau_full=tf))


@pytest.mark.parametrize("d,kind", _x_cases())
def test_tiers_guided(dev, spax, d, kind):
    for t in range(4):
        scale = synth.token_scale(d, t)
        x = synth.activations(d * 7 + t, d, 9, token_scale=scale) if kind == "laplace" else _make_x(d, kind, t)
        for s in (0.3, 0.5, 0.7):
            tau = -math.log(1 - s)
            for delta in (0.01, 0.1):
                lo, hi = otiers.guided_bounds(d, s, delta)
                if lo > hi:
                    continue
                got = _run_tiers(spax, dev, x, spax.guided_params(tau, lo, hi, 3, 10))
                want = otiers.build_tiers(x, otiers.MODE_TOPK_GUIDED, tau=tau, n_lo=lo, n_hi=hi,
                                          num=3, den=10)
                _compare_tiers(got, want)
                assert lo <= got[3][2] <= hi


def test_tiers_golden_on_gpu(dev, spax, golden):
    g = golden("tiers_tiny.json")
    vecs = {k: np.array([float(v) for v in vals]).astype(np.float16) for k, vals in g["vectors"].items()}
    for c in g["cases"]:
        x = vecs[c["x"]]
        if c["mode"] == "topk":
            p = spax.topk_params(c["n_full"], c["n_approx"])
        elif c["mode"] == "threshold":
            p = spax.threshold_params(c["tau_skip"], c["tau_full"])
        else:
            p = spax.guided_params(c["tau"], c["n_lo"], c["n_hi"], c["num"], c["den"])
        tier, f, a, cnt = _run_tiers(spax, dev, x, p)
        assert list(tier) == c["tier"] and list(f) == c["full"] and list(a) == c["approx"]
        assert list(cnt) == c["counts"]


# ------------------------------------------------------------------ GEMV

GEMV_CASES = [
    # (d_in, d_out list, base_fmt, G, p_full, p_approx)
    (1, [64], 0, 64, 1.0, 0.0), (5, [64], 0, 64, 0.2, 0.4), (31, [576], 0, 64, 0.3, 0.3),
    (512, [512], 0, 64, 0.2, 0.3), (200, [1088], 0, 64, 0.5, 0.5), (700, [4096], 0, 128, 0.3, 0.3),
    (300, [1024, 256, 256], 0, 128, 0.25, 0.35), (1000, [2048, 2048], 0, 128, 0.3, 0.3),
    (257, [4096], 0, 128, 0.0, 1.0), (257, [4096], 0, 128, 1.0, 0.0),
    (64, [128], 1, 128, 0.3, 0.3), (333, [1152], 1, 128, 0.25, 0.35), (900, [4096, 512], 1, 64, 0.3, 0.3),
    (100, [640], 1, 128, 1.0, 0.0),
    # int4 layouts use 2048-row tiles (32 rows per lane): several tiles and a ragged last one
    (1500, [4096, 2048, 2048, 1152], 1, 128, 0.2, 0.3), (257, [2048], 1, 64, 0.0, 1.0),
    (4000, [6144], 1, 128, 0.25, 0.35), (3, [128], 1, 64, 0.5, 0.5),
]


def _setup_phase(spax, dev, d_in, d_out, fmt, G, seed):
    import torch
    L = spax.spax_layout_init(d_in, d_out, fmt, 128, G)
    O = opack.Layout(d_in, d_out, fmt, 128, G)
    Ws = [synth.weights(seed, d_in, r, m) for m, r in enumerate(d_out)]
    packed = _empty(L.total_bytes, torch.uint8, dev)
    spax.spax_pack_columns(L, [_t(w, dev) for w in Ws], packed)
    ws = torch.zeros(spax.spax_gemv_workspace_bytes(L), dtype=torch.uint8, device=dev)
    return L, O, Ws, packed, ws


@pytest.mark.parametrize("case", GEMV_CASES)
def test_gemv_parity(dev, spax, case):
    import torch
    d_in, d_out, fmt, G, pf, pa = case
    seed = zlib.crc32(repr(case).encode()) % 10000
    L, O, Ws, packed, ws = _setup_phase(spax, dev, d_in, d_out, fmt, G, seed)
    x16 = synth.activations(seed, d_in, 1)
    nf, na = otiers.counts_from_fractions(d_in, pf, pa)
    _, f, a, cnt = otiers.build_tiers(x16, otiers.MODE_TOPK, n_full=nf, n_approx=na)
    y = _fill_garbage(_empty(int(L.d_out_total), torch.float32, dev))
    dx = _t(x16, dev)
    df, da, dc = (_t(np.concatenate([f, [0]]).astype(np.int32), dev),
                  _t(np.concatenate([a, [0]]).astype(np.int32), dev), _t(cnt, dev))
    spax.spax_tiered_gemv(L, packed, dx, df, da, dc, y, ws)
    got = _np(y)
    err, _ = check_y_oracle(got, O, Ws, x16, f, a, repr(case))
    # expected fp32 accuracy is far tighter than the bar; a wrong row or column would not be
    assert err <= 1e-5, err


@pytest.mark.parametrize("case", GEMV_CASES[:6])
def test_gemv_empty_selection_is_exact_zero(dev, spax, case):
    import torch
    d_in, d_out, fmt, G, _, _ = case
    L, O, Ws, packed, ws = _setup_phase(spax, dev, d_in, d_out, fmt, G, 3)
    x16 = synth.activations(3, d_in, 1)
    y = _fill_garbage(_empty(int(L.d_out_total), torch.float32, dev))
    z = _t(np.zeros(4, np.int32), dev)
    cnt = _t(np.array([0, 0, d_in], np.int32), dev)
    spax.spax_tiered_gemv(L, packed, _t(x16, dev), z, z, cnt, y, ws)
    got = _np(y)
    assert np.array_equal(got, np.zeros_like(got)) and not np.signbit(got).any()


def test_gemv_repeatable(dev, spax):
    """Ten calls agree to fp32 rounding (chunks meet through atomics in any order) and each
    meets the bar; y is overwritten every call, whatever it held."""
    import torch
    L, O, Ws, packed, ws = _setup_phase(spax, dev, 3000, [4096, 4096], 0, 128, 5)
    x16 = synth.activations(5, 3000, 2)
    nf, na = otiers.counts_from_fractions(3000, 0.3, 0.3)
    _, f, a, cnt = otiers.build_tiers(x16, otiers.MODE_TOPK, n_full=nf, n_approx=na)
    ref = ogemv.tiered_gemv(O, Ws, x16, f, a)
    bound = row_bound(O, Ws, x16, f, a)
    args = [_t(x16, dev), _t(f, dev), _t(a, dev), _t(cnt, dev)]
    outs = []
    y = _fill_garbage(_empty(int(L.d_out_total), torch.float32, dev))
    for _ in range(10):
        spax.spax_tiered_gemv(L, packed, *args, y, ws)
        outs.append(_np(y).copy())
    for o in outs:
        check_y(o, ref, bound)
        assert rel_l2(o, outs[0]) <= 1e-6


# ------------------------------------------------------------------ mask -> GEMV chain

@pytest.mark.parametrize("fmt", [0, 1])
def test_tiers_then_gemv(dev, spax, fmt):
    import torch
    d_in, d_out = 1536, [1024, 512]
    L, O, Ws, packed, ws = _setup_phase(spax, dev, d_in, d_out, fmt, 128, 77 + fmt)
    for t in range(5):
        x16 = synth.activations(77, d_in, t)
        lo, hi = otiers.guided_bounds(d_in, 0.5, 0.01)
        p = spax.guided_params(-math.log(0.5), lo, hi, 3, 10)
        dx = _t(x16, dev)
        tier = _empty(d_in, torch.uint8, dev)
        f = _empty(d_in, torch.int32, dev)
        a = _empty(d_in, torch.int32, dev)
        cnt = _empty(3, torch.int32, dev)
        y = _fill_garbage(_empty(int(L.d_out_total), torch.float32, dev))
        spax.spax_build_tiers(dx, d_in, p, tier, f, a, cnt)
        spax.spax_tiered_gemv(L, packed, dx, f, a, cnt, y, ws)
        wt, wf, wa, wc = otiers.build_tiers(x16, otiers.MODE_TOPK_GUIDED, tau=-math.log(0.5),
                                            n_lo=lo, n_hi=hi, num=3, den=10)
        c = _np(cnt)
        assert list(c) == list(wc)
        assert np.array_equal(_np(f)[:c[0]], wf) and np.array_equal(_np(a)[:c[1]], wa)
        check_y_oracle(_np(y), O, Ws, x16, wf, wa, f"fmt {fmt} token {t}")


def test_decode_step_small(dev, spax):
    """A short stack of phases through spax_decode_step_projections."""
    import torch
    shapes = [("qkv", 256, [256, 128, 128]), ("o", 256, [256]), ("gateup", 256, [640, 640]),
              ("down", 640, [256])]
    layers = 3
    phases, keep, refs = [], [], []
    for l in range(layers):
        for k, (name, d_in, d_out) in enumerate(shapes):
            L, O, Ws, packed, _ = _setup_phase(spax, dev, d_in, d_out, 0, 128, 1000 + 10 * l + k)
            x16 = synth.activations(1000, d_in, l, k)
            lo, hi = otiers.guided_bounds(d_in, 0.5, 0.02)
            p = spax.guided_params(-math.log(0.5), lo, hi, 3, 10)
            bufs = dict(x=_t(x16, dev), tier=_empty(d_in, torch.uint8, dev),
                        f=_empty(d_in, torch.int32, dev), a=_empty(d_in, torch.int32, dev),
                        c=_empty(3, torch.int32, dev),
                        y=_fill_garbage(_empty(int(L.d_out_total), torch.float32, dev)))
            phases.append(spax.make_phase(L, packed, bufs["x"], p, bufs["tier"], bufs["f"],
                                          bufs["a"], bufs["c"], bufs["y"]))
            keep.append((L, packed, bufs))
            refs.append((O, Ws, x16, lo, hi))
    arr = spax.phase_array(phases)
    ws = torch.zeros(spax.spax_step_workspace_bytes(arr), dtype=torch.uint8, device=dev)
    for rep in range(2):
        spax.spax_decode_step_projections(arr, ws)
        for (L, packed, bufs), (O, Ws, x16, lo, hi) in zip(keep, refs):
            wt, wf, wa, wc = otiers.build_tiers(x16, otiers.MODE_TOPK_GUIDED, tau=-math.log(0.5),
                                                n_lo=lo, n_hi=hi, num=3, den=10)
            c = _np(bufs["c"])
            assert list(c) == list(wc)
            assert np.array_equal(_np(bufs["tier"])[:x16.size], wt)
            check_y_oracle(_np(bufs["y"]), O, Ws, x16, wf, wa, f"rep {rep}")
