"""Pins for the oracle's quantizer and packed blob (host only).

Pinned against: hand-derived byte images (tests/golden/pack_tiny.json), exact rational
brute force of the nearest level, closed-form invariants of min-max quantization, and
weights that lie exactly on the quantization levels (whose approximation must be exact).
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import pack, quant
from tests.conftest import load_golden


def _column(pattern, rows):
    p = [float(v) for v in pattern]
    return np.array([p[r % len(p)] for r in range(rows)], dtype=np.float64).astype(np.float16)


def _fmt(name):
    return pack.FMT_FP16 if name == "fp16" else pack.FMT_INT4


def test_pack_golden_bytes():
    g = load_golden("pack_tiny.json")
    for c in g["cases"]:
        L = pack.Layout(c["d_in"], c["d_out"], _fmt(c["base_fmt"]), c["base_group"],
                        c["approx_group"])
        assert (L.stride_F, L.stride_A, L.off_A, L.total_bytes) == (
            c["stride_F"], c["stride_A"], c["off_A"], c["total"]), c["name"]
        T = L.d_out_total
        W = np.stack([_column(p, T) for p in c["columns"]])     # (d_in, T)
        blob = pack.pack_columns(L, [W])
        for region, stride, base in (("F", L.stride_F, 0), ("A", L.stride_A, L.off_A)):
            for j, parts in enumerate(c[region]):
                want = b"".join(bytes.fromhex(h) * n for h, n in parts)
                want = want + bytes(stride - len(want))
                got = bytes(blob[base + j * stride: base + (j + 1) * stride])
                assert got == want, (c["name"], region, j)


def _exact(v16):
    return Fraction(float(v16))


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("seed", range(25))
def test_quantizer_bruteforce_nearest_level(bits, seed):
    """Every code is the level s*q+z nearest to w (exact rationals), except true near-ties."""
    rng = np.random.default_rng(seed)
    G = int(rng.choice([4, 8, 64, 128]))
    scale = float(rng.choice([0.02, 1.0, 1e-4, 300.0]))
    w = (rng.standard_normal(G) * scale).astype(np.float16)
    s16, z16, q = quant.quantize_group(w, bits)
    L = (1 << bits) - 1
    s, z = _exact(s16), _exact(z16)
    near_ties = 0
    for i in range(G):
        wi = _exact(w[i])
        if s == 0:
            assert q[i] == 0
            continue
        dists = [abs(wi - (s * k + z)) for k in range(L + 1)]
        best = min(dists)
        cands = [k for k in range(L + 1) if dists[k] == best]
        t = (wi - z) / s
        frac_dist = abs(t - (int(t) + Fraction(1, 2)))
        if frac_dist < Fraction(1, 2**20):
            near_ties += 1
            assert q[i] in (int(t), int(t) + 1) or q[i] == L
            continue
        assert int(q[i]) in cands, (i, float(wi), int(q[i]), cands)
    assert near_ties <= 1


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("seed", range(25))
def test_quantizer_invariants(bits, seed):
    rng = np.random.default_rng(500 + seed)
    G = int(rng.choice([64, 128]))
    w = (rng.standard_normal(G) * 0.02).astype(np.float16)
    s16, z16, q = quant.quantize_group(w, bits)
    L = (1 << bits) - 1
    w64 = w.astype(np.float64)
    # z is the group minimum exactly (as a value; -0 becomes +0)
    assert float(z16) == w64.min()
    # s is within half an fp16 spacing (+ the float32 step) of (max - min) / L
    s_exact = (w64.max() - w64.min()) / L
    assert abs(float(s16) - s_exact) <= abs(s_exact) * (2.0**-11 + 2.0**-22)
    # min element -> code 0, max element -> code L
    assert q[np.argmin(w64)] == 0
    assert q[np.argmax(w64)] == L
    # reconstruction error bound |w - w_hat| <= s/2 (1 + 2^-9)
    w_hat = quant.dequant(s16, z16, q)
    assert np.max(np.abs(w_hat - w64)) <= float(s16) / 2 * (1 + 2.0**-9)
    assert q.max() <= L


def test_quantizer_constant_group():
    for v in [0.0, -0.0, 1.5, -3.0]:
        w = np.full(64, v, dtype=np.float16)
        s16, z16, q = quant.quantize_group(w, 2)
        assert float(s16) == 0.0 and not np.any(q)
        assert np.array_equal(quant.dequant(s16, z16, q), w.astype(np.float64))
        assert np.float16(z16).view(np.uint16) == np.float16(abs(v) if v == 0 else v).view(np.uint16)


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("seed", range(10))
def test_exact_level_weights_reconstruct_exactly(bits, seed):
    """Weights exactly on {z + k*s} with power-of-two s, z and every level present
    reconstruct without error."""
    rng = np.random.default_rng(800 + seed)
    L = (1 << bits) - 1
    G = 64
    s = 2.0 ** int(rng.integers(-12, 2))
    z = -(2.0 ** int(rng.integers(-10, 3)))
    k = rng.integers(0, L + 1, G)
    k[:L + 1] = np.arange(L + 1)
    rng.shuffle(k)
    w = (z + k * s).astype(np.float16)
    assert np.array_equal(w.astype(np.float64), z + k * s)
    s16, z16, q = quant.quantize_group(w, bits)
    assert float(s16) == s and float(z16) == z
    assert np.array_equal(q, k)
    assert np.array_equal(quant.dequant(s16, z16, q), w.astype(np.float64))


@pytest.mark.parametrize("base", ["fp16", "int4"])
@pytest.mark.parametrize("seed", range(6))
def test_blob_decodes_to_definition(base, seed):
    """The blob decoder returns the same values as the definition (fp16 master for the
    original fp16 tier, per-group reconstructions otherwise), for fused matrices."""
    rng = np.random.default_rng(900 + seed)
    d_in = int(rng.integers(1, 40))
    G = 128 if base == "int4" else int(rng.choice([64, 128]))
    d_out = [G * int(rng.integers(1, 5)) for _ in range(int(rng.integers(1, 4)))]
    L = pack.Layout(d_in, d_out, _fmt(base), 128, G)
    Ws = [(rng.standard_normal((d_in, r)) * 0.02).astype(np.float16) for r in d_out]
    blob = pack.pack_columns(L, Ws)
    assert blob.size == L.total_bytes
    assert L.stride_F % 128 == 0 and L.stride_A % 128 == 0
    assert np.array_equal(pack.decode_full_region(L, blob), pack.full_values(L, Ws))
    assert np.array_equal(pack.decode_approx_region(L, blob), pack.approx_values(L, Ws))
    # fp16 region holds the master bits
    if base == "fp16":
        cat = np.concatenate(Ws, axis=1)
        rec = blob[:L.off_A].reshape(d_in, L.stride_F)[:, :2 * L.d_out_total]
        assert np.array_equal(np.ascontiguousarray(rec).view("<f2"), cat)
    # padding is zero
    recA = blob[L.off_A:].reshape(d_in, L.stride_A)
    assert not np.any(recA[:, L.rec_A:])
    recF = blob[:L.off_A].reshape(d_in, L.stride_F)
    assert not np.any(recF[:, L.rec_F:])


def test_layout_closed_forms():
    """Record sizes of the 7B shapes: fp16 2*T; int4 T/2 + 4*T/128; 2-bit T/4 + 4*T/G."""
    for T, G, sA in [(512, 64, 256), (4096, 128, 1152), (11008, 128, 3200),
                     (12288, 128, 3456), (22016, 128, 6272), (6144, 128, 1792),
                     (28672, 128, 8064)]:
        L = pack.Layout(7, [T], pack.FMT_FP16, 128, G)
        assert L.rec_A == T // 4 + 4 * T // G
        assert L.stride_A == sA
        assert L.stride_F == 2 * T
    L = pack.Layout(3, [4096], pack.FMT_INT4, 128, 128)
    assert L.rec_F == 2176 and L.stride_F == 2176
    L = pack.Layout(3, [22016], pack.FMT_INT4, 128, 128)
    assert L.rec_F == 11696 and L.stride_F == 11776
    with pytest.raises(ValueError):
        pack.Layout(3, [100], pack.FMT_FP16, 128, 64)
