"""Storage-granularity byte ledger (eigenradar commentary on SpAx, "The route outside GPU
memory", third and last paragraphs): oracle/ranges.py's storage_ledger pinned on hand-worked
cases and by brute force over the bytes of each read, and the C ABI's spax_storage_ledger
against the oracle.  Host only."""

import numpy as np
import pytest

import activation_sparse_tiered_amd as spax
from activation_sparse_tiered_amd import _lib
from oracle import pack as opack
from oracle import ranges


def test_hand_worked():
    """d_in = 8, 4096 fp16 rows, two-bit groups of 128: stride_F = 8192, stride_A = 1024 +
    32 * 4 = 1152, off_A = 8 * 8192 = 65536; blocks of 4096 bytes.
    FULL {1, 2, 5}: ranges (1, 2) = bytes [8192, 24576) = blocks 2..5 (4) and (5, 1) =
    [40960, 49152) = blocks 10, 11 (2).  APPROX {0, 3, 4, 7}: (0, 1) = [65536, 66688) =
    block 16; (3, 2) = [68992, 71296) = blocks 16, 17; (7, 1) = [73600, 74752) = blocks 17,
    18.  11 blocks read = 45056 bytes for 3 * 8192 + 4 * 1152 = 29184 selected.
    With gap 2 every region is one range: FULL 1..5 = [8192, 49152) = 10 blocks, APPROX 0..7
    = [65536, 74752) = 3 blocks; 13 blocks = 53248 bytes, moved 5 * 8192 + 8 * 1152."""
    L = opack.Layout(8, [4096], opack.FMT_FP16, 128, 128)
    assert (L.stride_F, L.stride_A, L.off_A) == (8192, 1152, 65536)
    f, a = [1, 2, 5], [0, 3, 4, 7]
    led = ranges.storage_ledger(f, a, L.stride_F, L.stride_A, L.off_A, 4096, 0)
    assert led == {"selected_bytes": 29184, "moved_bytes": 29184, "read_bytes": 45056,
                   "n_ranges": 5, "n_blocks": 11}
    assert ranges.storage_ledger(f, a, L.stride_F, L.stride_A, L.off_A, 4096, 1) == led
    led2 = ranges.storage_ledger(f, a, L.stride_F, L.stride_A, L.off_A, 4096, 2)
    assert led2 == {"selected_bytes": 29184, "moved_bytes": 5 * 8192 + 8 * 1152,
                    "read_bytes": 53248, "n_ranges": 2, "n_blocks": 13}
    S = spax.spax_layout_init(8, [4096], 0, 128, 128)
    st = spax.spax_storage_ledger(S, f, a, 0, 4096)
    assert (st.selected_bytes, st.moved_bytes, st.read_bytes, st.n_ranges, st.n_blocks) == \
        (29184, 29184, 45056, 5, 11)


@pytest.mark.parametrize("seed", range(30))
def test_brute_force_over_bytes(seed):
    """Blocks read = for each range, the distinct values of byte // block over its bytes."""
    rng = np.random.default_rng(seed)
    d = int(rng.integers(1, 40))
    sF, sA = int(rng.choice([128, 256, 384])), int(rng.choice([128, 256]))
    off = d * sF
    block = int(rng.choice([1, 96, 128, 500, 1024, 4096]))
    gap = int(rng.integers(0, 4))
    sel = rng.permutation(d)
    nf = int(rng.integers(0, d + 1))
    na = int(rng.integers(0, d - nf + 1))
    f, a = sorted(sel[:nf].tolist()), sorted(sel[nf:nf + na].tolist())
    led = ranges.storage_ledger(f, a, sF, sA, off, block, gap)
    blocks = 0
    for idx, stride, base in ((f, sF, 0), (a, sA, off)):
        for first, count in ranges.runs(idx, gap):
            blocks += len({b // block for b in range(base + first * stride,
                                                     base + (first + count) * stride)})
    assert led["n_blocks"] == blocks and led["read_bytes"] == blocks * block
    assert led["read_bytes"] >= led["moved_bytes"] >= led["selected_bytes"]
    if block == 1 or (sF % block == 0 and sA % block == 0):
        assert led["read_bytes"] == led["moved_bytes"]


@pytest.mark.parametrize("seed", range(12))
def test_abi_matches_oracle(seed):
    rng = np.random.default_rng(50 + seed)
    d = int(rng.integers(1, 3000))
    d_out = [int(rng.choice([512, 1024, 4096, 11008 // 128 * 128]))]
    fmt = int(rng.integers(0, 2))
    O = opack.Layout(d, d_out, fmt, 128, 128)
    L = spax.spax_layout_init(d, d_out, fmt, 128, 128)
    sel = rng.permutation(d)
    nf = int(rng.integers(0, d + 1))
    na = int(rng.integers(0, d - nf + 1))
    f, a = sorted(sel[:nf].tolist()), sorted(sel[nf:nf + na].tolist())
    for block in (512, 4096, 65536):
        for gap in (0, 3):
            led = ranges.storage_ledger(f, a, O.stride_F, O.stride_A, O.off_A, block, gap)
            st = spax.spax_storage_ledger(L, f, a, gap, block)
            assert (st.selected_bytes, st.moved_bytes, st.read_bytes, st.n_ranges,
                    st.n_blocks) == (led["selected_bytes"], led["moved_bytes"],
                                     led["read_bytes"], led["n_ranges"], led["n_blocks"])


def test_abi_errors():
    L = spax.spax_layout_init(8, [512], 0, 128, 128)
    for f, a, gap, block in (([3, 1], [], 0, 4096), ([1], [9], 0, 4096), ([1], [], -1, 4096),
                             ([1], [], 0, 0), (list(range(8)), [0], 0, 4096)):
        with pytest.raises(spax.SpaxError) as e:
            spax.spax_storage_ledger(L, f, a, gap, block)
        assert e.value.status == _lib.SPAX_ERR_PARAM, (f, a, gap, block)


# ---------------------------------------------------------------- placement

def test_placement_hand_worked():
    """Scores with stride_F = 8192, stride_A = 1152 over three tokens:
    channel 0: F, F, S -> 16384; 1: A, A, A -> 3456; 2: S, S, S -> 0; 3: F, A, S -> 9344;
    4: F, F, S -> 16384.  Order: 0, 4 (16384; ties by index), 3, 1, 2."""
    t = np.array([[2, 1, 0, 2, 2], [2, 1, 0, 1, 2], [0, 1, 0, 0, 0]])
    assert ranges.placement_order(t, 8192, 1152).tolist() == [0, 4, 3, 1, 2]


@pytest.mark.parametrize("seed", range(10))
def test_placement_joins_columns_always_used_together(seed):
    """If every calibration token selects the same FULL set and the same APPROX set, the
    placed blob holds each set as one contiguous run (FULL first, then APPROX), so each token
    reads one range per region; and the order is a permutation."""
    rng = np.random.default_rng(seed)
    d = int(rng.integers(3, 300))
    tier = rng.integers(0, 3, d)
    calib = np.tile(tier, (int(rng.integers(1, 6)), 1))
    order = ranges.placement_order(calib, 8192, 1152)
    assert sorted(order.tolist()) == list(range(d))
    placed = tier[order]                      # the tier of the channel at each position
    full_pos = np.flatnonzero(placed == 2)
    apx_pos = np.flatnonzero(placed == 1)
    assert len(ranges.runs(full_pos)) <= 1 and len(ranges.runs(apx_pos)) <= 1
    if full_pos.size and apx_pos.size:
        assert full_pos.max() < apx_pos.min()


@pytest.mark.parametrize("seed", range(8))
def test_placement_abi_matches_oracle(seed):
    rng = np.random.default_rng(70 + seed)
    d = int(rng.integers(1, 5000))
    L = spax.spax_layout_init(d, [1024], 0, 128, 128)
    T = int(rng.integers(1, 20))
    calib = rng.choice([0, 1, 2], size=(T, d), p=[0.5, 0.3, 0.2]).astype(np.uint8)
    got = spax.spax_placement_order(L, calib)
    assert np.array_equal(got, ranges.placement_order(calib, int(L.stride_F), int(L.stride_A)))
    with pytest.raises(spax.SpaxError):
        bad = calib.copy()
        bad[0, 0] = 3
        spax.spax_placement_order(L, bad)
