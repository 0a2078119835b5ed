"""Python binding of libspax: three-tier activation-sparse decoding GEMV on MI355X (gfx950).

Thin argument marshalling over the C ABI in ``include/spax.h``: every step of the path
(packing, tier masks, tiered GEMV, decode step) runs in the HIP kernels of libspax.so.
torch is used only for device memory (tensors are passed by ``data_ptr()``) and streams
(``torch.cuda.current_stream()`` by default).  The names match the C entry points.
"""

from __future__ import annotations

import ctypes as C

STEP_DEFAULT, STEP_SEPARATE, STEP_BATCHED, STEP_DETERMINISTIC = 0, 1, 2, 4

from ._lib import (FMT_FP16, FMT_INT4, MAX_DIN, MAX_MATS, MODE_THRESHOLD, MODE_TOPK,  # noqa: F401
                   MODE_TOPK_GUIDED, TIER_APPROX, TIER_FULL, TIER_SKIP, BLOCK_ERROR_FN,
                   SPAX_ERR_WORKSPACE, Layout, MoveStats, Phase, SpaxError, Step, StorageStats,
                   TierParams, check, lib, LIB_PATH)

__all__ = [
    "spax_layout_init", "spax_pack_columns", "spax_pack_columns_placed", "spax_placement_order",
    "spax_build_tiers", "spax_gemv_workspace_bytes",
    "spax_tiered_gemv", "spax_step_workspace_bytes", "spax_decode_step_projections",
    "spax_decode_step_projections_noalloc",
    "spax_key_threshold", "spax_counts_from_fractions", "spax_guided_bounds", "spax_version",
    "spax_column_ranges", "spax_pinned_workspace_bytes", "spax_tiered_gemv_pinned", "MoveStats",
    "spax_read_probe", "spax_storage_ledger", "StorageStats", "spax_block_sparsity",
    "spax_greedy_allocation", "spax_allocation_at",
    "topk_params", "threshold_params", "guided_params", "make_phase", "Layout", "TierParams",
    "Phase", "Step", "SpaxError", "LIB_PATH",
]


def _ptr(t) -> int:
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    return int(t.data_ptr())


def _stream(stream) -> int:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


# ------------------------------------------------------------------ layout / pack

def spax_layout_init(d_in: int, d_out, base_fmt: int = FMT_FP16, base_group: int = 128,
                     approx_group: int = 128) -> Layout:
    d_out = [int(v) for v in d_out]
    L = Layout()
    L.n_mats = len(d_out)
    L.d_in = int(d_in)
    for m, v in enumerate(d_out[:MAX_MATS]):
        L.d_out[m] = v
    L.base_fmt = int(base_fmt)
    L.base_group = int(base_group)
    L.approx_group = int(approx_group)
    if len(d_out) > MAX_MATS:
        L.n_mats = len(d_out)   # rejected by the library
    check(lib.spax_layout_init(C.byref(L)), "spax_layout_init")
    return L


def spax_pack_columns(layout: Layout, Ws, packed, stream=None) -> None:
    arr = (C.c_void_p * max(1, len(Ws)))(*[_ptr(w) for w in Ws])
    check(lib.spax_pack_columns(C.byref(layout), arr, _ptr(packed), _stream(stream)),
          "spax_pack_columns")


def spax_pack_columns_placed(layout: Layout, Ws, perm, packed, stream=None) -> None:
    """Pack with record p holding column perm[p] (perm: device int32 tensor of d_in)."""
    arr = (C.c_void_p * max(1, len(Ws)))(*[_ptr(w) for w in Ws])
    check(lib.spax_pack_columns_placed(C.byref(layout), arr, _ptr(perm), _ptr(packed),
                                       _stream(stream)), "spax_pack_columns_placed")


def spax_placement_order(layout: Layout, tiers):
    """Placement from calibration masks: ``tiers`` (n_tokens, d_in) uint8 on the host; returns
    the int32 order (position p holds channel order[p])."""
    import numpy as np
    t = np.ascontiguousarray(np.asarray(tiers, dtype=np.uint8))
    if t.ndim == 1:
        t = t[None, :]
    order = np.zeros(int(layout.d_in), dtype=np.int32)
    check(lib.spax_placement_order(C.byref(layout), t.ctypes.data if t.size else None,
                                   int(t.shape[0]), order.ctypes.data), "spax_placement_order")
    return order


# ------------------------------------------------------------------ tier masks

def topk_params(n_full: int, n_approx: int) -> TierParams:
    p = TierParams()
    p.mode, p.n_full, p.n_approx = MODE_TOPK, int(n_full), int(n_approx)
    p.approx_den = 1
    return p


def threshold_params(tau_skip: float, tau_full: float) -> TierParams:
    p = TierParams()
    p.mode, p.tau_skip, p.tau_full = MODE_THRESHOLD, float(tau_skip), float(tau_full)
    p.approx_den = 1
    return p


def guided_params(tau: float, n_skip_lo: int, n_skip_hi: int, approx_num: int,
                  approx_den: int) -> TierParams:
    p = TierParams()
    p.mode, p.tau = MODE_TOPK_GUIDED, float(tau)
    p.n_skip_lo, p.n_skip_hi = int(n_skip_lo), int(n_skip_hi)
    p.approx_num, p.approx_den = int(approx_num), int(approx_den)
    return p


def spax_build_tiers(x, d_in: int, params: TierParams, tier, full_idx, approx_idx, counts,
                     stream=None) -> None:
    check(lib.spax_build_tiers(_ptr(x), int(d_in), C.byref(params), _ptr(tier), _ptr(full_idx),
                               _ptr(approx_idx), _ptr(counts), _stream(stream)),
          "spax_build_tiers")


# ------------------------------------------------------------------ GEMV

def spax_gemv_workspace_bytes(layout: Layout) -> int:
    return int(lib.spax_gemv_workspace_bytes(C.byref(layout)))


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def spax_tiered_gemv(layout: Layout, packed, x, full_idx, approx_idx, counts, y, ws=None,
                     ws_bytes: int | None = None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = _nbytes(ws)
    check(lib.spax_tiered_gemv(C.byref(layout), _ptr(packed), _ptr(x), _ptr(full_idx),
                               _ptr(approx_idx), _ptr(counts), _ptr(y), _ptr(ws), int(ws_bytes),
                               _stream(stream)),
          "spax_tiered_gemv")


# ------------------------------------------------------------------ pinned-host path

def spax_column_ranges(idx, gap: int = 0):
    """Ascending channel indices -> [(first, count), ...] after merging gaps of <= gap."""
    import numpy as np
    a = np.ascontiguousarray(np.asarray(idx, dtype=np.int32))
    n = int(a.size)
    first = np.zeros(max(n, 1), dtype=np.int32)
    count = np.zeros(max(n, 1), dtype=np.int32)
    nr = C.c_int32()
    check(lib.spax_column_ranges(a.ctypes.data if n else None, n, int(gap), first.ctypes.data,
                                 count.ctypes.data, C.byref(nr)), "spax_column_ranges")
    return [(int(first[i]), int(count[i])) for i in range(nr.value)]


def spax_storage_ledger(layout: Layout, full_idx, approx_idx, gap: int = 0,
                        block_bytes: int = 4096) -> StorageStats:
    """Bytes selected against bytes physically read at a storage granularity (host lists)."""
    import numpy as np
    f = np.ascontiguousarray(np.asarray(full_idx, dtype=np.int32))
    a = np.ascontiguousarray(np.asarray(approx_idx, dtype=np.int32))
    out = StorageStats()
    check(lib.spax_storage_ledger(C.byref(layout), f.ctypes.data if f.size else None,
                                  int(f.size), a.ctypes.data if a.size else None, int(a.size),
                                  int(gap), int(block_bytes), C.byref(out)),
          "spax_storage_ledger")
    return out


def spax_pinned_workspace_bytes(layout: Layout) -> int:
    return int(lib.spax_pinned_workspace_bytes(C.byref(layout)))


PINNED_MEMCPY, PINNED_GATHER, PINNED_HOSTGATHER = 0, 1, 2


def spax_tiered_gemv_pinned(layout: Layout, packed_host, x, full_idx, approx_idx, counts, y,
                            gap: int, ws, ws_bytes: int | None = None, stream=None,
                            transfer: int = PINNED_MEMCPY, stats: bool = True):
    """The blob in pinned host memory (e.g. a torch tensor with pin_memory=True); returns the
    byte account of the call (MoveStats), or None with stats=False (the gather transfer then
    does not wait for the device)."""
    if ws_bytes is None:
        ws_bytes = _nbytes(ws)
    st = MoveStats() if stats else None
    check(lib.spax_tiered_gemv_pinned(C.byref(layout), _ptr(packed_host), _ptr(x), _ptr(full_idx),
                                      _ptr(approx_idx), _ptr(counts), _ptr(y), int(gap),
                                      int(transfer), _ptr(ws), int(ws_bytes),
                                      C.byref(st) if st is not None else None, _stream(stream)),
          "spax_tiered_gemv_pinned")
    return st


# ------------------------------------------------------------------ decode step

def make_phase(layout: Layout, packed, x, params: TierParams, tier, full_idx, approx_idx,
               counts, y) -> Phase:
    ph = Phase()
    ph.layout = C.pointer(layout)
    ph.packed, ph.x = _ptr(packed), _ptr(x)
    ph.params = params
    ph.tier, ph.full_idx, ph.approx_idx = _ptr(tier), _ptr(full_idx), _ptr(approx_idx)
    ph.counts, ph.y = _ptr(counts), _ptr(y)
    # The struct holds raw addresses: keep the layout and every buffer alive with it, so that
    # a caller dropping its own reference cannot free (and the allocator reuse) a buffer the
    # phase still points to.
    ph._keep = (layout, packed, x, tier, full_idx, approx_idx, counts, y)
    return ph


def phase_array(phases):
    arr = (Phase * len(phases))(*phases)
    arr._keep = [getattr(p, "_keep", None) for p in phases]  # the elements are copies
    return arr


def spax_step_workspace_bytes(phases) -> int:
    arr = phases if isinstance(phases, C.Array) else phase_array(phases)
    return int(lib.spax_step_workspace_bytes(arr, len(arr)))


def _step(phases, ws, ws_bytes, flags, events):
    arr = phases if isinstance(phases, C.Array) else phase_array(phases)
    if ws_bytes is None:
        ws_bytes = _nbytes(ws)
    st = Step()
    st.n_phases = len(arr)
    st.flags = int(flags)
    st.phases = C.cast(arr, C.POINTER(Phase))
    st.ws = _ptr(ws)
    st.ws_bytes = int(ws_bytes)
    if events is not None:
        if len(events) != 2 * len(arr):
            raise ValueError("need 2 * n_phases events")
        ev = (C.c_void_p * len(events))(*[int(e.cuda_event) for e in events])
        st.events = C.cast(ev, C.POINTER(C.c_void_p))
        st._keep = (arr, ev)
    else:
        st._keep = (arr,)
    return st


def spax_decode_step_projections(phases, ws, ws_bytes: int | None = None, flags: int = 0,
                                 stream=None, events=None) -> None:
    """``events``: optional list of 2 * n_phases torch.cuda.Event(enable_timing=True);
    events[2i] -> events[2i+1] then brackets phase i's GEMV launch on the stream."""
    st = _step(phases, ws, ws_bytes, flags, events)
    check(lib.spax_decode_step_projections(C.byref(st), _stream(stream)),
          "spax_decode_step_projections")


def spax_decode_step_projections_noalloc(phases, flags: int = 0, stream=None,
                                         events=None) -> None:
    """The same step with no workspace: the batched form keeps its descriptor tables in the
    library's static device scratch (calls on one GPU must not overlap)."""
    st = _step(phases, None, 0, flags, events)
    check(lib.spax_decode_step_projections_noalloc(C.byref(st), _stream(stream)),
          "spax_decode_step_projections_noalloc")


# ------------------------------------------------------------------ diagnostics

def spax_read_probe(buf, out, nbytes: int | None = None, offset: int = 0, stream=None) -> int:
    """Reads ``nbytes`` bytes of the device tensor ``buf`` from byte ``offset`` (default: all
    of it); every wave stores the XOR of the 32-bit words it read in its own word of the
    device tensor ``out`` (int32/uint32).  Returns how many leading words of ``out`` were
    written: their XOR is the XOR of all words read."""
    total = buf.numel() * buf.element_size()
    if nbytes is None:
        nbytes = total - offset
    if offset < 0 or nbytes < 0 or offset + nbytes > total:
        raise ValueError("read range outside the buffer")
    n = C.c_int32()
    words = out.numel() * out.element_size() // 4
    check(lib.spax_read_probe(C.c_void_p(_ptr(buf) + int(offset)), int(nbytes), _ptr(out),
                              int(min(words, 2**31 - 1)), C.byref(n), _stream(stream)),
          "spax_read_probe")
    return int(n.value)


# ------------------------------------------------------------------ sparsity budgets (host)

def spax_block_sparsity(sens, s: float, lam: float, s_min: float = 0.05, s_max: float = 0.95):
    """Per-block sparsity targets from block sensitivities (float64 array)."""
    import numpy as np
    a = np.ascontiguousarray(np.asarray(sens, dtype=np.float64))
    out = np.zeros(max(1, a.size), dtype=np.float64)
    check(lib.spax_block_sparsity(a.ctypes.data if a.size else None, int(a.size), float(s),
                                  float(lam), float(s_min), float(s_max), out.ctypes.data),
          "spax_block_sparsity")
    return out[:a.size]


def spax_greedy_allocation(params, alpha: float, P_max: float, block_error):
    """The greedy walk's rows as a float64 array [n_rows, 1 + n_mats] (P, then p per matrix).
    ``block_error(p)``: error of a trial allocation (a float64 array) -> float."""
    import numpy as np
    f = np.ascontiguousarray(np.asarray(params, dtype=np.float64))
    n = int(f.size)

    def _cb(p, n_mats, user):
        return float(block_error(np.ctypeslib.as_array(p, shape=(n_mats,)).copy()))

    cb = BLOCK_ERROR_FN(_cb)
    cap = 64
    while True:
        rows = np.zeros((cap, 1 + n), dtype=np.float64)
        nr = C.c_int32()
        st = lib.spax_greedy_allocation(f.ctypes.data if n else None, n, float(alpha),
                                        float(P_max), cb, None, rows.ctypes.data, cap,
                                        C.byref(nr))
        if st == SPAX_ERR_WORKSPACE and nr.value > cap:
            cap = nr.value
            continue
        check(st, "spax_greedy_allocation")
        return rows[:nr.value].copy()


def spax_allocation_at(rows, target: float):
    import numpy as np
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.float64))
    n_mats = r.shape[1] - 1
    p = np.zeros(max(1, n_mats), dtype=np.float64)
    check(lib.spax_allocation_at(r.ctypes.data, int(r.shape[0]), int(n_mats), float(target),
                                 p.ctypes.data), "spax_allocation_at")
    return p[:n_mats]


# ------------------------------------------------------------------ host helpers

def spax_key_threshold(tau: float) -> int:
    return int(lib.spax_key_threshold(float(tau)))


def spax_counts_from_fractions(d: int, p_full: float, p_approx: float):
    a, b = C.c_int32(), C.c_int32()
    check(lib.spax_counts_from_fractions(int(d), float(p_full), float(p_approx), C.byref(a),
                                         C.byref(b)), "spax_counts_from_fractions")
    return int(a.value), int(b.value)


def spax_guided_bounds(d: int, s: float, delta: float):
    a, b = C.c_int32(), C.c_int32()
    check(lib.spax_guided_bounds(int(d), float(s), float(delta), C.byref(a), C.byref(b)),
          "spax_guided_bounds")
    return int(a.value), int(b.value)


def spax_version() -> str:
    return lib.spax_version().decode()
