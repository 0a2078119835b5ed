"""ctypes view of libspax.so (the C ABI declared in include/spax.h).

Loads the in-tree library built by ``activation_sparse_tiered_amd/build.py``.  There is no
fallback: if the library is missing, importing this module raises.
"""

from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspax.so")

SPAX_OK = 0
STATUS_NAMES = {0: "SPAX_OK", -1: "SPAX_ERR_NULL", -2: "SPAX_ERR_SHAPE", -3: "SPAX_ERR_PARAM",
                -4: "SPAX_ERR_ALIGN", -5: "SPAX_ERR_WORKSPACE", -6: "SPAX_ERR_HIP",
                -7: "SPAX_ERR_UNSUPPORTED", -8: "SPAX_ERR_HOST"}
SPAX_ERR_NULL, SPAX_ERR_SHAPE, SPAX_ERR_PARAM, SPAX_ERR_ALIGN = -1, -2, -3, -4
SPAX_ERR_WORKSPACE, SPAX_ERR_HIP, SPAX_ERR_UNSUPPORTED, SPAX_ERR_HOST = -5, -6, -7, -8

FMT_FP16, FMT_INT4 = 0, 1
MODE_TOPK, MODE_THRESHOLD, MODE_TOPK_GUIDED = 0, 1, 2
TIER_SKIP, TIER_APPROX, TIER_FULL = 0, 1, 2
MAX_MATS = 4
MAX_DIN = 32768


class Layout(C.Structure):
    _fields_ = [("n_mats", C.c_int32), ("d_in", C.c_int32), ("d_out", C.c_int32 * MAX_MATS),
                ("base_fmt", C.c_int32), ("base_group", C.c_int32), ("approx_group", C.c_int32),
                ("reserved0", C.c_int32),
                ("d_out_total", C.c_int64), ("rec_F", C.c_int64), ("rec_A", C.c_int64),
                ("stride_F", C.c_int64), ("stride_A", C.c_int64), ("off_A", C.c_int64),
                ("total_bytes", C.c_int64)]

    @property
    def d_outs(self):
        return [int(self.d_out[m]) for m in range(self.n_mats)]


class TierParams(C.Structure):
    _fields_ = [("mode", C.c_int32), ("n_full", C.c_int32), ("n_approx", C.c_int32),
                ("n_skip_lo", C.c_int32), ("n_skip_hi", C.c_int32),
                ("approx_num", C.c_int32), ("approx_den", C.c_int32), ("reserved0", C.c_int32),
                ("tau_skip", C.c_double), ("tau_full", C.c_double), ("tau", C.c_double)]


class Phase(C.Structure):
    _fields_ = [("layout", C.POINTER(Layout)), ("packed", C.c_void_p), ("x", C.c_void_p),
                ("params", TierParams), ("tier", C.c_void_p), ("full_idx", C.c_void_p),
                ("approx_idx", C.c_void_p), ("counts", C.c_void_p), ("y", C.c_void_p)]


class Step(C.Structure):
    _fields_ = [("n_phases", C.c_int32), ("flags", C.c_int32), ("phases", C.POINTER(Phase)),
                ("ws", C.c_void_p), ("ws_bytes", C.c_size_t), ("events", C.POINTER(C.c_void_p))]


class StorageStats(C.Structure):
    _fields_ = [("selected_bytes", C.c_int64), ("moved_bytes", C.c_int64),
                ("read_bytes", C.c_int64), ("n_blocks", C.c_int64), ("n_ranges", C.c_int32),
                ("reserved0", C.c_int32)]


class MoveStats(C.Structure):
    _fields_ = [("selected_bytes", C.c_int64), ("moved_bytes", C.c_int64),
                ("list_bytes", C.c_int64), ("n_ranges", C.c_int32), ("n_full", C.c_int32),
                ("n_approx", C.c_int32), ("reserved0", C.c_int32)]


def _hip_runtimes():
    """Paths of the HIP runtime libraries mapped into this process."""
    out = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    out.add(line.split()[-1])
    except OSError:
        pass
    return out


# double (*)(const double* p, int32_t n_mats, void* user)
BLOCK_ERROR_FN = C.CFUNCTYPE(C.c_double, C.POINTER(C.c_double), C.c_int32, C.c_void_p)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                          "python activation_sparse_tiered_amd/build.py")
    # torch owns the device memory and the streams we are handed, so libspax must bind to the
    # HIP runtime torch has loaded.  Loading torch first makes libspax's libamdhip64.so.7
    # dependency resolve to that already-loaded copy (same soname); a second runtime in the
    # process would not see torch's streams or allocations.
    import torch  # noqa: F401
    lib = C.CDLL(LIB_PATH)
    rts = _hip_runtimes()
    if len(rts) > 1:
        raise ImportError(f"two HIP runtimes are mapped ({sorted(rts)}); import torch before "
                          f"loading {LIB_PATH}")
    P = C.c_void_p
    sig = {
        "spax_layout_init": (C.c_int, [C.POINTER(Layout)]),
        "spax_pack_columns": (C.c_int, [C.POINTER(Layout), C.POINTER(C.c_void_p), P, P]),
        "spax_pack_columns_placed": (C.c_int, [C.POINTER(Layout), C.POINTER(C.c_void_p), P, P,
                                               P]),
        "spax_placement_order": (C.c_int, [C.POINTER(Layout), P, C.c_int32, P]),
        "spax_build_tiers": (C.c_int, [P, C.c_int32, C.POINTER(TierParams), P, P, P, P, P]),
        "spax_gemv_workspace_bytes": (C.c_size_t, [C.POINTER(Layout)]),
        "spax_tiered_gemv": (C.c_int, [C.POINTER(Layout), P, P, P, P, P, P, P, C.c_size_t, P]),
        "spax_step_workspace_bytes": (C.c_size_t, [C.POINTER(Phase), C.c_int32]),
        "spax_decode_step_projections": (C.c_int, [C.POINTER(Step), P]),
        "spax_decode_step_projections_noalloc": (C.c_int, [C.POINTER(Step), P]),
        "spax_column_ranges": (C.c_int, [P, C.c_int32, C.c_int32, P, P, C.POINTER(C.c_int32)]),
        "spax_pinned_workspace_bytes": (C.c_size_t, [C.POINTER(Layout)]),
        "spax_storage_ledger": (C.c_int, [C.POINTER(Layout), P, C.c_int32, P, C.c_int32,
                                          C.c_int32, C.c_int64, C.POINTER(StorageStats)]),
        "spax_tiered_gemv_pinned": (C.c_int, [C.POINTER(Layout), P, P, P, P, P, P, C.c_int32,
                                              C.c_int32, P, C.c_size_t, C.POINTER(MoveStats), P]),
        "spax_read_probe": (C.c_int, [P, C.c_size_t, P, C.c_int32, C.POINTER(C.c_int32), P]),
        "spax_key_threshold": (C.c_int32, [C.c_double]),
        "spax_counts_from_fractions": (C.c_int, [C.c_int32, C.c_double, C.c_double,
                                                 C.POINTER(C.c_int32), C.POINTER(C.c_int32)]),
        "spax_guided_bounds": (C.c_int, [C.c_int32, C.c_double, C.c_double,
                                         C.POINTER(C.c_int32), C.POINTER(C.c_int32)]),
        "spax_block_sparsity": (C.c_int, [P, C.c_int32, C.c_double, C.c_double, C.c_double,
                                          C.c_double, P]),
        "spax_greedy_allocation": (C.c_int, [P, C.c_int32, C.c_double, C.c_double,
                                             BLOCK_ERROR_FN, P, P, C.c_int32,
                                             C.POINTER(C.c_int32)]),
        "spax_allocation_at": (C.c_int, [P, C.c_int32, C.c_int32, C.c_double, P]),
        "spax_status_string": (C.c_char_p, [C.c_int]),
        "spax_last_error": (C.c_char_p, []),
        "spax_version": (C.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


lib = _load()


class SpaxError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.spax_last_error().decode(errors="replace")
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {msg}")


def check(status: int, where: str) -> None:
    if status != SPAX_OK:
        raise SpaxError(status, where)
