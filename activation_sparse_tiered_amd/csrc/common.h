// Internal declarations shared by the libspax translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <exception>
#include <new>

#include "spax.h"

namespace spax {

// ------------------------------------------------------------------ errors
// Record a thread-local message and return the status.
int fail(int status, const char* fmt, ...);
void clear_error();
int hip_fail(hipError_t e, const char* what);

#define SPAX_HIP_CHECK(expr)                                   \
  do {                                                         \
    hipError_t e_ = (expr);                                    \
    if (e_ != hipSuccess) return ::spax::hip_fail(e_, #expr);  \
  } while (0)

// Runs f() (an entry point's body) and turns a C++ exception -- a host allocation or a host
// thread that could not be obtained -- into SPAX_ERR_HOST, so that no exception crosses the
// C ABI.
template <class F>
int no_throw(F&& f) noexcept {
  try {
    return f();
  } catch (const std::bad_alloc&) {
    return fail(SPAX_ERR_HOST, "host memory allocation failed");
  } catch (const std::exception& e) {
    return fail(SPAX_ERR_HOST, "host-side failure: %s", e.what());
  } catch (...) {
    return fail(SPAX_ERR_HOST, "host-side failure");
  }
}

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// ------------------------------------------------------------------ layout
// True if *L has been through spax_layout_init (derived fields consistent).
bool layout_ok(const spax_layout* L);

// ------------------------------------------------------------------ tier mask
// Tier parameters after host-side conversion: everything is integer on the device.
struct TierArgs {
  int32_t mode;
  int32_t d;
  int32_t n_full, n_approx;   // TOPK
  int32_t k_skip, k_full;     // THRESHOLD key thresholds
  int32_t k_tau;              // TOPK_GUIDED key threshold
  int32_t n_lo, n_hi, num, den;
};

// Validate *p against d and convert float thresholds to keys.
int tier_args_from_params(const spax_tier_params* p, int32_t d, TierArgs* out);

// y_zero/n_zero: an fp32 buffer the mask kernel also clears (NULL/0: none).
int launch_build_tiers(const TierArgs& a, const uint16_t* x, uint8_t* tier, int32_t* full_idx,
                       int32_t* approx_idx, int32_t* counts, float* y_zero, int64_t n_zero,
                       hipStream_t s);

// ------------------------------------------------------------------ pack
int launch_pack(const spax_layout* L, const uint16_t* const* W, const int32_t* perm,
                void* packed, hipStream_t s);

// ------------------------------------------------------------------ gemv
constexpr int kTileRows = 512;       // rows per workgroup tile (64 lanes x 8 rows)
// Rows per tile of the batched GEMV: an int4 layout's lanes own 32 rows each (one 16-byte
// code load per column), an fp16 layout's 8.  (The stand-alone GEMV, whose launch covers one
// phase, keeps 512-row tiles for both: it needs many small work items.)
inline int batched_tile_rows(const spax_layout* L) {
  return L->base_fmt == SPAX_FMT_INT4 ? 2048 : kTileRows;
}
#ifndef SPAX_GEMV_THREADS
#define SPAX_GEMV_THREADS 512
#endif
constexpr int kGemvThreads = SPAX_GEMV_THREADS;  // waves that share one tile, split the columns
constexpr int64_t kMaxRowsTotal = (int64_t)1 << 24;  // largest d_out_total of a layout

// Both regions of the layout's blob (FULL records, APPROX records) below 2 GiB: the GEMV kernels
// then address a column record from one buffer descriptor per region with a 32-bit offset
// (gemv::RegionBlob) instead of building a descriptor per record (gemv::RecordBlob).
inline bool narrow_regions(const spax_layout* L) {
  constexpr int64_t k2GiB = (int64_t)1 << 31;
  return L->off_A < k2GiB && (int64_t)L->d_in * L->stride_A < k2GiB;
}

struct GemvPlan {
  int32_t n_tiles;   // ceil(d_out_total / tile rows)
  int32_t n_chunks;  // split-K factor over the selected column lists
  size_t ws_bytes;   // workspace the launch needs (currently none)
};
GemvPlan gemv_plan(const spax_layout* L);

int launch_zero_f32(float* y, int64_t n, hipStream_t s);

// Largest y the single-workgroup mask kernel clears on the side.
constexpr int64_t kMaskClearMax = 65536;

// ------------------------------------------------------------------ decode step
// True if [a, a + na) and [b, b + nb) share a byte (false if either is empty or NULL).
bool overlaps(const void* a, size_t na, const void* b, size_t nb);
// True if [p, p + n) shares a byte with any buffer phase `ph` reads or writes: its x (whole
// dwords), tier bytes, both lists (d_in entries each), counts, blob and y.
bool phase_touches(const spax_phase& ph, const void* p, size_t n);
// The fused mask+GEMV kernel keeps the activations and its list slices in LDS.
constexpr int32_t kFusedMaxDin = 16384;
constexpr size_t kFusedMaxDynLds = 48 * 1024;
bool fused_phase_ok(const spax_layout* L);
// SPAX_STEP_BATCHED: workspace for the descriptor tables, and the two launches.
size_t batched_workspace_bytes(int n_phases);
int launch_decode_step_batched(const spax_step* st, int n_cu, hipStream_t s);
// The same with the descriptor tables in the library's static device scratch (no workspace,
// no allocation); at most kStaticScratchBytes of tables.
constexpr size_t kStaticScratchBytes = 256 * 1024;
int launch_decode_step_batched_static(const spax_step* st, int n_cu, hipStream_t s);
// Enqueue a validated step; noalloc: the batched form takes its tables from the static scratch.
int launch_decode_step(const spax_step* st, hipStream_t s, bool noalloc);

inline size_t aligned_size(size_t b) { return (b + 255) / 256 * 256; }

// ------------------------------------------------------------------ pinned-host path
// Ranges of an ascending list (-1 if it is not ascending / distinct / non-negative).
int32_t build_column_ranges(const int32_t* idx, int32_t n, int32_t gap, int32_t* first,
                            int32_t* count);
size_t pinned_workspace_bytes(const spax_layout* L);
// spax_placement_order after validation.
int placement_order(const spax_layout* L, const uint8_t* tiers, int32_t n_tokens,
                    int32_t* order);
// spax_storage_ledger after validation.
int storage_ledger(const spax_layout* L, const int32_t* full_idx, int32_t n_full,
                   const int32_t* approx_idx, int32_t n_approx, int32_t gap, int64_t block,
                   spax_storage_stats* out);
// Validated arguments; see spax_tiered_gemv_pinned.  host_dev: the device's address of the
// pinned blob (for SPAX_PINNED_GATHER).
int tiered_gemv_pinned(const spax_layout* L, const void* packed_host, const void* host_dev,
                       const uint16_t* x, const int32_t* full_idx, const int32_t* approx_idx,
                       const int32_t* counts, float* y, int32_t gap, int32_t transfer, void* ws,
                       spax_move_stats* stats, hipStream_t s);
// Pinned-host gather transfer with the ranges merged on the device: merge_ranges_kernel (two
// workgroups) writes the compacted lists, the slot tables and totals[6] = {slots F, slots A,
// ranges F, ranges A, entries F, entries A}; then one gather launch sized for the largest
// possible move reads the slot counts from totals.
int launch_merge_and_gather(const spax_layout* L, const void* host_dev, void* staging,
                            const int32_t* full_idx, const int32_t* approx_idx,
                            const int32_t* counts, int32_t gap, uint32_t* listF, uint32_t* listA,
                            int32_t* colF, int32_t* colA, int32_t* totals, hipStream_t s);
// y_zeroed: y already holds zeros (stream-ordered); otherwise a zero fill is enqueued first
// whenever the plan splits K.
// compact: the lists hold slot | channel << 16 entries into a compacted staging copy of the
// records, which `packed` then points to (pinned-host path).
// partials (deterministic mode): n_chunks x d_out_total floats; the chunks' partial sums are
// stored there and a second launch adds them in chunk order into y (y is then not cleared).
int launch_tiered_gemv(const spax_layout* L, const GemvPlan& plan, const void* packed,
                       const uint16_t* x, const int32_t* full_idx, const int32_t* approx_idx,
                       const int32_t* counts, float* y, bool y_zeroed, hipStream_t s,
                       bool compact = false, float* partials = nullptr);
// y = sum over the chunks of partials[c][0 .. T), c in increasing order (T a multiple of 4).
int launch_reduce_chunks(const float* partials, int32_t n_chunks, int64_t T, float* y,
                         hipStream_t s);
// Deterministic mode: bytes of the partial sums of the widest phase of a step (0 if none has
// more than one column chunk).
size_t deterministic_workspace_bytes(const spax_phase* phases, int32_t n_phases);

}  // namespace spax
