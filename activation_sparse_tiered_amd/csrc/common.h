// Internal declarations shared by the libspax translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

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
int launch_pack(const spax_layout* L, const uint16_t* const* W, void* packed, hipStream_t s);

// ------------------------------------------------------------------ gemv
constexpr int kTileRows = 512;       // rows per workgroup tile (64 lanes x 8 rows)
#ifndef SPAX_GEMV_THREADS
#define SPAX_GEMV_THREADS 512
#endif
constexpr int kGemvThreads = SPAX_GEMV_THREADS;  // waves that share one tile, split the columns
constexpr int64_t kMaxRowsTotal = (int64_t)1 << 24;  // largest d_out_total of a layout

struct GemvPlan {
  int32_t n_tiles;   // ceil(d_out_total / kTileRows)
  int32_t n_chunks;  // split-K factor over the selected column lists
  size_t ws_bytes;   // workspace the launch needs (currently none)
};
GemvPlan gemv_plan(const spax_layout* L);

int launch_zero_f32(float* y, int64_t n, hipStream_t s);

// Largest y the single-workgroup mask kernel clears on the side.
constexpr int64_t kMaskClearMax = 65536;

// ------------------------------------------------------------------ decode step
// The fused mask+GEMV kernel keeps the activations and its list slices in LDS.
constexpr int32_t kFusedMaxDin = 16384;
constexpr size_t kFusedMaxDynLds = 48 * 1024;
bool fused_phase_ok(const spax_layout* L);
// Enqueue a validated step.
int launch_decode_step(const spax_step* st, hipStream_t s);
// SPAX_STEP_BATCHED: workspace for the descriptor tables, and the two launches.
size_t batched_workspace_bytes(int n_phases);
int launch_decode_step_batched(const spax_step* st, int n_cu, hipStream_t s);

inline size_t aligned_size(size_t b) { return (b + 255) / 256 * 256; }

// ------------------------------------------------------------------ pinned-host path
// Ranges of an ascending list (-1 if it is not ascending / distinct / non-negative).
int32_t build_column_ranges(const int32_t* idx, int32_t n, int32_t gap, int32_t* first,
                            int32_t* count);
size_t pinned_workspace_bytes(const spax_layout* L);
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
int launch_tiered_gemv(const spax_layout* L, const GemvPlan& plan, const void* packed,
                       const uint16_t* x, const int32_t* full_idx, const int32_t* approx_idx,
                       const int32_t* counts, float* y, bool y_zeroed, hipStream_t s,
                       bool compact = false);

}  // namespace spax
