// Entry points of libspax: argument validation, then kernel launches.
// Every check runs before anything is enqueued; on error no output is touched.
#include <algorithm>
#include <mutex>
#include <vector>
#include <cstdio>
#include <cstring>

#include "common.h"

using namespace spax;

namespace {

// Prefix the current thread-local message with the phase number.
int phase_fail(int st, int i) {
  char msg[400];
  snprintf(msg, sizeof(msg), "%s", spax_last_error());
  return fail(st, "phase %d: %s", i, msg);
}

int check_tier_outputs(const uint16_t* x, int32_t d_in, const int32_t* full_idx,
                       const int32_t* approx_idx, const int32_t* counts) {
  if (!x || !full_idx || !approx_idx || !counts)
    return fail(SPAX_ERR_NULL, "x, full_idx, approx_idx and counts are required");
  if (d_in < 1 || d_in > SPAX_MAX_DIN)
    return fail(SPAX_ERR_SHAPE, "d_in %d outside 1..%d", d_in, SPAX_MAX_DIN);
  if (!aligned(x, 4) || !aligned(full_idx, 4) || !aligned(approx_idx, 4) || !aligned(counts, 4))
    return fail(SPAX_ERR_ALIGN, "x, lists and counts must be 4-byte aligned");
  return SPAX_OK;
}

// SPAX_STEP_BATCHED runs all phases at once: no output may overlap another output or any
// input x.
struct Range {
  uintptr_t b, e;
  int phase;
  bool out;
};
constexpr int kRangesPerPhase = 7;
// The check over a caller-provided buffer of kRangesPerPhase ranges per phase.
int check_independent_in(const spax_step* st, Range* buf) {
  Range* end = buf;
  for (int i = 0; i < st->n_phases; ++i) {
    const spax_phase& ph = st->phases[i];
    const spax_layout* L = ph.layout;
    const auto add = [&](const void* p, size_t n, bool out) {
      if (p && n) *end++ = Range{(uintptr_t)p, (uintptr_t)p + n, i, out};
    };
    add(ph.x, 2 * (size_t)L->d_in, false);
    add(ph.packed, (size_t)L->total_bytes, false);
    add(ph.tier, (size_t)L->d_in, true);
    add(ph.full_idx, 4 * (size_t)L->d_in, true);
    add(ph.approx_idx, 4 * (size_t)L->d_in, true);
    add(ph.counts, 12, true);
    add(ph.y, 4 * (size_t)L->d_out_total, true);
  }
  std::sort(buf, end, [](const Range& a, const Range& b) { return a.b < b.b; });
  // any overlap involving an output is an error (two inputs may share memory)
  uintptr_t end_out = 0, end_any = 0;
  int ph_out = -1, ph_any = -1;
  for (const Range* px = buf; px != end; ++px) {
    const Range& x = *px;
    if (x.b < end_out) return fail(SPAX_ERR_PARAM, "batched step: phase %d overlaps an output of phase %d", x.phase, ph_out);
    if (x.out && x.b < end_any) return fail(SPAX_ERR_PARAM, "batched step: an output of phase %d overlaps phase %d", x.phase, ph_any);
    if (x.out && x.e > end_out) { end_out = x.e; ph_out = x.phase; }
    if (x.e > end_any) { end_any = x.e; ph_any = x.phase; }
  }
  return SPAX_OK;
}

// noalloc: the ranges go to a static buffer (the no-alloc step holds at most
// kNoallocMaxPhases phases: its descriptor tables must fit the static device scratch), taken
// under a lock, so the check allocates nothing.
constexpr int kNoallocMaxPhases = 2048;
int check_independent(const spax_step* st, bool noalloc) {
  if (noalloc) {
    if (st->n_phases > kNoallocMaxPhases)
      return fail(SPAX_ERR_WORKSPACE, "%d phases: the no-alloc step takes at most %d",
                  st->n_phases, kNoallocMaxPhases);
    static std::mutex mu;
    static Range buf[kRangesPerPhase * kNoallocMaxPhases];
    std::lock_guard<std::mutex> lock(mu);
    return check_independent_in(st, buf);
  }
  std::vector<Range> r((size_t)kRangesPerPhase * (size_t)st->n_phases);
  return check_independent_in(st, r.data());
}

// Within one phase of a step, no output (tier bytes, lists, counts, y) shares a byte with
// another output or with the phase's inputs (x, blob): the phase's kernels read and write
// them concurrently.  Phases may share buffers with each other (stream order).
int check_phase_aliasing(const spax_phase& ph) {
  const spax_layout* L = ph.layout;
  const size_t d = (size_t)L->d_in;
  struct Buf {
    const void* p;
    size_t n;
    const char* name;
  };
  const Buf out[] = {{ph.tier, d, "tier"},
                     {ph.full_idx, 4 * d, "full_idx"},
                     {ph.approx_idx, 4 * d, "approx_idx"},
                     {ph.counts, 12, "counts"},
                     {ph.y, 4 * (size_t)L->d_out_total, "y"}};
  const Buf in[] = {{ph.x, 4 * ((d + 1) / 2), "x"}, {ph.packed, (size_t)L->total_bytes, "packed"}};
  for (size_t i = 0; i < sizeof(out) / sizeof(out[0]); ++i) {
    for (size_t k = i + 1; k < sizeof(out) / sizeof(out[0]); ++k)
      if (overlaps(out[i].p, out[i].n, out[k].p, out[k].n))
        return fail(SPAX_ERR_PARAM, "%s overlaps %s of the same phase", out[i].name, out[k].name);
    for (const Buf& b : in)
      if (overlaps(out[i].p, out[i].n, b.p, b.n))
        return fail(SPAX_ERR_PARAM, "%s overlaps %s of the same phase", out[i].name, b.name);
  }
  return SPAX_OK;
}

int check_gemv_args(const spax_layout* L, const void* packed, const uint16_t* x,
                    const int32_t* full_idx, const int32_t* approx_idx, const int32_t* counts,
                    const float* y, const void* ws, size_t ws_bytes, GemvPlan* plan) {
  if (!L) return fail(SPAX_ERR_NULL, "layout is NULL");
  if (!layout_ok(L)) return fail(SPAX_ERR_SHAPE, "layout not initialised by spax_layout_init");
  if (!packed || !x || !full_idx || !approx_idx || !counts || !y)
    return fail(SPAX_ERR_NULL, "a required pointer is NULL");
  if (!aligned(packed, 256) || !aligned(ws, 256))
    return fail(SPAX_ERR_ALIGN, "packed and ws must be 256-byte aligned");
  if (!aligned(x, 4) || !aligned(full_idx, 4) || !aligned(approx_idx, 4) || !aligned(counts, 4) ||
      !aligned(y, 16))
    return fail(SPAX_ERR_ALIGN, "x/lists/counts must be 4-byte aligned and y 16-byte aligned");
  if (overlaps(y, 4 * (size_t)L->d_out_total, packed, (size_t)L->total_bytes) ||
      overlaps(y, 4 * (size_t)L->d_out_total, x, 4 * (((size_t)L->d_in + 1) / 2)))
    return fail(SPAX_ERR_PARAM, "y overlaps the blob or x");
  *plan = gemv_plan(L);
  if (plan->ws_bytes > 0 && !ws) return fail(SPAX_ERR_NULL, "workspace is NULL");
  if (ws_bytes < plan->ws_bytes)
    return fail(SPAX_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, plan->ws_bytes);
  return SPAX_OK;
}

// Every check of spax_decode_step_projections, before anything is enqueued.  noalloc: the
// workspace is not used (the batched form's tables go to the static scratch, whose size
// bounds the number of phases).
int validate_step(const spax_step* step, bool noalloc) {
  if (!step || !step->phases) return fail(SPAX_ERR_NULL, "step and step->phases are required");
  if (step->n_phases < 1) return fail(SPAX_ERR_SHAPE, "n_phases %d < 1", step->n_phases);
  if (step->flags & ~(SPAX_STEP_SEPARATE | SPAX_STEP_BATCHED | SPAX_STEP_DETERMINISTIC))
    return fail(SPAX_ERR_UNSUPPORTED, "unknown step flags 0x%x", step->flags);
  const bool batched = (step->flags & SPAX_STEP_BATCHED) != 0;
  const bool deterministic = (step->flags & SPAX_STEP_DETERMINISTIC) != 0;
  if (batched && (step->flags & SPAX_STEP_SEPARATE))
    return fail(SPAX_ERR_PARAM, "SPAX_STEP_BATCHED cannot be combined with SPAX_STEP_SEPARATE");
  if (deterministic && (batched || noalloc))
    return fail(SPAX_ERR_UNSUPPORTED, "SPAX_STEP_DETERMINISTIC is not available %s",
                batched ? "with SPAX_STEP_BATCHED" : "without a workspace");
  // The per-phase GEMV needs no workspace (checked against a size of 0 when none is used).
  const void* ws = noalloc ? nullptr : step->ws;
  const size_t ws_bytes = noalloc ? 0 : step->ws_bytes;
  for (int i = 0; i < step->n_phases; ++i) {
    const spax_phase& ph = step->phases[i];
    if (!ph.layout) return fail(SPAX_ERR_NULL, "phase %d: layout is NULL", i);
    int st = check_tier_outputs(ph.x, ph.layout->d_in, ph.full_idx, ph.approx_idx, ph.counts);
    if (st) return phase_fail(st, i);
    TierArgs a;
    st = tier_args_from_params(&ph.params, ph.layout->d_in, &a);
    if (st) return phase_fail(st, i);
    GemvPlan plan;
    st = check_gemv_args(ph.layout, ph.packed, ph.x, ph.full_idx, ph.approx_idx, ph.counts, ph.y,
                         ws, ws_bytes, &plan);
    if (st) return phase_fail(st, i);
    st = check_phase_aliasing(ph);
    if (st) return phase_fail(st, i);
  }
  if (deterministic) {
    const size_t need = deterministic_workspace_bytes(step->phases, step->n_phases);
    if (need > 0 && (!step->ws || step->ws_bytes < need))
      return fail(SPAX_ERR_WORKSPACE, "SPAX_STEP_DETERMINISTIC needs a workspace of %zu bytes",
                  need);
    for (int i = 0; i < step->n_phases; ++i)
      if (need > 0 && phase_touches(step->phases[i], step->ws, need))
        return fail(SPAX_ERR_PARAM, "the workspace overlaps a buffer of phase %d", i);
  }
  if (batched) {
    const size_t need = batched_workspace_bytes(step->n_phases);
    if (noalloc) {
      if (need > kStaticScratchBytes)
        return fail(SPAX_ERR_WORKSPACE, "SPAX_STEP_BATCHED over %d phases needs %zu bytes of "
                    "tables; the static scratch holds %zu", step->n_phases, need,
                    kStaticScratchBytes);
    } else if (!step->ws || step->ws_bytes < need) {
      return fail(SPAX_ERR_WORKSPACE, "SPAX_STEP_BATCHED needs a workspace of %zu bytes", need);
    }
    int st = check_independent(step, noalloc);
    if (st) return st;
  }
  return SPAX_OK;
}

}  // namespace

extern "C" {

namespace {
int check_pack_args(const spax_layout* L, const uint16_t* const* W, const void* packed) {
  if (!L || !W || !packed) return fail(SPAX_ERR_NULL, "layout, W and packed are required");
  if (!layout_ok(L)) return fail(SPAX_ERR_SHAPE, "layout not initialised by spax_layout_init");
  if (!aligned(packed, 256)) return fail(SPAX_ERR_ALIGN, "packed must be 256-byte aligned");
  for (int m = 0; m < L->n_mats; ++m) {
    if (!W[m]) return fail(SPAX_ERR_NULL, "W[%d] is NULL", m);
    if (!aligned(W[m], 16)) return fail(SPAX_ERR_ALIGN, "W[%d] must be 16-byte aligned", m);
  }
  return SPAX_OK;
}
}  // namespace

int spax_pack_columns(const spax_layout* L, const uint16_t* const* W, void* packed,
                      hipStream_t stream) {
  clear_error();
  int st = check_pack_args(L, W, packed);
  if (st) return st;
  return launch_pack(L, W, nullptr, packed, stream);
}

int spax_pack_columns_placed(const spax_layout* L, const uint16_t* const* W,
                             const int32_t* perm, void* packed, hipStream_t stream) {
  clear_error();
  int st = check_pack_args(L, W, packed);
  if (st) return st;
  if (!perm) return fail(SPAX_ERR_NULL, "perm is required");
  if (!aligned(perm, 4)) return fail(SPAX_ERR_ALIGN, "perm must be 4-byte aligned");
  return launch_pack(L, W, perm, packed, stream);
}

int spax_placement_order(const spax_layout* L, const uint8_t* tiers, int32_t n_tokens,
                         int32_t* order) {
  clear_error();
  if (!L || !order || (n_tokens > 0 && !tiers))
    return fail(SPAX_ERR_NULL, "layout, tiers and order are required");
  if (!layout_ok(L)) return fail(SPAX_ERR_SHAPE, "layout not initialised by spax_layout_init");
  if (n_tokens < 0) return fail(SPAX_ERR_PARAM, "n_tokens %d < 0", n_tokens);
  return no_throw([&] { return placement_order(L, tiers, n_tokens, order); });
}

int spax_build_tiers(const uint16_t* x, int32_t d_in, const spax_tier_params* p, uint8_t* tier,
                     int32_t* full_idx, int32_t* approx_idx, int32_t* counts, hipStream_t stream) {
  clear_error();
  int st = check_tier_outputs(x, d_in, full_idx, approx_idx, counts);
  if (st) return st;
  TierArgs a;
  st = tier_args_from_params(p, d_in, &a);
  if (st) return st;
  return launch_build_tiers(a, x, tier, full_idx, approx_idx, counts, nullptr, 0, stream);
}

size_t spax_gemv_workspace_bytes(const spax_layout* L) {
  if (!layout_ok(L)) return 0;
  return gemv_plan(L).ws_bytes;
}

int spax_tiered_gemv(const spax_layout* L, const void* packed, const uint16_t* x,
                     const int32_t* full_idx, const int32_t* approx_idx, const int32_t* counts,
                     float* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  clear_error();
  GemvPlan plan;
  int st = check_gemv_args(L, packed, x, full_idx, approx_idx, counts, y, ws, ws_bytes, &plan);
  if (st) return st;
  return launch_tiered_gemv(L, plan, packed, x, full_idx, approx_idx, counts, y, false, stream);
}

int spax_column_ranges(const int32_t* idx, int32_t n, int32_t gap, int32_t* first,
                       int32_t* count, int32_t* n_ranges) {
  clear_error();
  if (!n_ranges || (n > 0 && !idx)) return fail(SPAX_ERR_NULL, "idx and n_ranges are required");
  if (n < 0 || gap < 0) return fail(SPAX_ERR_PARAM, "n %d and gap %d must be >= 0", n, gap);
  const int32_t r = build_column_ranges(idx, n, gap, first, count);
  if (r < 0) return fail(SPAX_ERR_PARAM, "idx must be ascending, distinct and non-negative");
  *n_ranges = r;
  return SPAX_OK;
}

int spax_storage_ledger(const spax_layout* L, const int32_t* full_idx, int32_t n_full,
                        const int32_t* approx_idx, int32_t n_approx, int32_t gap,
                        int64_t block_bytes, spax_storage_stats* out) {
  clear_error();
  if (!L || !out || (n_full > 0 && !full_idx) || (n_approx > 0 && !approx_idx))
    return fail(SPAX_ERR_NULL, "layout, out and the non-empty lists are required");
  if (!layout_ok(L)) return fail(SPAX_ERR_SHAPE, "layout not initialised by spax_layout_init");
  if (n_full < 0 || n_approx < 0 || n_full > L->d_in || n_approx > L->d_in ||
      (int64_t)n_full + n_approx > L->d_in)
    return fail(SPAX_ERR_PARAM, "list lengths (%d, %d) out of range for d_in %d", n_full,
                n_approx, L->d_in);
  if (gap < 0 || block_bytes < 1)
    return fail(SPAX_ERR_PARAM, "gap %d must be >= 0 and block_bytes %lld >= 1", gap,
                (long long)block_bytes);
  for (int32_t i = 0; i < n_full; ++i)
    if (full_idx[i] >= L->d_in) return fail(SPAX_ERR_PARAM, "full_idx[%d] >= d_in", i);
  for (int32_t i = 0; i < n_approx; ++i)
    if (approx_idx[i] >= L->d_in) return fail(SPAX_ERR_PARAM, "approx_idx[%d] >= d_in", i);
  return storage_ledger(L, full_idx, n_full, approx_idx, n_approx, gap, block_bytes, out);
}

size_t spax_pinned_workspace_bytes(const spax_layout* L) {
  if (!L || !layout_ok(L)) return 0;
  return pinned_workspace_bytes(L);
}

int spax_tiered_gemv_pinned(const spax_layout* L, const void* packed_host, const uint16_t* x,
                            const int32_t* full_idx, const int32_t* approx_idx,
                            const int32_t* counts, float* y, int32_t gap, int32_t transfer,
                            void* ws, size_t ws_bytes, spax_move_stats* stats,
                            hipStream_t stream) {
  clear_error();
  GemvPlan plan;
  // the device-side arguments as for spax_tiered_gemv (packed_host stands in for packed)
  int st = check_gemv_args(L, packed_host, x, full_idx, approx_idx, counts, y, nullptr, 0, &plan);
  if (st) return st;
  if (gap < 0) return fail(SPAX_ERR_PARAM, "gap %d < 0", gap);
  if (transfer != SPAX_PINNED_MEMCPY && transfer != SPAX_PINNED_GATHER &&
      transfer != SPAX_PINNED_HOSTGATHER)
    return fail(SPAX_ERR_PARAM, "unknown transfer %d", transfer);
  if (!ws) return fail(SPAX_ERR_NULL, "ws is required");
  if (!aligned(ws, 256)) return fail(SPAX_ERR_ALIGN, "ws must be 256-byte aligned");
  if (ws_bytes < pinned_workspace_bytes(L))
    return fail(SPAX_ERR_WORKSPACE, "ws_bytes %zu < %zu", ws_bytes, pinned_workspace_bytes(L));
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, packed_host) != hipSuccess || attr.type != hipMemoryTypeHost ||
      !attr.devicePointer) {
    (void)hipGetLastError();
    return fail(SPAX_ERR_PARAM, "packed_host is not pinned host memory mapped for the device");
  }
  return no_throw([&] {
    return tiered_gemv_pinned(L, packed_host, attr.devicePointer, x, full_idx, approx_idx,
                              counts, y, gap, transfer, ws, stats, stream);
  });
}

size_t spax_step_workspace_bytes(const spax_phase* phases, int32_t n_phases) {
  if (!phases || n_phases < 1) return 0;
  size_t mx = batched_workspace_bytes(n_phases);
  for (int i = 0; i < n_phases; ++i) {
    if (!layout_ok(phases[i].layout)) return 0;
    const size_t b = gemv_plan(phases[i].layout).ws_bytes;
    if (b > mx) mx = b;
  }
  const size_t det = deterministic_workspace_bytes(phases, n_phases);
  return det > mx ? det : mx;
}

int spax_decode_step_projections(const spax_step* step, hipStream_t stream) {
  clear_error();
  return no_throw([&] {
    int st = validate_step(step, false);
    if (st) return st;
    return launch_decode_step(step, stream, false);
  });
}

int spax_decode_step_projections_noalloc(const spax_step* step, hipStream_t stream) {
  clear_error();
  return no_throw([&] {
    int st = validate_step(step, true);
    if (st) return st;
    return launch_decode_step(step, stream, true);
  });
}

}  // extern "C"
