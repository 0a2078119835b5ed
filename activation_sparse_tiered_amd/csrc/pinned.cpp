// Pinned-host path: the packed blob stays in host memory; per call only the selected column
// records cross PCIe, as merged ranges, into a compacted staging area, and the tiered GEMV
// runs over the staged records.  Gather transfer: the ranges are merged on the device and one
// copy kernel reads them from the mapped blob (nothing waits for the host).  Memcpy transfer:
// the lists come back to the host, which merges them and issues one hipMemcpyAsync per range.
//
// Pages: SpAx Abstract (weights offloaded to system memory; per token, read each column in
// full, as an approximation, or not at all); eigenradar commentary on SpAx, "The route outside
// GPU memory", third paragraph (jointly accessed columns placed together, adjacent read ranges
// merged, coarse granularity moving more than was selected) and last paragraph (count the bytes
// selected and the bytes moved apart).
#include <cstring>
#include <mutex>

#include "common.h"

namespace spax {
namespace {

// Runs of consecutive channels, merged across gaps of at most `gap` channels.  idx ascending,
// distinct, non-negative (checked).  Calls on(first, count, index_of_first_entry, n_entries)
// per range; returns the number of ranges or -1 if idx is not ascending.
template <class F>
int for_ranges(const int32_t* idx, int32_t n, int32_t gap, F on) {
  int n_ranges = 0;
  int32_t first = 0, last = 0, e0 = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t j = idx[i];
    if (j < 0 || (i > 0 && j <= idx[i - 1])) return -1;
    if (i > 0 && (int64_t)j - last - 1 <= gap) {
      last = j;
      continue;
    }
    if (i > 0) {
      on(first, last - first + 1, e0, i - e0);
      ++n_ranges;
    }
    first = last = j;
    e0 = i;
  }
  if (n > 0) {
    on(first, last - first + 1, e0, n - e0);
    ++n_ranges;
  }
  return n_ranges;
}

// Library-owned pinned host scratch per device: the lists read back and the compacted lists
// sent out.  `done` marks when the last outgoing copy from it has completed.
struct Scratch {
  std::mutex mu;
  char* host = nullptr;
  size_t bytes = 0;
  hipEvent_t done = nullptr;
  bool pending = false;
};
Scratch g_scratch[64];

}  // namespace

int32_t build_column_ranges(const int32_t* idx, int32_t n, int32_t gap, int32_t* first,
                            int32_t* count) {
  return for_ranges(idx, n, gap, [&](int32_t f, int32_t c, int32_t, int32_t) {
    if (first) *first++ = f;
    if (count) *count++ = c;
  });
}

namespace {

// Workspace layout after the staging copy of the blob: FULL entries, APPROX entries, FULL slot
// table, APPROX slot table (d int32 each), then the device-merge totals.
struct PinnedTables {
  uint32_t *listF, *listA;
  int32_t *colF, *colA, *totals;
};
PinnedTables pinned_tables(const spax_layout* L, void* ws) {
  const int d = L->d_in;
  PinnedTables t;
  t.listF = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + aligned_size((size_t)L->total_bytes));
  t.listA = t.listF + d;
  t.colF = reinterpret_cast<int32_t*>(t.listA + d);
  t.colA = t.colF + d;
  t.totals = t.colA + d;
  return t;
}
constexpr int kTotals = 6;

// Gather transfer with the ranges merged on the device: nothing waits for the host unless
// the byte account is asked for.
int tiered_gemv_pinned_device_merge(const spax_layout* L, const void* host_dev,
                                    const uint16_t* x, const int32_t* full_idx,
                                    const int32_t* approx_idx, const int32_t* counts, float* y,
                                    int32_t gap, void* ws, spax_move_stats* stats,
                                    hipStream_t s) {
  const PinnedTables t = pinned_tables(L, ws);
  int rc = launch_merge_and_gather(L, host_dev, ws, full_idx, approx_idx, counts, gap, t.listF,
                                   t.listA, t.colF, t.colA, t.totals, s);
  if (rc) return rc;
  rc = launch_tiered_gemv(L, gemv_plan(L), ws, x, reinterpret_cast<const int32_t*>(t.listF),
                          reinterpret_cast<const int32_t*>(t.listA), counts, y, false, s, true);
  if (rc) return rc;
  if (stats) {
    int32_t h[kTotals];
    SPAX_HIP_CHECK(hipMemcpyAsync(h, t.totals, sizeof(h), hipMemcpyDeviceToHost, s));
    SPAX_HIP_CHECK(hipStreamSynchronize(s));
    stats->selected_bytes = (int64_t)h[4] * L->stride_F + (int64_t)h[5] * L->stride_A;
    stats->moved_bytes = (int64_t)h[0] * L->stride_F + (int64_t)h[1] * L->stride_A;
    stats->list_bytes = 0;
    stats->n_ranges = h[2] + h[3];
    stats->n_full = h[4];
    stats->n_approx = h[5];
    stats->reserved0 = 0;
  }
  return SPAX_OK;
}

}  // namespace

int tiered_gemv_pinned(const spax_layout* L, const void* packed_host, const void* host_dev,
                       const uint16_t* x, const int32_t* full_idx, const int32_t* approx_idx,
                       const int32_t* counts, float* y, int32_t gap, int32_t transfer, void* ws,
                       spax_move_stats* stats, hipStream_t s) {
  if (transfer == SPAX_PINNED_GATHER)
    return tiered_gemv_pinned_device_merge(L, host_dev, x, full_idx, approx_idx, counts, y, gap,
                                           ws, stats, s);
  // SPAX_PINNED_MEMCPY: the ranges are merged on the host, one hipMemcpyAsync each
  const int d = L->d_in;
  int dev = 0;
  SPAX_HIP_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) return fail(SPAX_ERR_UNSUPPORTED, "device index %d", dev);
  Scratch& sc = g_scratch[dev];
  std::lock_guard<std::mutex> lock(sc.mu);
  const size_t need = 16 + 16 * (size_t)d;  // counts, two lists in, two compacted lists out
  if (sc.pending) {
    SPAX_HIP_CHECK(hipEventSynchronize(sc.done));
    sc.pending = false;
  }
  if (sc.bytes < need) {
    if (sc.host) SPAX_HIP_CHECK(hipHostFree(sc.host));
    sc.host = nullptr;
    sc.bytes = 0;
    void* h = nullptr;
    SPAX_HIP_CHECK(hipHostMalloc(&h, need, hipHostMallocDefault));
    sc.host = static_cast<char*>(h);
    sc.bytes = need;
  }
  if (!sc.done) SPAX_HIP_CHECK(hipEventCreateWithFlags(&sc.done, hipEventDisableTiming));
  int32_t* h_counts = reinterpret_cast<int32_t*>(sc.host);
  int32_t* h_full = h_counts + 4;
  int32_t* h_apx = h_full + d;
  uint32_t* h_outF = reinterpret_cast<uint32_t*>(h_apx + d);
  uint32_t* h_outA = h_outF + d;

  // ---- the mask, back on the host
  SPAX_HIP_CHECK(hipMemcpyAsync(h_counts, counts, 12, hipMemcpyDeviceToHost, s));
  SPAX_HIP_CHECK(hipMemcpyAsync(h_full, full_idx, 4 * (size_t)d, hipMemcpyDeviceToHost, s));
  SPAX_HIP_CHECK(hipMemcpyAsync(h_apx, approx_idx, 4 * (size_t)d, hipMemcpyDeviceToHost, s));
  SPAX_HIP_CHECK(hipStreamSynchronize(s));
  const int nF = h_counts[0] < 0 ? 0 : (h_counts[0] > d ? d : h_counts[0]);
  const int nA = h_counts[1] < 0 ? 0 : (h_counts[1] > d ? d : h_counts[1]);

  // ---- ranges -> record copies into the compacted staging area; compacted lists
  uint8_t* staging = static_cast<uint8_t*>(ws);
  const uint8_t* host = static_cast<const uint8_t*>(packed_host);
  int64_t moved = 0;
  int n_ranges = 0;
  int rc = SPAX_OK;
  const auto region = [&](const int32_t* idx, int n, uint32_t* out, int64_t off, int64_t stride) {
    int32_t slot = 0;
    const int r = for_ranges(idx, n, gap, [&](int32_t f, int32_t c, int32_t e0, int32_t ne) {
      if (rc) return;
      for (int32_t k = 0; k < ne; ++k)
        out[e0 + k] = (uint32_t)(slot + (idx[e0 + k] - f)) | ((uint32_t)idx[e0 + k] << 16);
      const hipError_t e = hipMemcpyAsync(staging + off + (int64_t)slot * stride,
                                          host + off + (int64_t)f * stride, (size_t)c * stride,
                                          hipMemcpyHostToDevice, s);
      if (e != hipSuccess) rc = hip_fail(e, "hipMemcpyAsync of a record range");
      moved += (int64_t)c * stride;
      slot += c;
    });
    if (r < 0 && !rc) rc = fail(SPAX_ERR_PARAM, "column list read back is not ascending");
    if (r > 0) n_ranges += r;
  };
  region(h_full, nF, h_outF, 0, L->stride_F);
  if (rc) return rc;
  region(h_apx, nA, h_outA, L->off_A, L->stride_A);
  if (rc) return rc;
  // The two host lists and their device copies have the same layout (d entries each), so one
  // upload of the span that holds the used entries replaces two (an upload costs more to
  // enqueue than to move).
  const PinnedTables t = pinned_tables(L, ws);
  const size_t words = nA ? (size_t)d + (size_t)nA : (size_t)nF;
  if (words) SPAX_HIP_CHECK(hipMemcpyAsync(t.listF, h_outF, 4 * words, hipMemcpyHostToDevice, s));
  SPAX_HIP_CHECK(hipEventRecord(sc.done, s));
  sc.pending = true;

  // ---- the GEMV over the staged records (counts are still the device's)
  rc = launch_tiered_gemv(L, gemv_plan(L), staging, x, reinterpret_cast<const int32_t*>(t.listF),
                          reinterpret_cast<const int32_t*>(t.listA), counts, y, false, s, true);
  if (rc) return rc;
  if (stats) {
    stats->selected_bytes = (int64_t)nF * L->stride_F + (int64_t)nA * L->stride_A;
    stats->moved_bytes = moved;
    stats->list_bytes = 4 * (int64_t)words;
    stats->n_ranges = n_ranges;
    stats->n_full = nF;
    stats->n_approx = nA;
    stats->reserved0 = 0;
  }
  return SPAX_OK;
}

size_t pinned_workspace_bytes(const spax_layout* L) {
  return aligned_size((size_t)L->total_bytes) + 16 * (size_t)L->d_in + 4 * kTotals;
}

}  // namespace spax
