// Pinned-host path: the packed blob stays in host memory; per call only the selected column
// records cross PCIe, as merged ranges copied with hipMemcpyAsync into a compacted staging
// area, and the tiered GEMV runs over the staged records.
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

int tiered_gemv_pinned(const spax_layout* L, const void* packed_host, const void* host_dev,
                       const uint16_t* x, const int32_t* full_idx, const int32_t* approx_idx,
                       const int32_t* counts, float* y, int32_t gap, int32_t transfer, void* ws,
                       spax_move_stats* stats, hipStream_t s) {
  const int d = L->d_in;
  int dev = 0;
  SPAX_HIP_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) return fail(SPAX_ERR_UNSUPPORTED, "device index %d", dev);
  Scratch& sc = g_scratch[dev];
  std::lock_guard<std::mutex> lock(sc.mu);
  const size_t need = 16 + 24 * (size_t)d;  // counts, two lists in, two lists out, 2 tables
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
  int32_t* h_colF = reinterpret_cast<int32_t*>(h_outA + d);  // staging slot -> column
  int32_t* h_colA = h_colF + d;
  const bool gather = transfer == SPAX_PINNED_GATHER;

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
  const auto region = [&](const int32_t* idx, int n, uint32_t* out, int32_t* col, int64_t off,
                          int64_t stride) {
    int32_t slot = 0;
    const int r = for_ranges(idx, n, gap, [&](int32_t f, int32_t c, int32_t e0, int32_t ne) {
      if (rc) return;
      for (int32_t k = 0; k < ne; ++k)
        out[e0 + k] = (uint32_t)(slot + (idx[e0 + k] - f)) | ((uint32_t)idx[e0 + k] << 16);
      if (gather) {
        for (int32_t k = 0; k < c; ++k) col[slot + k] = f + k;
      } else {
        const hipError_t e = hipMemcpyAsync(staging + off + (int64_t)slot * stride,
                                            host + off + (int64_t)f * stride, (size_t)c * stride,
                                            hipMemcpyHostToDevice, s);
        if (e != hipSuccess) rc = hip_fail(e, "hipMemcpyAsync of a record range");
      }
      moved += (int64_t)c * stride;
      slot += c;
    });
    if (r < 0 && !rc) rc = fail(SPAX_ERR_PARAM, "column list read back is not ascending");
    if (r > 0) n_ranges += r;
    return slot;
  };
  const int32_t slotsF = region(h_full, nF, h_outF, h_colF, 0, L->stride_F);
  if (rc) return rc;
  const int32_t slotsA = region(h_apx, nA, h_outA, h_colA, L->off_A, L->stride_A);
  if (rc) return rc;
  uint32_t* d_listF = reinterpret_cast<uint32_t*>(staging + aligned_size((size_t)L->total_bytes));
  uint32_t* d_listA = d_listF + d;
  int32_t* d_colF = reinterpret_cast<int32_t*>(d_listA + d);
  int32_t* d_colA = d_colF + d;
  // The host tables and their device copies have the same layout (four arrays of d entries:
  // FULL list, APPROX list, FULL slot columns, APPROX slot columns), so one upload of the span
  // that holds the used entries replaces four (each upload costs more to enqueue than to move).
  size_t words = 0;
  if (nF) words = (size_t)nF;
  if (nA) words = (size_t)d + (size_t)nA;
  if (gather && slotsF) words = 2 * (size_t)d + (size_t)slotsF;
  if (gather && slotsA) words = 3 * (size_t)d + (size_t)slotsA;
  if (words) SPAX_HIP_CHECK(hipMemcpyAsync(d_listF, h_outF, 4 * words, hipMemcpyHostToDevice, s));
  SPAX_HIP_CHECK(hipEventRecord(sc.done, s));
  sc.pending = true;
  if (gather) {
    rc = launch_gather_records(L, host_dev, staging, d_colF, slotsF, d_colA, slotsA, s);
    if (rc) return rc;
  }

  // ---- the GEMV over the staged records (counts are still the device's)
  rc = launch_tiered_gemv(L, gemv_plan(L), staging, x, reinterpret_cast<const int32_t*>(d_listF),
                          reinterpret_cast<const int32_t*>(d_listA), counts, y, false, s, true);
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
  return aligned_size((size_t)L->total_bytes) + 16 * (size_t)L->d_in;
}

}  // namespace spax
