// Pinned-host path: the packed blob stays in host memory; per call only the selected column
// records cross PCIe, as merged ranges, into a compacted staging area, and the tiered GEMV
// runs over the staged records.  Gather transfer: the ranges are merged on the device and one
// copy kernel reads them from the mapped blob (nothing waits for the host).  Memcpy transfer:
// the lists come back to the host, which merges them and issues one hipMemcpyAsync per range.
// Host-gather transfer: the host merges the ranges, a pool of host threads copies their
// records into one pinned staging buffer, and the buffer moves in DMA chunks as it fills.
//
// Pages: SpAx Abstract (weights offloaded to system memory; per token, read each column in
// full, as an approximation, or not at all); eigenradar commentary on SpAx, "The route outside
// GPU memory", third paragraph (jointly accessed columns placed together, adjacent read ranges
// merged, coarse granularity moving more than was selected) and last paragraph (count the bytes
// selected and the bytes moved apart).
#include <unistd.h>

#include <algorithm>
#include <condition_variable>
#include <cstring>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

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
  char* stage = nullptr;     // SPAX_PINNED_HOSTGATHER: the gathered records
  size_t stage_bytes = 0;
  hipEvent_t done = nullptr;
  bool pending = false;
};

// One host-side copy of a range's records into the staging buffer.
struct CopyJob {
  const uint8_t* src;
  int64_t dst_off;  // byte offset in the staging buffer; jobs follow each other without gaps
  int64_t bytes;
};

// A fixed pool of host threads for the host-gather transfer, started on first use (per
// process: a forked child starts its own) and never destroyed, so no thread is joined during
// static teardown.  run(fn) calls fn(i) once on each of the n threads and returns when all
// have returned; calls from several host threads take turns.
class GatherPool {
 public:
  explicit GatherPool(int n) : n_(n) {
    for (int i = 0; i < n; ++i) std::thread([this, i] { loop(i); }).detach();
  }
  int size() const { return n_; }
  void run(const std::function<void(int)>& fn) {
    std::lock_guard<std::mutex> turn(run_mu_);
    std::unique_lock<std::mutex> lk(mu_);
    fn_ = &fn;
    pending_ = n_;
    ++gen_;
    cv_.notify_all();
    done_.wait(lk, [&] { return pending_ == 0; });
    fn_ = nullptr;
  }

 private:
  void loop(int i) {
    uint64_t seen = 0;
    for (;;) {
      const std::function<void(int)>* fn;
      {
        std::unique_lock<std::mutex> lk(mu_);
        cv_.wait(lk, [&] { return gen_ != seen; });
        seen = gen_;
        fn = fn_;
      }
      (*fn)(i);
      std::lock_guard<std::mutex> lk(mu_);
      if (--pending_ == 0) done_.notify_one();
    }
  }
  const int n_;
  std::mutex run_mu_, mu_;
  std::condition_variable cv_, done_;
  const std::function<void(int)>* fn_ = nullptr;
  int pending_ = 0;
  uint64_t gen_ = 0;
};

GatherPool& gather_pool() {
  static std::mutex mu;
  static GatherPool* pool = nullptr;
  static pid_t owner = 0;
  std::lock_guard<std::mutex> lk(mu);
  if (!pool || owner != getpid()) {  // a forked child has none of the parent's threads
    const unsigned hw = std::thread::hardware_concurrency();
    pool = new GatherPool(hw == 0 ? 1 : (int)std::min(16u, hw));
    owner = getpid();
  }
  return *pool;
}

// Copies the bytes [b, e) of the staging buffer from the jobs' sources (the jobs tile
// [0, total) in order).
void gather_span(const std::vector<CopyJob>& jobs, int64_t b, int64_t e, uint8_t* dst) {
  // first job that ends after b
  size_t k = std::upper_bound(jobs.begin(), jobs.end(), b,
                              [](int64_t v, const CopyJob& j) { return v < j.dst_off + j.bytes; }) -
             jobs.begin();
  for (; k < jobs.size() && jobs[k].dst_off < e; ++k) {
    const int64_t lo = std::max(b, jobs[k].dst_off);
    const int64_t hi = std::min(e, jobs[k].dst_off + jobs[k].bytes);
    std::memcpy(dst + lo, jobs[k].src + (lo - jobs[k].dst_off), (size_t)(hi - lo));
  }
}

// Host gather + DMA: the staging bytes are filled chunk by chunk, each chunk split over the
// pool's threads, and each chunk's hipMemcpyAsync is issued as soon as it is filled, so the
// copy of one chunk overlaps the gathering of the next.
// (2, 4 and 16 MiB measured 151.7, 104.3 and 94.8 ms per host8b token against 91.3-92.6 for
// 8: each chunk wakes the pool once.)
constexpr int64_t kDmaChunk = (int64_t)8 << 20;
int gather_and_upload(const std::vector<CopyJob>& jobs, int64_t total, uint8_t* stage,
                      uint8_t* dst_dev, hipStream_t s) {
  GatherPool* pool = total >= ((int64_t)1 << 20) ? &gather_pool() : nullptr;
  for (int64_t b = 0; b < total; b += kDmaChunk) {
    const int64_t e = std::min(total, b + kDmaChunk);
    if (pool) {
      const int n = pool->size();
      pool->run([&](int i) { gather_span(jobs, b + (e - b) * i / n, b + (e - b) * (i + 1) / n, stage); });
    } else {
      gather_span(jobs, b, e, stage);
    }
    SPAX_HIP_CHECK(hipMemcpyAsync(dst_dev + b, stage + b, (size_t)(e - b), hipMemcpyHostToDevice, s));
  }
  return SPAX_OK;
}
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
  // SPAX_PINNED_MEMCPY: the ranges are merged on the host, one hipMemcpyAsync each.
  // SPAX_PINNED_HOSTGATHER: the ranges are merged on the host, host threads copy their records
  // into one pinned staging buffer (FULL records, then APPROX records), which moves in DMA
  // chunks as it fills; region A of the staged records then starts right after the FULL
  // records.
  const bool host_gather = transfer == SPAX_PINNED_HOSTGATHER;
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
  std::vector<CopyJob> jobs;
  // stage_off: where the region's first slot lands in the staging area
  const auto region = [&](const int32_t* idx, int n, uint32_t* out, int64_t off, int64_t stride,
                          int64_t stage_off) {
    int32_t slot = 0;
    const int r = for_ranges(idx, n, gap, [&](int32_t f, int32_t c, int32_t e0, int32_t ne) {
      if (rc) return;
      for (int32_t k = 0; k < ne; ++k)
        out[e0 + k] = (uint32_t)(slot + (idx[e0 + k] - f)) | ((uint32_t)idx[e0 + k] << 16);
      const uint8_t* src = host + off + (int64_t)f * stride;
      if (host_gather) {
        jobs.push_back(CopyJob{src, stage_off + (int64_t)slot * stride, (int64_t)c * stride});
      } else {
        const hipError_t e = hipMemcpyAsync(staging + stage_off + (int64_t)slot * stride, src,
                                            (size_t)c * stride, hipMemcpyHostToDevice, s);
        if (e != hipSuccess) rc = hip_fail(e, "hipMemcpyAsync of a record range");
      }
      moved += (int64_t)c * stride;
      slot += c;
    });
    if (r < 0 && !rc) rc = fail(SPAX_ERR_PARAM, "column list read back is not ascending");
    if (r > 0) n_ranges += r;
  };
  region(h_full, nF, h_outF, 0, L->stride_F, 0);
  if (rc) return rc;
  const int64_t movedF = moved;  // host gather: the APPROX records follow the FULL ones
  region(h_apx, nA, h_outA, L->off_A, L->stride_A, host_gather ? movedF : L->off_A);
  if (rc) return rc;
  spax_layout staged = *L;
  if (host_gather) {
    if (sc.stage_bytes < (size_t)moved) {
      if (sc.stage) SPAX_HIP_CHECK(hipHostFree(sc.stage));
      sc.stage = nullptr;
      sc.stage_bytes = 0;
      void* h = nullptr;
      SPAX_HIP_CHECK(hipHostMalloc(&h, (size_t)moved, hipHostMallocDefault));
      sc.stage = static_cast<char*>(h);
      sc.stage_bytes = (size_t)moved;
    }
    rc = gather_and_upload(jobs, moved, reinterpret_cast<uint8_t*>(sc.stage), staging, s);
    if (rc) return rc;
    staged.off_A = movedF;  // the GEMV reads region A of the staged records here
  }
  // The two host lists and their device copies have the same layout (d entries each), so one
  // upload of the span that holds the used entries replaces two (an upload costs more to
  // enqueue than to move).
  const PinnedTables t = pinned_tables(L, ws);
  const size_t words = nA ? (size_t)d + (size_t)nA : (size_t)nF;
  if (words) SPAX_HIP_CHECK(hipMemcpyAsync(t.listF, h_outF, 4 * words, hipMemcpyHostToDevice, s));
  SPAX_HIP_CHECK(hipEventRecord(sc.done, s));
  sc.pending = true;

  // ---- the GEMV over the staged records (counts are still the device's)
  rc = launch_tiered_gemv(&staged, gemv_plan(L), staging, x,
                          reinterpret_cast<const int32_t*>(t.listF),
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

// Byte ledger of one mask at a storage granularity (host only): each merged range of a region
// is one read request, rounded out to whole blocks of the blob (which starts on a block
// boundary).
int storage_ledger(const spax_layout* L, const int32_t* full_idx, int32_t n_full,
                   const int32_t* approx_idx, int32_t n_approx, int32_t gap, int64_t block,
                   spax_storage_stats* out) {
  spax_storage_stats st{};
  const struct {
    const int32_t* idx;
    int32_t n;
    int64_t stride, off;
  } regions[2] = {{full_idx, n_full, L->stride_F, 0}, {approx_idx, n_approx, L->stride_A, L->off_A}};
  for (const auto& r : regions) {
    const int nr = for_ranges(r.idx, r.n, gap, [&](int32_t f, int32_t c, int32_t, int32_t) {
      const int64_t begin = r.off + (int64_t)f * r.stride, end = begin + (int64_t)c * r.stride;
      st.moved_bytes += (int64_t)c * r.stride;
      st.n_blocks += (end + block - 1) / block - begin / block;
    });
    if (nr < 0) return fail(SPAX_ERR_PARAM, "lists must be ascending, distinct and non-negative");
    st.n_ranges += nr;
    st.selected_bytes += (int64_t)r.n * r.stride;
  }
  st.read_bytes = st.n_blocks * block;
  *out = st;
  return SPAX_OK;
}

// Channels by descending bytes selected over the calibration masks (stride_F per FULL,
// stride_A per APPROX), equal scores by channel index.
int placement_order(const spax_layout* L, const uint8_t* tiers, int32_t n_tokens,
                    int32_t* order) {
  const int d = L->d_in;
  std::vector<int64_t> score(d, 0);
  for (int32_t t = 0; t < n_tokens; ++t) {
    const uint8_t* row = tiers + (size_t)t * d;
    for (int j = 0; j < d; ++j) {
      if (row[j] > SPAX_TIER_FULL)
        return fail(SPAX_ERR_PARAM, "tiers[%d][%d] = %d is not a tier", t, j, (int)row[j]);
      score[j] += row[j] == SPAX_TIER_FULL ? L->stride_F : row[j] == SPAX_TIER_APPROX ? L->stride_A : 0;
    }
  }
  for (int j = 0; j < d; ++j) order[j] = j;
  std::stable_sort(order, order + d, [&](int32_t a, int32_t b) { return score[a] > score[b]; });
  return SPAX_OK;
}

size_t pinned_workspace_bytes(const spax_layout* L) {
  return aligned_size((size_t)L->total_bytes) + 16 * (size_t)L->d_in + 4 * kTotals;
}

}  // namespace spax
