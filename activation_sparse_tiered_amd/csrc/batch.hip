// Batched decode step (SPAX_STEP_BATCHED): every phase's mask in one launch, then every
// phase's tiered GEMV in one persistent launch.
//
// Pages: eigenradar commentary on SpAx, second and last paragraphs (per-token selection at
// batch one); ByteCross abstract (fixed kernel costs on top of the byte account).  Legal only
// when all activation vectors are ready when the step is enqueued and no phase reads another
// phase's output; the layer-serial forms make no such assumption.  It removes the per-phase
// launch and ramp cost, so it shows what the byte account alone allows.
//
// Launch 1: one 1024-thread workgroup per phase runs the stand-alone mask (mask_core.h,
// tiers_to_global) and clears the phase's y.  Then, per base format present (fp16, int4), one
// persistent grid walks the work items of that format's phases, (row tile, column chunk)
// pairs numbered phase after phase, each handled like one workgroup of the stand-alone GEMV
// (gemv_core.h, gemv_item; an int4 tile is 2048 rows, 32 per lane).  The per-phase arguments
// reach the device as two descriptor tables copied into the caller's workspace from a
// library-owned ring of pinned host buffers.
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "gemv_core.h"
#include "mask_core.h"

namespace spax {
namespace {

constexpr int kMaskThreads = 1024;
constexpr int kRingSlots = 4;

struct MaskDesc {
  TierArgs ta;
  const uint16_t* x;
  uint8_t* tier;
  int32_t* full_idx;
  int32_t* approx_idx;
  int32_t* counts;
  float4* y;
  int32_t n_zero4;
  int32_t pad;
};

struct GemvDesc {
  gemv::Shape sh;
  const uint8_t* packed;
  const uint32_t* x32;
  const int32_t* full_idx;
  const int32_t* approx_idx;
  const int32_t* counts;
  float* y;
  int32_t item0;  // first work item of this phase
  int32_t fmt;
};

__global__ __launch_bounds__(kMaskThreads) void batched_mask_kernel(const MaskDesc* __restrict__ md) {
  __shared__ mask::KeyHist<kMaskThreads> sh;
  __shared__ uint32_t xs32[SPAX_MAX_DIN / 2];
  const MaskDesc& m = md[blockIdx.x];
  mask::tiers_to_global<kMaskThreads, SPAX_MAX_DIN>(sh, xs32, m.ta, m.x, m.tier, m.full_idx,
                                                    m.approx_idx, m.counts);
  for (int i = threadIdx.x; i < m.n_zero4; i += kMaskThreads)
    m.y[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// Work item -> phase by binary search over the phases' first items (wave-uniform).
__device__ __forceinline__ int phase_of(const GemvDesc* __restrict__ gd, int n, int item) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (gemv::uniform(gd[mid].item0) <= item) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// The descriptor in scalar registers (see gemv::uniform): loop bounds and addresses derived
// from it are then uniform, and the loop's branches are scalar branches.
__device__ __forceinline__ GemvDesc uniform_desc(const GemvDesc& g) {
  using gemv::uniform;
  GemvDesc u;
  u.sh.stride_F = uniform(g.sh.stride_F);
  u.sh.stride_A = uniform(g.sh.stride_A);
  u.sh.off_A = uniform(g.sh.off_A);
  u.sh.T = uniform(g.sh.T);
  u.sh.n_tiles = uniform(g.sh.n_tiles);
  u.sh.n_chunks = uniform(g.sh.n_chunks);
  u.sh.approx_group = uniform(g.sh.approx_group);
  u.sh.base_group = uniform(g.sh.base_group);
  u.sh.d_in = uniform(g.sh.d_in);
  u.packed = uniform(g.packed);
  u.x32 = uniform(g.x32);
  u.full_idx = uniform(g.full_idx);
  u.approx_idx = uniform(g.approx_idx);
  u.counts = uniform(g.counts);
  u.y = uniform(g.y);
  u.item0 = uniform(g.item0);
  u.fmt = uniform(g.fmt);
  return u;
}

// The work items of the phases whose base format is FMT (one launch per format present, so
// each format gets its own register and LDS budget).
template <int FMT, class Blob>
__global__ __launch_bounds__(kGemvThreads) void batched_gemv_kernel(const GemvDesc* __restrict__ gd,
                                                                    int n_phases, int n_items) {
  __shared__ float red[gemv::kWaves * gemv::ItemRows<FMT>::tile];
  // Item i runs on XCD i % 8 (the grid is a multiple of 8 or holds one item per
  // workgroup), so the XCD-aware order applies to the item index.  Only the speed depends on
  // this: the order is a bijection whatever the grid.
  for (int i = blockIdx.x; i < n_items; i += gridDim.x) {
    const int item = gemv::xcd_order(i, n_items);
    const int p = phase_of(gd, n_phases, item);
    const GemvDesc g = uniform_desc(gd[p]);
    const int local = item - g.item0;
    const int tile = (int)((uint32_t)local % (uint32_t)g.sh.n_tiles);
    const int chunk = (int)((uint32_t)local / (uint32_t)g.sh.n_tiles);
    gemv::gemv_item<FMT, Blob, false, gemv::ItemRows<FMT>::rpl, gemv::ItemRows<FMT>::unroll>(
        g.sh, g.packed, g.x32, g.full_idx, g.approx_idx, g.counts, g.y, tile, chunk, red);
    __syncthreads();  // red is reused by the next item
  }
}

// Column chunks of a batched phase: about 2048 input channels each, so a work item streams
// hundreds of columns and its fixed cost (lists, reduction, atomics) stays small.  For int4
// layouts (2048-row tiles) 512 to 6144 channels were measured; 2048 was the fastest.
GemvPlan batched_plan(const spax_layout* L) {
  constexpr int channels = 2048;
  GemvPlan p{};
  const int rows = batched_tile_rows(L);
  p.n_tiles = (int32_t)((L->d_out_total + rows - 1) / rows);
  int k = (L->d_in + channels - 1) / channels;
  const int kmax = L->d_in / 16 > 1 ? L->d_in / 16 : 1;
  p.n_chunks = k < 1 ? 1 : (k > kmax ? kmax : k);
  p.ws_bytes = 0;
  return p;
}

size_t table_bytes(int n) {
  return aligned_size((size_t)n * sizeof(MaskDesc)) + (size_t)n * sizeof(GemvDesc);
}

// Library-owned pinned staging: kRingSlots slots per device, each reused only after the copy
// that last read it has completed.
struct Ring {
  std::mutex mu;
  char* host = nullptr;
  size_t slot_bytes = 0;
  hipEvent_t ev[kRingSlots] = {};
  bool pending[kRingSlots] = {};
  int next = 0;
};
Ring g_rings[64];

int stage_and_copy(const void* src, size_t bytes, void* dst, hipStream_t s) {
  int dev = 0;
  SPAX_HIP_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) return fail(SPAX_ERR_UNSUPPORTED, "device index %d", dev);
  Ring& r = g_rings[dev];
  std::lock_guard<std::mutex> lock(r.mu);
  if (r.slot_bytes < bytes) {
    for (int i = 0; i < kRingSlots; ++i)
      if (r.pending[i]) {
        SPAX_HIP_CHECK(hipEventSynchronize(r.ev[i]));
        r.pending[i] = false;
      }
    if (r.host) SPAX_HIP_CHECK(hipHostFree(r.host));
    r.host = nullptr;
    r.slot_bytes = 0;
    const size_t sb = (bytes + 4095) / 4096 * 4096;
    void* h = nullptr;
    SPAX_HIP_CHECK(hipHostMalloc(&h, sb * kRingSlots, hipHostMallocDefault));
    r.host = static_cast<char*>(h);
    r.slot_bytes = sb;
  }
  const int k = r.next;
  if (!r.ev[k]) SPAX_HIP_CHECK(hipEventCreateWithFlags(&r.ev[k], hipEventDisableTiming));
  if (r.pending[k]) SPAX_HIP_CHECK(hipEventSynchronize(r.ev[k]));
  char* slot = r.host + (size_t)k * r.slot_bytes;
  std::memcpy(slot, src, bytes);
  SPAX_HIP_CHECK(hipMemcpyAsync(dst, slot, bytes, hipMemcpyHostToDevice, s));
  SPAX_HIP_CHECK(hipEventRecord(r.ev[k], s));
  r.pending[k] = true;
  r.next = (k + 1) % kRingSlots;
  return SPAX_OK;
}

// Work items of a batched step's GEMV launches: the fp16 phases' and the int4 phases'.
struct BatchItems {
  int32_t n_phases[2];  // phases per base format (their descriptors: fp16 first, then int4)
  int64_t items[2];     // work items per base format
  bool narrow[2];       // every blob of that format has both regions below 2 GiB
};

// The descriptor tables of a batched step, written into `table` (table_bytes(n) bytes): the
// mask descriptors in phase order, then the GEMV descriptors grouped by base format (fp16
// phases first), each group numbering its work items from 0.  Returns false (error set) if
// there are too many work items.
bool build_tables(const spax_step* st, char* table, BatchItems* bi) {
  const int n = st->n_phases;
  MaskDesc* md = reinterpret_cast<MaskDesc*>(table);
  GemvDesc* gd = reinterpret_cast<GemvDesc*>(table + aligned_size((size_t)n * sizeof(MaskDesc)));
  *bi = BatchItems{};
  bi->narrow[0] = bi->narrow[1] = true;
  for (int i = 0; i < n; ++i) {
    const spax_layout* L = st->phases[i].layout;
    const int f = L->base_fmt == SPAX_FMT_INT4;
    bi->n_phases[f]++;
    bi->narrow[f] = bi->narrow[f] && narrow_regions(L);
  }
  int slot[2] = {0, bi->n_phases[0]};
  for (int i = 0; i < n; ++i) {
    const spax_phase& ph = st->phases[i];
    const spax_layout* L = ph.layout;
    MaskDesc m{};
    tier_args_from_params(&ph.params, L->d_in, &m.ta);
    m.x = ph.x;
    m.tier = ph.tier;
    m.full_idx = ph.full_idx;
    m.approx_idx = ph.approx_idx;
    m.counts = ph.counts;
    m.y = reinterpret_cast<float4*>(ph.y);
    m.n_zero4 = (int32_t)((L->d_out_total + 3) / 4);
    md[i] = m;
    const int f = L->base_fmt == SPAX_FMT_INT4;
    const GemvPlan plan = batched_plan(L);
    GemvDesc g{};
    g.sh = gemv_shape(L, plan);
    g.packed = static_cast<const uint8_t*>(ph.packed);
    g.x32 = reinterpret_cast<const uint32_t*>(ph.x);
    g.full_idx = ph.full_idx;
    g.approx_idx = ph.approx_idx;
    g.counts = ph.counts;
    g.y = ph.y;
    g.item0 = (int32_t)bi->items[f];
    g.fmt = L->base_fmt;
    gd[slot[f]++] = g;
    bi->items[f] += (int64_t)plan.n_tiles * plan.n_chunks;
    if (bi->items[f] > INT32_MAX) {
      fail(SPAX_ERR_SHAPE, "too many work items (%lld)", (long long)bi->items[f]);
      return false;
    }
  }
  return true;
}

template <int FMT, class Blob>
int launch_gemvs(const GemvDesc* dgd, int n_phases, int64_t items, int n_cu, hipStream_t s) {
  // as many workgroups as can be resident at once
  static const int per_cu = [] {
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, batched_gemv_kernel<FMT, Blob>,
                                                     kGemvThreads, 0) != hipSuccess || occ < 1)
      occ = 2;
    return occ;
  }();
  const int64_t cap = (int64_t)n_cu * per_cu;
  const int64_t grid = items < cap ? items : cap;
  if (grid > 0) {
    hipLaunchKernelGGL((batched_gemv_kernel<FMT, Blob>), dim3((unsigned)grid), dim3(kGemvThreads),
                       0, s, dgd, n_phases, (int)items);
    SPAX_HIP_CHECK(hipGetLastError());
  }
  return SPAX_OK;
}

// The launches over tables already on the device (in stream order): all masks, then the
// GEMVs of the fp16 phases and of the int4 phases.
int launch_from_tables(const spax_step* st, int n_cu, const void* dtables, const BatchItems& bi,
                       hipStream_t s) {
  const int n = st->n_phases;
  const auto* dmd = static_cast<const MaskDesc*>(dtables);
  const auto* dgd = reinterpret_cast<const GemvDesc*>(static_cast<const char*>(dtables) +
                                                      aligned_size((size_t)n * sizeof(MaskDesc)));
  // events (optional): [0, 1] bracket the mask launch and [2, 3] the GEMV launches; with one
  // phase, [0, 1] bracket both.
  const bool four = st->events && n >= 2;
  if (st->events) SPAX_HIP_CHECK(hipEventRecord(st->events[0], s));
  hipLaunchKernelGGL(batched_mask_kernel, dim3((unsigned)n), dim3(kMaskThreads), 0, s, dmd);
  SPAX_HIP_CHECK(hipGetLastError());
  if (four) {
    SPAX_HIP_CHECK(hipEventRecord(st->events[1], s));
    SPAX_HIP_CHECK(hipEventRecord(st->events[2], s));
  }
  const GemvDesc* dgd4 = dgd + bi.n_phases[0];
  const int n16 = bi.n_phases[0], n4 = bi.n_phases[1];
  int rc = bi.narrow[0]
               ? launch_gemvs<SPAX_FMT_FP16, gemv::RegionBlob>(dgd, n16, bi.items[0], n_cu, s)
               : launch_gemvs<SPAX_FMT_FP16, gemv::RecordBlob>(dgd, n16, bi.items[0], n_cu, s);
  if (rc) return rc;
  rc = bi.narrow[1]
           ? launch_gemvs<SPAX_FMT_INT4, gemv::RegionBlob>(dgd4, n4, bi.items[1], n_cu, s)
           : launch_gemvs<SPAX_FMT_INT4, gemv::RecordBlob>(dgd4, n4, bi.items[1], n_cu, s);
  if (rc) return rc;
  if (st->events) SPAX_HIP_CHECK(hipEventRecord(st->events[four ? 3 : 1], s));
  return SPAX_OK;
}

// ---- the entry point that allocates nothing: descriptor tables in a file-scope device array
//
// Each device holds its own copy of `scratch`; host code reaches it only through the address
// hipGetSymbolAddress returns for the current device (the array's name in host code is a
// host-side stand-in, not a device address).  The host side of the tables is one static
// buffer, reused after the event of its last copy has completed.
__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

struct StaticScratch {
  std::mutex mu;
  void* dev_ptr[64] = {};           // scratch on each device
  hipEvent_t copied[64] = {};       // the last table copy from `host` to that device
  bool pending[64] = {};
  alignas(256) char host[kStaticScratchBytes];
};
StaticScratch g_static;

}  // namespace

size_t batched_workspace_bytes(int n_phases) { return n_phases > 0 ? table_bytes(n_phases) : 0; }

int launch_decode_step_batched(const spax_step* st, int n_cu, hipStream_t s) {
  const int n = st->n_phases;
  std::vector<char> table(table_bytes(n));
  BatchItems bi;
  if (!build_tables(st, table.data(), &bi)) return SPAX_ERR_SHAPE;
  int rc = stage_and_copy(table.data(), table.size(), st->ws, s);
  if (rc) return rc;
  return launch_from_tables(st, n_cu, st->ws, bi, s);
}

int launch_decode_step_batched_static(const spax_step* st, int n_cu, hipStream_t s) {
  const size_t bytes = table_bytes(st->n_phases);
  if (bytes > kStaticScratchBytes)
    return fail(SPAX_ERR_WORKSPACE, "%d phases need %zu bytes of descriptor tables; the static "
                "scratch holds %zu", st->n_phases, bytes, kStaticScratchBytes);
  int dev = 0;
  SPAX_HIP_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) return fail(SPAX_ERR_UNSUPPORTED, "device index %d", dev);
  std::lock_guard<std::mutex> lock(g_static.mu);
  if (!g_static.dev_ptr[dev]) {  // once per device, with that device current
    void* p = nullptr;
    SPAX_HIP_CHECK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(SPAX_ERR_HIP, "hipGetSymbolAddress returned NULL for the scratch");
    SPAX_HIP_CHECK(hipEventCreateWithFlags(&g_static.copied[dev], hipEventDisableTiming));
    g_static.dev_ptr[dev] = p;
  }
  // The host buffer is shared by every device: wait for each copy still reading it.
  for (int d = 0; d < 64; ++d) {
    if (!g_static.pending[d]) continue;
    SPAX_HIP_CHECK(hipEventSynchronize(g_static.copied[d]));
    g_static.pending[d] = false;
  }
  BatchItems bi;
  if (!build_tables(st, g_static.host, &bi)) return SPAX_ERR_SHAPE;
  void* dtables = g_static.dev_ptr[dev];
  SPAX_HIP_CHECK(hipMemcpyAsync(dtables, g_static.host, bytes, hipMemcpyHostToDevice, s));
  SPAX_HIP_CHECK(hipEventRecord(g_static.copied[dev], s));
  g_static.pending[dev] = true;
  return launch_from_tables(st, n_cu, dtables, bi, s);
}

}  // namespace spax
