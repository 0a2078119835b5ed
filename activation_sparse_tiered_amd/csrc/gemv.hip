// Stand-alone tiered gather-GEMV (spax_tiered_gemv): column lists and counts in global
// memory, as written by spax_build_tiers.
//
// Pages: SpAx Abstract (arXiv:2610.02598); eigenradar commentary on SpAx, "The route outside
// GPU memory" (per-column tiers, two-bit approximations reconstructed on the GPU).  The
// column loops are in gemv_core.h.
//
// Work decomposition: a workgroup of 8 wavefronts owns one 512-row tile and one chunk of
// each selected-column list (split-K over columns); its waves split the chunk.  Waves add
// through LDS; chunks of one tile meet in y through fp32 atomic adds.  A fence-based "last
// workgroup reduces" scheme was measured two orders of magnitude slower: a device-scope
// fence writes back and invalidates the L2 of the caller's XCD.  The order in which chunks
// land is not fixed, so y may differ in the last bits between runs.
#include <algorithm>

#include "gemv_core.h"

namespace spax {
namespace {

using gemv::kWaves;

template <int FMT, bool kCompact, class Blob>
__global__ __launch_bounds__(kGemvThreads) void tiered_gemv_kernel(
    gemv::Shape sh, const uint8_t* __restrict__ packed, const uint32_t* __restrict__ x32,
    const int32_t* __restrict__ full_idx, const int32_t* __restrict__ approx_idx,
    const int32_t* __restrict__ counts, float* __restrict__ y, float* __restrict__ partials) {
  __shared__ float red[kWaves * kTileRows];
  const int item = gemv::xcd_order((int)blockIdx.x, (int)gridDim.x);
  const int tile = (int)((uint32_t)item % (uint32_t)sh.n_tiles);
  const int chunk = (int)((uint32_t)item / (uint32_t)sh.n_tiles);
  gemv::gemv_item<FMT, Blob, kCompact>(sh, packed, x32, full_idx, approx_idx, counts, y, tile,
                                       chunk, red, partials);
}

// Deterministic mode: y[r] = sum over c = 0 .. n_chunks - 1, in that order, of
// partials[c][r] (four rows per thread; T is a multiple of 4).
__global__ __launch_bounds__(256) void reduce_chunks_kernel(const float4* __restrict__ partials,
                                                            int32_t n_chunks, int64_t T4,
                                                            float4* __restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T4) return;
  float4 s = partials[i];
  for (int32_t c = 1; c < n_chunks; ++c) {
    const float4 v = partials[(int64_t)c * T4 + i];
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  }
  y[i] = s;
}

// Range merging on the device (pinned-host path, gather transfer): workgroup r merges region
// r's list (0 FULL, 1 APPROX) into runs of channels whose gaps are at most `gap` unselected
// channels, and writes what the host merge would: the compacted entries (staging slot |
// channel << 16), the slot -> channel table and the totals.  Entry i contributes the columns
// from its channel up to (not including) the next entry of its run, or just its own column
// when it ends the run; its slot is the exclusive prefix sum of those contributions, so the
// columns of a run land in consecutive slots and runs follow each other.  Each thread takes
// a contiguous share of the entries; one block-wide scan gives the prefixes.  Lists that
// are not strictly ascending start a new run at every descent and stay memory-safe (slots
// and table writes are kept below d), with an unspecified y.
constexpr int kMergeThreads = 1024;
constexpr int kMergeWaves = kMergeThreads / 64;

__device__ __forceinline__ int merge_wave_scan(int x) {  // inclusive, DPP
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);
  return x;
}

__global__ __launch_bounds__(kMergeThreads) void merge_ranges_kernel(
    const int32_t* __restrict__ full_idx, const int32_t* __restrict__ approx_idx,
    const int32_t* __restrict__ counts, int32_t d, int32_t gap, uint32_t* __restrict__ listF,
    uint32_t* __restrict__ listA, int32_t* __restrict__ colF, int32_t* __restrict__ colA,
    int32_t* __restrict__ totals) {
  __shared__ int wsum[2][kMergeWaves];
  const int r = blockIdx.x;
  const int32_t* idx = r ? approx_idx : full_idx;
  uint32_t* out = r ? listA : listF;
  int32_t* col = r ? colA : colF;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = min(max(counts[r], 0), d);
  const int per = (n + kMergeThreads - 1) / kMergeThreads;
  const int b = min(tid * per, n), e = min(b + per, n);
  auto chan = [&](int i) { return min(max(idx[i], 0), d - 1); };
  // does entry i + 1 continue entry i's run?
  auto joins = [&](int i) {
    if (i + 1 >= n) return false;
    const int a = chan(i), c = chan(i + 1);
    return c > a && c - a - 1 <= gap;
  };
  int cols = 0, runs = 0;
  for (int i = b; i < e; ++i) {
    cols += joins(i) ? chan(i + 1) - chan(i) : 1;
    runs += (i == 0 || !joins(i - 1)) ? 1 : 0;
  }
  const int sc = merge_wave_scan(cols), sr = merge_wave_scan(runs);
  if (lane == 63) {
    wsum[0][wave] = sc;
    wsum[1][wave] = sr;
  }
  __syncthreads();
  int base = 0, tot_cols = 0, tot_runs = 0;
  for (int w = 0; w < kMergeWaves; ++w) {
    base += w < wave ? wsum[0][w] : 0;
    tot_cols += wsum[0][w];
    tot_runs += wsum[1][w];
  }
  int slot = base + sc - cols;  // exclusive prefix of this thread's first entry
  for (int i = b; i < e; ++i) {
    const int c = chan(i);
    const int len = joins(i) ? chan(i + 1) - c : 1;
    out[i] = (uint32_t)min(slot, d - 1) | ((uint32_t)c << 16);
    for (int t = 0; t < len && slot + t < d; ++t) col[slot + t] = c + t;
    slot += len;
  }
  if (tid == 0) {
    totals[r] = min(tot_cols, d);  // staging slots used
    totals[2 + r] = tot_runs;      // ranges
    totals[4 + r] = n;             // entries
  }
}

// Pinned-host gather: staging slot s of a region receives the record of column col[s] read
// from the mapped host blob.  16-byte chunks, grid-stride; records are multiples of 128 bytes;
// the slot counts are read on the device (totals[0], totals[1] from merge_ranges_kernel).
__global__ __launch_bounds__(256) void gather_records_kernel(
    const uint8_t* __restrict__ host, uint8_t* __restrict__ staging,
    const int32_t* __restrict__ colF, int64_t strideF, const int32_t* __restrict__ colA,
    int64_t strideA, int64_t offA, const int32_t* __restrict__ totals, int32_t d) {
  const int64_t chunksF = (int64_t)totals[0] * strideF / 16;
  const int64_t chunksA = (int64_t)totals[1] * strideA / 16;
  const int64_t n = chunksF + chunksA;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < n;
       c += (int64_t)gridDim.x * blockDim.x) {
    const bool a = c >= chunksF;
    const int64_t b = (a ? c - chunksF : c) * 16;
    const int64_t stride = a ? strideA : strideF;
    const int64_t base = a ? offA : 0;
    const int64_t slot = b / stride, in = b - slot * stride;
    const int32_t col = min(max((a ? colA : colF)[slot], 0), d - 1);  // never outside the blob
    const uint4 v = *reinterpret_cast<const uint4*>(host + base + (int64_t)col * stride + in);
    *reinterpret_cast<uint4*>(staging + base + b) = v;
  }
}

__global__ __launch_bounds__(256) void zero_f32_kernel(float4* __restrict__ p, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n4) p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

}  // namespace

GemvPlan gemv_plan(const spax_layout* L) {
  GemvPlan p{};
  const int64_t T = L->d_out_total;
  p.n_tiles = (int32_t)((T + kTileRows - 1) / kTileRows);
  // Split-K: aim for about 1024 workgroups (four per compute unit), but keep >= 16 input
  // channels per chunk.
  constexpr int target = 1024;
  int k = (target + p.n_tiles / 2) / p.n_tiles;
  const int kmax = L->d_in / 16 > 1 ? L->d_in / 16 : 1;
  if (k > kmax) k = kmax;
  if (k < 1) k = 1;
  p.n_chunks = k;
  p.ws_bytes = 0;
  return p;
}

gemv::Shape gemv_shape(const spax_layout* L, const GemvPlan& plan) {
  gemv::Shape sh{};
  sh.stride_F = L->stride_F;
  sh.stride_A = L->stride_A;
  sh.off_A = L->off_A;
  sh.T = (int32_t)L->d_out_total;
  sh.n_tiles = plan.n_tiles;
  sh.n_chunks = plan.n_chunks;
  sh.approx_group = L->approx_group;
  sh.base_group = L->base_group;
  sh.d_in = L->d_in;
  return sh;
}

int launch_zero_f32(float* y, int64_t n, hipStream_t s) {
  const int64_t n4 = (n + 3) / 4;
  const int threads = 256;
  hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)((n4 + threads - 1) / threads)), dim3(threads),
                     0, s, reinterpret_cast<float4*>(y), n4);
  SPAX_HIP_CHECK(hipGetLastError());
  return SPAX_OK;
}

int launch_merge_and_gather(const spax_layout* L, const void* host_dev, void* staging,
                            const int32_t* full_idx, const int32_t* approx_idx,
                            const int32_t* counts, int32_t gap, uint32_t* listF, uint32_t* listA,
                            int32_t* colF, int32_t* colA, int32_t* totals, hipStream_t s) {
  hipLaunchKernelGGL(merge_ranges_kernel, dim3(2), dim3(kMergeThreads), 0, s, full_idx,
                     approx_idx, counts, L->d_in, gap, listF, listA, colF, colA, totals);
  SPAX_HIP_CHECK(hipGetLastError());
  // grid for the largest possible move (every column of both regions)
  const int64_t most = (L->d_in * L->stride_F + L->d_in * L->stride_A) / 16;
  const int64_t blocks = std::min<int64_t>((most + 255) / 256, 4096);
  hipLaunchKernelGGL(gather_records_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<const uint8_t*>(host_dev), static_cast<uint8_t*>(staging), colF,
                     L->stride_F, colA, L->stride_A, L->off_A, totals, L->d_in);
  SPAX_HIP_CHECK(hipGetLastError());
  return SPAX_OK;
}

int launch_reduce_chunks(const float* partials, int32_t n_chunks, int64_t T, float* y,
                         hipStream_t s) {
  const int64_t T4 = T / 4;
  const int threads = 256;
  hipLaunchKernelGGL(reduce_chunks_kernel, dim3((unsigned)((T4 + threads - 1) / threads)),
                     dim3(threads), 0, s, reinterpret_cast<const float4*>(partials), n_chunks,
                     T4, reinterpret_cast<float4*>(y));
  SPAX_HIP_CHECK(hipGetLastError());
  return SPAX_OK;
}

int launch_tiered_gemv(const spax_layout* L, const GemvPlan& plan, const void* packed,
                       const uint16_t* x, const int32_t* full_idx, const int32_t* approx_idx,
                       const int32_t* counts, float* y, bool y_zeroed, hipStream_t s,
                       bool compact, float* partials) {
  if (plan.n_chunks == 1) partials = nullptr;  // one chunk: plain stores, already deterministic
  if (plan.n_chunks > 1 && !y_zeroed && !partials) {
    int st = launch_zero_f32(y, L->d_out_total, s);
    if (st) return st;
  }
  const gemv::Shape sh = gemv_shape(L, plan);
  const dim3 grid((unsigned)(plan.n_tiles * plan.n_chunks));
  const auto* pk = static_cast<const uint8_t*>(packed);
  const auto* x32 = reinterpret_cast<const uint32_t*>(x);
  // The compacted staging copy has the blob's layout (record slots in place of channels).
  const bool narrow = narrow_regions(L);
#define SPAX_GEMV_LAUNCH(F, C, B)                                                             \
  hipLaunchKernelGGL((tiered_gemv_kernel<F, C, gemv::B>), grid, dim3(kGemvThreads), 0, s, sh, \
                     pk, x32, full_idx, approx_idx, counts, y, partials)
#define SPAX_GEMV_LAUNCH_FMT(F)                                    \
  if (compact && narrow) SPAX_GEMV_LAUNCH(F, true, RegionBlob);    \
  else if (compact) SPAX_GEMV_LAUNCH(F, true, RecordBlob);         \
  else if (narrow) SPAX_GEMV_LAUNCH(F, false, RegionBlob);         \
  else SPAX_GEMV_LAUNCH(F, false, RecordBlob)
  if (L->base_fmt == SPAX_FMT_FP16) {
    SPAX_GEMV_LAUNCH_FMT(SPAX_FMT_FP16);
  } else {
    SPAX_GEMV_LAUNCH_FMT(SPAX_FMT_INT4);
  }
#undef SPAX_GEMV_LAUNCH_FMT
#undef SPAX_GEMV_LAUNCH
  SPAX_HIP_CHECK(hipGetLastError());
  if (partials) return launch_reduce_chunks(partials, plan.n_chunks, L->d_out_total, y, s);
  return SPAX_OK;
}

}  // namespace spax
