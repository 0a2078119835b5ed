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
#include <cstdlib>

#include "gemv_core.h"

namespace spax {
namespace {

using gemv::kWaves;

template <int FMT, bool kCompact>
__global__ __launch_bounds__(kGemvThreads) void tiered_gemv_kernel(
    gemv::Shape sh, const uint8_t* __restrict__ packed, const uint32_t* __restrict__ x32,
    const int32_t* __restrict__ full_idx, const int32_t* __restrict__ approx_idx,
    const int32_t* __restrict__ counts, float* __restrict__ y) {
  __shared__ float red[kWaves][kTileRows];
  const int item = gemv::xcd_order((int)blockIdx.x, (int)gridDim.x);
  const int tile = (int)((uint32_t)item % (uint32_t)sh.n_tiles);
  const int chunk = (int)((uint32_t)item / (uint32_t)sh.n_tiles);
  gemv::gemv_item<FMT, kCompact>(sh, packed, x32, full_idx, approx_idx, counts, y, tile, chunk,
                                 red);
}

// Pinned-host gather: staging slot s of a region receives the record of column col[s] read
// from the mapped host blob.  16-byte chunks, grid-stride; records are multiples of 128 bytes.
__global__ __launch_bounds__(256) void gather_records_kernel(
    const uint8_t* __restrict__ host, uint8_t* __restrict__ staging,
    const int32_t* __restrict__ colF, int64_t chunksF, int64_t strideF,
    const int32_t* __restrict__ colA, int64_t chunksA, int64_t strideA, int64_t offA) {
  const int64_t n = chunksF + chunksA;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < n;
       c += (int64_t)gridDim.x * blockDim.x) {
    const bool a = c >= chunksF;
    const int64_t b = (a ? c - chunksF : c) * 16;
    const int64_t stride = a ? strideA : strideF;
    const int64_t base = a ? offA : 0;
    const int64_t slot = b / stride, in = b - slot * stride;
    const int32_t col = (a ? colA : colF)[slot];
    const uint4 v = *reinterpret_cast<const uint4*>(host + base + (int64_t)col * stride + in);
    *reinterpret_cast<uint4*>(staging + base + b) = v;
  }
}

__global__ __launch_bounds__(256) void zero_f32_kernel(float4* __restrict__ p, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n4) p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  if (!v || !*v) return dflt;
  return atoi(v);
}

}  // namespace

GemvPlan gemv_plan(const spax_layout* L) {
  GemvPlan p{};
  const int64_t T = L->d_out_total;
  p.n_tiles = (int32_t)((T + kTileRows - 1) / kTileRows);
  // Split-K: aim for about `target` resident workgroups, but keep >= 16 input channels per
  // chunk.
  static const int target = env_int("SPAX_GEMV_TARGET_WGS", 1024);
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

int launch_gather_records(const spax_layout* L, const void* host_dev, void* staging,
                          const int32_t* colF, int32_t nF_slots, const int32_t* colA,
                          int32_t nA_slots, hipStream_t s) {
  const int64_t cF = (int64_t)nF_slots * L->stride_F / 16, cA = (int64_t)nA_slots * L->stride_A / 16;
  if (cF + cA == 0) return SPAX_OK;
  const int64_t blocks = std::min<int64_t>((cF + cA + 255) / 256, 4096);
  hipLaunchKernelGGL(gather_records_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<const uint8_t*>(host_dev), static_cast<uint8_t*>(staging), colF,
                     cF, L->stride_F, colA, cA, L->stride_A, L->off_A);
  SPAX_HIP_CHECK(hipGetLastError());
  return SPAX_OK;
}

int launch_tiered_gemv(const spax_layout* L, const GemvPlan& plan, const void* packed,
                       const uint16_t* x, const int32_t* full_idx, const int32_t* approx_idx,
                       const int32_t* counts, float* y, bool y_zeroed, hipStream_t s,
                       bool compact) {
  if (plan.n_chunks > 1 && !y_zeroed) {
    int st = launch_zero_f32(y, L->d_out_total, s);
    if (st) return st;
  }
  const gemv::Shape sh = gemv_shape(L, plan);
  const dim3 grid((unsigned)(plan.n_tiles * plan.n_chunks));
  const auto* pk = static_cast<const uint8_t*>(packed);
  const auto* x32 = reinterpret_cast<const uint32_t*>(x);
#define SPAX_GEMV_LAUNCH(F, C)                                                              \
  hipLaunchKernelGGL((tiered_gemv_kernel<F, C>), grid, dim3(kGemvThreads), 0, s, sh, pk, x32, \
                     full_idx, approx_idx, counts, y)
  if (L->base_fmt == SPAX_FMT_FP16) {
    if (compact) SPAX_GEMV_LAUNCH(SPAX_FMT_FP16, true);
    else SPAX_GEMV_LAUNCH(SPAX_FMT_FP16, false);
  } else {
    if (compact) SPAX_GEMV_LAUNCH(SPAX_FMT_INT4, true);
    else SPAX_GEMV_LAUNCH(SPAX_FMT_INT4, false);
  }
#undef SPAX_GEMV_LAUNCH
  SPAX_HIP_CHECK(hipGetLastError());
  return SPAX_OK;
}

}  // namespace spax
