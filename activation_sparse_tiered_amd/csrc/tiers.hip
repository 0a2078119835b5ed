// Stand-alone tier mask of one activation vector: one workgroup of 16 wavefronts.
//
// Pages: SpAx Abstract (arXiv:2610.02598) -- tiers by |x|; TopK-Guided (arXiv:2610.01763)
// section 2.1 -- clipped natural sparsity then TopK, O(d) per token.  The selection logic
// lives in mask_core.h; this kernel writes the tier bytes, both ascending index lists and
// the counts to global memory.
#include "mask_core.h"

namespace spax {
namespace {

constexpr int kTierThreads = 1024;

__global__ __launch_bounds__(kTierThreads) void build_tiers_kernel(
    TierArgs a, const uint16_t* __restrict__ x, uint8_t* __restrict__ tier,
    int32_t* __restrict__ full_idx, int32_t* __restrict__ approx_idx,
    int32_t* __restrict__ counts, float4* __restrict__ y_zero, int32_t n_zero4) {
  __shared__ mask::Shared<kTierThreads> sh;
  __shared__ uint32_t xs32[SPAX_MAX_DIN / 2];
  const int tid = threadIdx.x;

  // Side job: clear the fp32 output the following GEMV accumulates into.
  for (int i = tid; i < n_zero4; i += kTierThreads) y_zero[i] = make_float4(0.f, 0.f, 0.f, 0.f);

  mask::Keys k;
  const mask::Plan p = mask::build_plan<kTierThreads, SPAX_MAX_DIN>(sh, k, xs32, x, a);
  mask::emit<kTierThreads>(
      sh, k, p,
      [&](int t, int rank, int j, uint32_t) {
        if (t == SPAX_TIER_FULL) full_idx[rank] = j;
        else approx_idx[rank] = j;
      },
      [&](int j, int t) {
        if (tier) tier[j] = (uint8_t)t;
      });
  if (tid == 0) {
    counts[0] = p.n_full;
    counts[1] = p.n_kept - p.n_full;
    counts[2] = a.d - p.n_kept;
  }
}

}  // namespace

int launch_build_tiers(const TierArgs& a, const uint16_t* x, uint8_t* tier, int32_t* full_idx,
                       int32_t* approx_idx, int32_t* counts, float* y_zero, int64_t n_zero,
                       hipStream_t s) {
  const int32_t n4 = y_zero ? (int32_t)((n_zero + 3) / 4) : 0;
  hipLaunchKernelGGL(build_tiers_kernel, dim3(1), dim3(kTierThreads), 0, s, a, x, tier, full_idx,
                     approx_idx, counts, reinterpret_cast<float4*>(y_zero), n4);
  SPAX_HIP_CHECK(hipGetLastError());
  return SPAX_OK;
}

}  // namespace spax
