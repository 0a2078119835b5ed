// Stand-alone tier mask of one activation vector: one workgroup of 16 wavefronts.
//
// Pages: SpAx Abstract (arXiv:2610.02598) -- tiers by |x|; TopK-Guided (arXiv:2610.01763)
// section 2.1 -- clipped natural sparsity then TopK, O(d) per token.  The selection logic
// lives in mask_core.h; this kernel writes the tier bytes, both ascending index lists and
// the counts to global memory.
#include <climits>

#include "mask_core.h"

namespace spax {
namespace {

// One workgroup of 16 waves: the kernel is issue- and latency-bound inside one CU.
constexpr int kTierThreads = 1024;

template <int NT>
__global__ __launch_bounds__(NT) void build_tiers_kernel(
    TierArgs a, const uint16_t* __restrict__ x, uint8_t* __restrict__ tier,
    int32_t* __restrict__ full_idx, int32_t* __restrict__ approx_idx,
    int32_t* __restrict__ counts, float4* __restrict__ y_zero, int32_t n_zero4) {
  __shared__ mask::KeyHist<NT> sh;
  __shared__ uint32_t xs32[SPAX_MAX_DIN / 2];
  mask::tiers_to_global<NT, SPAX_MAX_DIN>(sh, xs32, a, x, tier, full_idx, approx_idx, counts);
  // Side job: clear the fp32 output the following GEMV accumulates into.  Issued last, so
  // that waiting for the activation loads never includes these stores.
  for (int i = threadIdx.x; i < n_zero4; i += NT) y_zero[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

}  // namespace

int launch_build_tiers(const TierArgs& a, const uint16_t* x, uint8_t* tier, int32_t* full_idx,
                       int32_t* approx_idx, int32_t* counts, float* y_zero, int64_t n_zero,
                       hipStream_t s) {
  const int32_t n4 = y_zero ? (int32_t)((n_zero + 3) / 4) : 0;
  float4* yz = reinterpret_cast<float4*>(y_zero);
  hipLaunchKernelGGL(build_tiers_kernel<kTierThreads>, dim3(1), dim3(kTierThreads), 0, s, a, x,
                     tier, full_idx, approx_idx, counts, yz, n4);
  SPAX_HIP_CHECK(hipGetLastError());
  return SPAX_OK;
}

}  // namespace spax
