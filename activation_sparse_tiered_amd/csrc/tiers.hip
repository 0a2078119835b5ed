// Tier mask of one activation vector: one workgroup of 16 wavefronts.
//
// Pages: SpAx Abstract (arXiv:2610.02598): the largest-magnitude activations read original
// weights, smaller ones approximate weights, those closest to zero nothing.  TopK-Guided
// (arXiv:2610.01763) section 2.1: estimate the natural sparsity from the calibrated
// threshold, clip it to +-delta around the target, then TopK; O(d) per token.
//
// Everything on the device is integer.  key = bits(x) & 0x7FFF orders |x| (NaN above +Inf);
// the ranking is (key descending, index ascending), a total order, so each output has one
// correct value.  A TopK boundary of R elements is found by a two-level radix select over
// the 15-bit keys (8 high bits, then 7 low bits, LDS histograms); it becomes a pair
// (kb, m): an element is selected iff key > kb, or key == kb and it is among the first m
// channels (by index) whose key equals kb.  Threshold masks use (K(tau), all).  The ascending
// index lists are compacted with wavefront ballots: each wave owns a contiguous index
// range, so ballot prefix counts plus a per-wave base give the ascending order directly.
#include "common.h"

namespace spax {
namespace {

constexpr int kTierThreads = 1024;
constexpr int kWaves = kTierThreads / 64;

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }

struct Select {
  int32_t kb;  // boundary key
  int32_t m;   // how many channels with key == kb are selected (lowest indices first)
};

// One wave: find the bucket of a suffix histogram holding rank target R.
// hist has nb = 64 * per bins; `above` is the count of elements in higher buckets before
// this histogram.  Returns bucket b and the count strictly above b (including `above`).
template <int per>
__device__ void suffix_find(const int* hist, int R, int above, int lane, int* out_b,
                            int* out_above) {
  int local[per];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < per; ++i) {
    local[i] = hist[lane * per + i];
    sum += local[i];
  }
  // inclusive suffix scan over lanes: S_l = sum over lanes >= l
  int suf = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int v = __shfl_down(suf, off, 64);
    if (lane + off < 64) suf += v;
  }
  // count strictly above this lane's bins
  int run = above + suf - sum;
  // walk this lane's bins from the top; the crossing bin is where run + bin >= R first
#pragma unroll
  for (int i = per - 1; i >= 0; --i) {
    if (run < R && run + local[i] >= R) {
      *out_b = lane * per + i;
      *out_above = run;
    }
    run += local[i];
  }
}

__global__ __launch_bounds__(kTierThreads) void build_tiers_kernel(
    TierArgs a, const uint16_t* __restrict__ x, uint8_t* __restrict__ tier,
    int32_t* __restrict__ full_idx, int32_t* __restrict__ approx_idx,
    int32_t* __restrict__ counts, float4* __restrict__ y_zero, int32_t n_zero4) {
  __shared__ uint16_t keys[SPAX_MAX_DIN];
  __shared__ int hist_hi[256];
  __shared__ int hist_lo[2][128];
  __shared__ int wave_a[kWaves], wave_b[kWaves];
  __shared__ int sel_b[2], sel_above[2];
  __shared__ Select sel[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int d = a.d;
  const int chunk = ((d + kWaves - 1) / kWaves + 63) / 64 * 64;
  const int w_begin = min(wave * chunk, d);
  const int w_end = min(w_begin + chunk, d);

  // Side job: clear the fp32 output the following GEMV accumulates into.
  for (int i = tid; i < n_zero4; i += kTierThreads) y_zero[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int i = tid; i < 256; i += kTierThreads) hist_hi[i] = 0;
  for (int i = tid; i < 256; i += kTierThreads) (&hist_lo[0][0])[i] = 0;
  __syncthreads();

  // ---- pass 0: keys into LDS, natural count below K(tau), high-byte histogram
  int nat = 0;
  for (int base = w_begin; base < w_end; base += 64) {
    const int j = base + lane;
    const bool valid = j < w_end;
    const int key = valid ? (int)(x[j] & 0x7FFFu) : 0;
    if (valid) {
      keys[j] = (uint16_t)key;
      atomicAdd(&hist_hi[key >> 7], 1);
    }
    nat += popc64(__ballot(valid && key < a.k_tau));
  }
  if (lane == 0) wave_a[wave] = nat;
  __syncthreads();

  // ---- counts of the two boundaries (uniform across the workgroup)
  int total_nat = 0;
  for (int w = 0; w < kWaves; ++w) total_nat += wave_a[w];
  int R[2] = {0, 0};
  bool thresholds = false;
  if (a.mode == SPAX_MODE_TOPK) {
    R[0] = a.n_full;
    R[1] = a.n_full + a.n_approx;
  } else if (a.mode == SPAX_MODE_TOPK_GUIDED) {
    const int n_skip = min(max(total_nat, a.n_lo), a.n_hi);
    const int kept = d - n_skip;
    const int n_approx = (int)(((int64_t)a.num * kept + a.den / 2) / a.den);
    R[0] = kept - n_approx;
    R[1] = kept;
  } else {
    thresholds = true;
  }

  if (!thresholds) {
    // ---- level 1: high byte
    if (wave < 2) {
      const int r = R[wave];
      if (r == 0) {
        if (lane == 0) { sel_b[wave] = -1; sel_above[wave] = 0; }
      } else {
        int b = 0, ab = 0;
        bool found = false;
        {
          int ob = -1, oab = 0;
          suffix_find<4>(hist_hi, r, 0, lane, &ob, &oab);
          const uint64_t hit = __ballot(ob >= 0);
          const int src = hit ? (int)__builtin_ctzll(hit) : 0;
          b = __shfl(ob, src, 64);
          ab = __shfl(oab, src, 64);
          found = hit != 0;
        }
        if (lane == 0) { sel_b[wave] = found ? b : 0; sel_above[wave] = ab; }
      }
    }
    __syncthreads();
    const int b0 = sel_b[0], b1 = sel_b[1];
    // ---- level 2: low 7 bits inside the boundary buckets
    for (int j = tid; j < d; j += kTierThreads) {
      const int key = keys[j];
      if ((key >> 7) == b0) atomicAdd(&hist_lo[0][key & 127], 1);
      if ((key >> 7) == b1) atomicAdd(&hist_lo[1][key & 127], 1);
    }
    __syncthreads();
    if (wave < 2) {
      const int r = R[wave];
      if (r == 0) {
        if (lane == 0) sel[wave] = Select{0x8000, 0};
      } else {
        int ov = -1, oab = 0;
        suffix_find<2>(hist_lo[wave], r, sel_above[wave], lane, &ov, &oab);
        const uint64_t hit = __ballot(ov >= 0);
        const int src = hit ? (int)__builtin_ctzll(hit) : 0;
        const int v = __shfl(ov, src, 64);
        const int ab = __shfl(oab, src, 64);
        if (lane == 0) sel[wave] = Select{(sel_b[wave] << 7) | v, r - ab};
      }
    }
    __syncthreads();
  } else {
    if (tid == 0) {
      sel[0] = Select{a.k_full, d};
      sel[1] = Select{a.k_skip, d};
    }
    __syncthreads();
  }
  const Select s0 = sel[0], s1 = sel[1];

  // ---- pass 3a: per-wave counts of boundary-key channels (for the index tie-break)
  int eq0 = 0, eq1 = 0;
  for (int base = w_begin; base < w_end; base += 64) {
    const int j = base + lane;
    const bool valid = j < w_end;
    const int key = valid ? keys[j] : -1;
    eq0 += popc64(__ballot(key == s0.kb));
    eq1 += popc64(__ballot(key == s1.kb));
  }
  __syncthreads();  // wave_a reuse
  if (lane == 0) { wave_a[wave] = eq0; wave_b[wave] = eq1; }
  __syncthreads();
  int eqbase0 = 0, eqbase1 = 0;
  for (int w = 0; w < wave; ++w) { eqbase0 += wave_a[w]; eqbase1 += wave_b[w]; }

  // ---- pass 3b: classify, write tier bytes, count per wave
  int nF = 0, nA = 0;
  {
    int e0 = eqbase0, e1 = eqbase1;
    for (int base = w_begin; base < w_end; base += 64) {
      const int j = base + lane;
      const bool valid = j < w_end;
      const int key = valid ? keys[j] : -1;
      const uint64_t m0 = __ballot(key == s0.kb);
      const uint64_t m1 = __ballot(key == s1.kb);
      const bool isF = valid && (key > s0.kb || (key == s0.kb && (int)(e0 + lanes_below(m0)) < s0.m));
      const bool kept = valid && (key > s1.kb || (key == s1.kb && (int)(e1 + lanes_below(m1)) < s1.m));
      const bool isA = kept && !isF;
      e0 += popc64(m0);
      e1 += popc64(m1);
      nF += popc64(__ballot(isF));
      nA += popc64(__ballot(isA));
      if (valid && tier) tier[j] = isF ? (uint8_t)SPAX_TIER_FULL : isA ? (uint8_t)SPAX_TIER_APPROX
                                                                        : (uint8_t)SPAX_TIER_SKIP;
    }
  }
  __syncthreads();
  if (lane == 0) { wave_a[wave] = nF; wave_b[wave] = nA; }
  __syncthreads();
  int fbase = 0, abase = 0, fTot = 0, aTot = 0;
  for (int w = 0; w < kWaves; ++w) {
    if (w < wave) { fbase += wave_a[w]; abase += wave_b[w]; }
    fTot += wave_a[w];
    aTot += wave_b[w];
  }

  // ---- pass 3c: compact ascending index lists
  {
    int e0 = eqbase0, e1 = eqbase1;
    int fp = fbase, ap = abase;
    for (int base = w_begin; base < w_end; base += 64) {
      const int j = base + lane;
      const bool valid = j < w_end;
      const int key = valid ? keys[j] : -1;
      const uint64_t m0 = __ballot(key == s0.kb);
      const uint64_t m1 = __ballot(key == s1.kb);
      const bool isF = valid && (key > s0.kb || (key == s0.kb && (int)(e0 + lanes_below(m0)) < s0.m));
      const bool kept = valid && (key > s1.kb || (key == s1.kb && (int)(e1 + lanes_below(m1)) < s1.m));
      const bool isA = kept && !isF;
      e0 += popc64(m0);
      e1 += popc64(m1);
      const uint64_t bf = __ballot(isF);
      const uint64_t ba = __ballot(isA);
      if (isF) full_idx[fp + lanes_below(bf)] = j;
      if (isA) approx_idx[ap + lanes_below(ba)] = j;
      fp += popc64(bf);
      ap += popc64(ba);
    }
  }
  if (tid == 0) {
    counts[0] = fTot;
    counts[1] = aTot;
    counts[2] = d - fTot - aTot;
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
