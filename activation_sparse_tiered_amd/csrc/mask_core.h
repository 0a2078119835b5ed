// Tier-mask construction inside one workgroup, shared by the stand-alone mask kernel and
// the fused mask+GEMV kernel of the decode step.
//
// Pages: SpAx Abstract (arXiv:2610.02598) -- tiers follow |x| (largest: original, smaller:
// approximation, closest to zero: skipped).  TopK-Guided (arXiv:2610.01763) section 2.1 --
// natural sparsity from the calibrated threshold, clipped to +-delta, then TopK; O(d).
//
// All device work is integer.  key = bits(x) & 0x7FFF orders |x| (NaN above +Inf); the
// ranking is (key descending, index ascending).  A boundary holding R channels is a pair
// (kb, m): a channel is selected iff key > kb, or key == kb and it is among the first m
// channels (by index) whose key is kb.  Threshold masks use (K(tau), all).
//
// x is copied to LDS once; wave w owns the contiguous channels [w*C, (w+1)*C), C a multiple
// of 128.  Passes over the wave's channels:
//   1. 256-bin histogram of the high key bits (LDS atomics into lane-group copies) and
//      per-lane counters, summed once per wave;
//   2. (TopK boundaries) per-wave 128-bin histograms of the low bits inside the boundary
//      buckets, from which each wave gets its own "greater" / "equal" counts;
//   3. emit: ranks from ballots plus per-wave bases that wave 0 derives with one scan.
// The kernels are issue-bound inside one CU (every wave instruction competes with those of
// the other waves), so fixed per-wave work is kept small and is not repeated by each wave:
// two 16-bit counts share one 32-bit lane sum (a wave holds at most 32768 channels), and a
// step without boundary keys skips the tie ranking.
#pragma once

#include <climits>

#include "common.h"

namespace spax {
namespace mask {

struct Select {
  int32_t kb;  // boundary key
  int32_t m;   // channels with key == kb that are selected (lowest indices first)
};

template <int NT>
struct Shared {
  static constexpr int W = NT / 64;
  // Level-1 histogram in 8 copies (one per lane & 7, odd stride so the copies of a bin sit
  // in different banks): lanes whose keys share a bin mostly hit different addresses.
  static constexpr int kCopies = 8, kStride = 257;
  static constexpr int kRep = (kCopies * kStride + 3) / 4 * 4;
  alignas(16) int hist_rep[kRep];
  alignas(16) int wave_hist[2][W][128];
  int hist_hi[256];
  int wave_cnt[W][2];   // (gt | eq << 16) against the FULL and the kept boundary
  int wave_nat[W];      // natural count (keys below K(tau))
  int wave_base[W + 1][4];  // FULL rank base, APPROX rank base, ties before (FULL, kept);
                            // row W holds the totals
  int totals[2];        // n_full, n_kept
  int R[2];
  int sel_b[2], sel_above[2];
  Select sel[2];
};

// Channel layout: wave w owns channels [j0, j0 + n), j0 = w*C; at step s, lane l handles
// the two adjacent channels j0 + 128 s + 2 l + {0, 1}, stored as one dword of raw fp16 bits
// (low half: even channel) in LDS, so every step is one conflict-free 256-byte LDS read per
// wave.  Passes are rolled loops: the kernels run once per token, so their code is fetched
// cold and must stay small.
struct Keys {
  const uint32_t* xs32;  // LDS, d halves rounded up to dwords
  int C;                 // channels per wave (multiple of 128)
  int j0;                // first channel of this wave (even)
  int n;                 // channels of this wave
  int steps;             // steps of this wave
  __device__ __forceinline__ int off(int s, int lane, int e) const { return 128 * s + 2 * lane + e; }
  __device__ __forceinline__ bool valid(int s, int lane, int e) const { return off(s, lane, e) < n; }
  __device__ __forceinline__ uint32_t word(int s, int lane) const {
    return xs32[(j0 + off(s, lane, 0)) >> 1];
  }
};

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}
__device__ __forceinline__ int popc(uint64_t m) { return __popcll(m); }

// Inclusive prefix sum over the 64 lanes with DPP (row shifts, then row broadcasts); no LDS.
__device__ __forceinline__ int wave_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

// Sum over the 64 lanes, as a wave-uniform value.
__device__ __forceinline__ int wave_sum(int x) {
  return __builtin_amdgcn_readlane(wave_scan(x), 63);
}

// One wave: the bin of a suffix histogram (64 * per bins, lane l holding bins l*per..) where
// rank target R falls, and the count strictly above it (including `above`).  Wave-uniform.
template <int per>
__device__ __forceinline__ void suffix_find(const int (&local)[per], int R, int above, int lane,
                                            int* bin, int* bin_above) {
  int sum = 0;
#pragma unroll
  for (int i = 0; i < per; ++i) sum += local[i];
  const int pre = wave_scan(sum);
  const int total = __builtin_amdgcn_readlane(pre, 63);
  int run = above + total - pre;  // strictly above this lane's bins
  int ob = -1, oab = 0;
#pragma unroll
  for (int i = per - 1; i >= 0; --i) {
    if (run < R && run + local[i] >= R) {
      ob = lane * per + i;
      oab = run;
    }
    run += local[i];
  }
  const uint64_t hit = __ballot(ob >= 0);
  const int src = hit ? (int)__builtin_ctzll(hit) : 0;
  *bin = __builtin_amdgcn_readlane(ob, src);
  *bin_above = __builtin_amdgcn_readlane(oab, src);
}

// The two boundaries and the list totals (same on every thread).
struct Plan {
  Select s0, s1;  // FULL boundary, kept boundary
  int n_full, n_kept;
};

// Stage 1: load x into LDS (xs32: roundup(d, 2) halves), pass 1 and level 1.  Afterwards
// sh.sel holds the exact boundaries for THRESHOLD; otherwise sh.R holds the rank targets and
// sh.sel_b / sh.sel_above the level-1 buckets (-1: R == 0).  Ends with a barrier.  d <= MAXD.
template <int NT, int MAXD>
__device__ __forceinline__ void plan_stage1(Shared<NT>& sh, Keys& k, uint32_t* xs32,
                                            const uint16_t* __restrict__ x, const TierArgs& a) {
  constexpr int W = NT / 64;
  using S = Shared<NT>;
  static_assert(MAXD <= 32768 && NT >= 256, "per-wave counts are packed in 16 bits");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int d = a.d;
  k.xs32 = xs32;
  k.C = ((d + W - 1) / W + 127) / 128 * 128;
  k.j0 = min(wave * k.C, d);
  k.n = min(k.j0 + k.C, d) - k.j0;
  k.steps = (k.n + 127) / 128;
  const bool thresholds = a.mode == SPAX_MODE_THRESHOLD;

  // ---- x into LDS, four loads in flight per thread and iteration.  For odd d the last
  // dword also holds the two bytes past x (same dword, never used as a channel).
  {
    const uint32_t* x32 = reinterpret_cast<const uint32_t*>(x);
    const int ndw = (d + 1) >> 1;
    for (int i = tid; i < ndw; i += 4 * NT) {
      uint32_t v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = i + q * NT < ndw ? x32[i + q * NT] : 0u;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (i + q * NT < ndw) xs32[i + q * NT] = v[q];
    }
    // Every load has landed: say so to the compiler's wait tracking, so that loads issued
    // after the mask passes are not made to wait for these conditional ones.
    __builtin_amdgcn_s_waitcnt(0);
  }
  if (!thresholds) {
    const int4 z = make_int4(0, 0, 0, 0);
    int4* hr = reinterpret_cast<int4*>(sh.hist_rep);
    for (int i = tid; i < S::kRep / 4; i += NT) hr[i] = z;
    int4* wh = reinterpret_cast<int4*>(&sh.wave_hist[0][0][0]);
    for (int i = tid; i < 2 * W * 128 / 4; i += NT) wh[i] = z;
  }
  __syncthreads();

  // ---- pass 1: high-bit histogram and natural count, or the threshold counts
  if (thresholds) {
    int c0 = 0, c1 = 0;  // gt | eq << 16
    for (int s = 0; s < k.steps; ++s) {
      const uint32_t wd = k.word(s, lane);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int key = k.valid(s, lane, e) ? (int)((e ? wd >> 16 : wd) & 0x7FFFu) : -1;
        c0 += key > a.k_full ? 1 : key == a.k_full ? 0x10000 : 0;
        c1 += key > a.k_skip ? 1 : key == a.k_skip ? 0x10000 : 0;
      }
    }
    c0 = wave_sum(c0);
    c1 = wave_sum(c1);
    if (lane == 0) {
      sh.wave_cnt[wave][0] = c0;
      sh.wave_cnt[wave][1] = c1;
    }
    if (tid == 0) {
      sh.sel[0] = Select{a.k_full, d};
      sh.sel[1] = Select{a.k_skip, d};
    }
  } else {
    int nat = 0;
    for (int s = 0; s < k.steps; ++s) {
      const uint32_t wd = k.word(s, lane);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const bool valid = k.valid(s, lane, e);
        const int key = (int)((e ? wd >> 16 : wd) & 0x7FFFu);
        // unconditional (zero past the range): see select_begin
        atomicAdd(&sh.hist_rep[(lane & (S::kCopies - 1)) * S::kStride + (key >> 7)], valid ? 1 : 0);
        nat += valid && key < a.k_tau;
      }
    }
    nat = wave_sum(nat);
    if (lane == 0) sh.wave_nat[wave] = nat;
  }
  __syncthreads();

  if (!thresholds) {
    // ---- rank targets (wave 0) and the folded level-1 histogram (threads < 256)
    if (wave == 0) {
      int R0, R1;
      if (a.mode == SPAX_MODE_TOPK) {
        R0 = a.n_full;
        R1 = a.n_full + a.n_approx;
      } else {
        const int natural = wave_sum(lane < W ? sh.wave_nat[lane] : 0);
        const int n_skip = min(max(natural, a.n_lo), a.n_hi);
        const int kept = d - n_skip;
        // num <= den <= 65535 and kept <= 32768: fits 32 bits
        const int n_approx = (int)(((uint32_t)a.num * (uint32_t)kept + (uint32_t)(a.den / 2)) /
                                   (uint32_t)a.den);
        R0 = kept - n_approx;
        R1 = kept;
      }
      if (lane == 0) {
        sh.R[0] = R0;
        sh.R[1] = R1;
      }
    }
    for (int b = tid; b < 256; b += NT) {
      int t = 0;
#pragma unroll
      for (int c = 0; c < S::kCopies; ++c) t += sh.hist_rep[c * S::kStride + b];
      sh.hist_hi[b] = t;
    }
    __syncthreads();
    const int R[2] = {sh.R[0], sh.R[1]};
    // ---- level 1: bucket of each boundary (waves 0 and 1)
    if (wave < 2) {
      int local[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) local[i] = sh.hist_hi[lane * 4 + i];
      int b = -1, ab = 0;
      if (R[wave] > 0) suffix_find<4>(local, R[wave], 0, lane, &b, &ab);
      if (lane == 0) {
        sh.sel_b[wave] = R[wave] > 0 ? b : -1;
        sh.sel_above[wave] = ab;
      }
    }
    __syncthreads();
  }
}

// Stage 2: pass 2 and level 2 (TopK boundaries), then every wave's rank bases
// (sh.wave_base).  Returns the plan on every thread; ends with a barrier.
template <int NT>
__device__ __forceinline__ Plan plan_stage2(Shared<NT>& sh, const Keys& k, const TierArgs& a) {
  constexpr int W = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (a.mode != SPAX_MODE_THRESHOLD) {
    const int R[2] = {sh.R[0], sh.R[1]};
    const int b0 = sh.sel_b[0], b1 = sh.sel_b[1];
    // ---- pass 2: per-wave low-bit histograms inside the buckets; keys above the buckets
    // (above0 | above1 << 16)
    int above = 0;
    for (int s = 0; s < k.steps; ++s) {
      const uint32_t wd = k.word(s, lane);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const bool valid = k.valid(s, lane, e);
        const int key = (int)((e ? wd >> 16 : wd) & 0x7FFFu);
        const int hi = valid ? key >> 7 : -2;
        atomicAdd(&sh.wave_hist[0][wave][key & 127], hi == b0 ? 1 : 0);  // see select_begin
        atomicAdd(&sh.wave_hist[1][wave][key & 127], hi == b1 ? 1 : 0);
        above += (b0 >= 0 && hi > b0 ? 1 : 0) + (b1 >= 0 && hi > b1 ? 0x10000 : 0);
      }
    }
    above = wave_sum(above);
    __syncthreads();
    // ---- level 2: exact boundary keys (waves 0 and 1 sum the per-wave histograms)
    if (wave < 2) {
      int local[2] = {0, 0};
      for (int w = 0; w < W; ++w) {
        const int2 h = *reinterpret_cast<const int2*>(&sh.wave_hist[wave][w][lane * 2]);
        local[0] += h.x;
        local[1] += h.y;
      }
      int v = -1, ab = 0;
      if (R[wave] > 0) suffix_find<2>(local, R[wave], sh.sel_above[wave], lane, &v, &ab);
      if (lane == 0)
        sh.sel[wave] =
            R[wave] > 0 ? Select{(sh.sel_b[wave] << 7) | v, R[wave] - ab} : Select{0x8000, 0};
    }
    __syncthreads();
    // ---- this wave's (gt | eq << 16) against the boundaries, from its own histograms
    const int low0 = sh.sel[0].kb & 127, low1 = sh.sel[1].kb & 127;
    const int2 h0 = *reinterpret_cast<const int2*>(&sh.wave_hist[0][wave][lane * 2]);
    const int2 h1 = *reinterpret_cast<const int2*>(&sh.wave_hist[1][wave][lane * 2]);
    auto ge = [&](int bin, int c, int low) { return bin > low ? c : bin == low ? c << 16 : 0; };
    const int c0 = wave_sum(ge(lane * 2, h0.x, low0) + ge(lane * 2 + 1, h0.y, low0));
    const int c1 = wave_sum(ge(lane * 2, h1.x, low1) + ge(lane * 2 + 1, h1.y, low1));
    if (lane == 0) {
      // R == 0: boundary above every key, nothing greater or equal
      sh.wave_cnt[wave][0] = R[0] > 0 ? c0 + (above & 0xFFFF) : 0;
      sh.wave_cnt[wave][1] = R[1] > 0 ? c1 + (above >> 16) : 0;
    }
    __syncthreads();
  }

  // ---- rank bases of every wave (wave 0, lane w <-> wave w).  Ties are taken in index
  // order, so a wave's selected ties are clamp(m - ties before it, 0, its ties).
  Plan p;
  p.s0 = sh.sel[0];
  p.s1 = sh.sel[1];
  if (wave == 0) {
    const bool on = lane < W;
    const int w0 = on ? sh.wave_cnt[lane][0] : 0, w1 = on ? sh.wave_cnt[lane][1] : 0;  // lane W: 0
    const int g0 = w0 & 0xFFFF, e0 = w0 >> 16, g1 = w1 & 0xFFFF, e1 = w1 >> 16;
    const int eb0 = wave_scan(e0) - e0, eb1 = wave_scan(e1) - e1;  // up to 32768 each
    const int f = g0 + min(max(p.s0.m - eb0, 0), e0);
    const int kk = g1 + min(max(p.s1.m - eb1, 0), e1);
    const int fs = wave_scan(f), ks = wave_scan(kk);
    if (lane <= W) {
      sh.wave_base[lane][0] = fs - f;
      sh.wave_base[lane][1] = (ks - kk) - (fs - f);  // FULL is a subset of kept
      sh.wave_base[lane][2] = eb0;
      sh.wave_base[lane][3] = eb1;
    }
    if (lane == 0) {
      sh.totals[0] = __builtin_amdgcn_readlane(fs, 63);
      sh.totals[1] = __builtin_amdgcn_readlane(ks, 63);
    }
  }
  __syncthreads();
  p.n_full = sh.totals[0];
  p.n_kept = sh.totals[1];
  return p;
}

// Both stages: boundaries, totals and rank bases.
template <int NT, int MAXD>
__device__ __forceinline__ Plan build_plan(Shared<NT>& sh, Keys& k, uint32_t* xs32,
                                           const uint16_t* __restrict__ x, const TierArgs& a) {
  plan_stage1<NT, MAXD>(sh, k, xs32, x, a);
  return plan_stage2<NT>(sh, k, a);
}

// Exact selection from a per-key histogram (used by the fused decode kernel, which needs the
// boundaries but no ranks): one pass of LDS atomics into 32768 16-bit counters (two keys per
// dword; a count never exceeds 32768, so it cannot carry into its neighbour), 1024 partial
// sums of 32 keys each, then one wave finds each boundary with two suffix scans (partial
// sums, then the 32 keys of the chosen partial sum).  Compared with the two-level radix
// select above there is no second pass over the keys, and far fewer lanes collide in one
// counter (equal keys only).
template <int NT>
struct KeyHist {
  static constexpr int W = NT / 64;
  alignas(16) uint32_t fine[16384];  // count of key 2i in bits 0..15, of key 2i + 1 in 16..31
  alignas(16) int coarse[1024];      // channels with key in [32c, 32c + 32)
  int wave_nat[W];
  // For a caller that shares out column lists among its waves after the search: per wave,
  // the next unclaimed FULL / APPROX entry ([0], [1]) and the published list lengths ([2],
  // [3]); zeroed by select_begin before its first barrier.
  int lists_q[4][W];
  Select sel[2];
  int E[2];
};

// Exact boundaries from a per-key histogram, in two parts (a caller may do other work in
// between).  select_begin loads x into LDS (xs32: roundup(d, 2) halves), sets k like
// build_plan, builds the per-key histogram and the coarse one (32 keys per bin), and gives
// every wave the two target ranks R (FULL, kept; counted from the largest key).  For
// THRESHOLD the boundaries are the given keys: sel and E are set and false is returned.
// Both histograms are complete on return (its last barrier follows the last atomic).
template <int NT, int MAXD>
__device__ __forceinline__ bool select_begin(KeyHist<NT>& h, Keys& k, uint32_t* xs32,
                                             const uint16_t* __restrict__ x, const TierArgs& a,
                                             int (&R)[2], Select (&sel)[2], int (&E)[2]) {
  constexpr int W = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int d = a.d;
  k.xs32 = xs32;
  k.C = ((d + W - 1) / W + 127) / 128 * 128;
  k.j0 = min(wave * k.C, d);
  k.n = min(k.j0 + k.C, d) - k.j0;
  k.steps = (k.n + 127) / 128;
  const bool thresholds = a.mode == SPAX_MODE_THRESHOLD;
  {
    // Every load of x in flight while the histogram is cleared, then x into LDS.
    constexpr int PER = (MAXD / 2 + NT - 1) / NT;
    const uint32_t* x32 = reinterpret_cast<const uint32_t*>(x);
    const int ndw = (d + 1) >> 1;
    uint32_t v[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) v[q] = tid + q * NT < ndw ? x32[tid + q * NT] : 0u;
    if (!thresholds) {
      const uint4 z = make_uint4(0u, 0u, 0u, 0u);
      uint4* f4 = reinterpret_cast<uint4*>(h.fine);
      for (int i = tid; i < 16384 / 4; i += NT) f4[i] = z;
      uint4* c4 = reinterpret_cast<uint4*>(h.coarse);
      for (int i = tid; i < 1024 / 4; i += NT) c4[i] = z;
    }
    if (tid < 4 * W) (&h.lists_q[0][0])[tid] = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q)
      if (tid + q * NT < ndw) xs32[tid + q * NT] = v[q];
    __builtin_amdgcn_s_waitcnt(0);  // see plan_stage1
  }
  __syncthreads();
  if (thresholds) {
    sel[0] = Select{a.k_full, d};
    sel[1] = Select{a.k_skip, d};
    E[0] = E[1] = 0;
    R[0] = R[1] = 0;
    return false;
  }
  int nat = 0;
  for (int s = 0; s < k.steps; ++s) {
    const uint32_t wd = k.word(s, lane);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const bool valid = k.valid(s, lane, e);
      const int key = (int)((e ? wd >> 16 : wd) & 0x7FFFu);
      // Unconditional (a zero increment past the range): a conditional LDS atomic makes the
      // compiler wait for every earlier LDS operation before it.  The coarse count is kept
      // by a second atomic rather than summed from the fine counters afterwards, which would
      // cost one more pass and one more barrier before the boundary search can start.
      atomicAdd(&h.fine[key >> 1], valid ? 1u << ((key & 1) << 4) : 0u);
      atomicAdd(&h.coarse[key >> 5], valid ? 1 : 0);
      nat += valid && key < a.k_tau;
    }
  }
  nat = wave_sum(nat);
  if (lane == 0) h.wave_nat[wave] = nat;
  __syncthreads();
  if (a.mode == SPAX_MODE_TOPK) {
    R[0] = a.n_full;
    R[1] = a.n_full + a.n_approx;
  } else {
    const int natural = wave_sum(lane < W ? h.wave_nat[lane] : 0);
    const int n_skip = min(max(natural, a.n_lo), a.n_hi);
    const int kept = d - n_skip;
    // num <= den <= 65535 and kept <= 32768: fits 32 bits
    const int n_approx = (int)(((uint32_t)a.num * (uint32_t)kept + (uint32_t)(a.den / 2)) /
                               (uint32_t)a.den);
    R[0] = kept - n_approx;
    R[1] = kept;
  }
  return true;
}

// The coarse bin cb (keys [32 cb, 32 cb + 32)) that holds the R-th largest key, R >= 1, and
// the number of keys above it.  One wave, after select_begin; the result is wave-uniform.
template <int NT>
__device__ __forceinline__ void coarse_find(const KeyHist<NT>& h, int R, int lane, int& cb,
                                            int& above) {
  int local[16];
  const int4* c4 = reinterpret_cast<const int4*>(h.coarse) + 4 * lane;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int4 v = c4[q];
    local[4 * q] = v.x;
    local[4 * q + 1] = v.y;
    local[4 * q + 2] = v.z;
    local[4 * q + 3] = v.w;
  }
  cb = 0;
  above = 0;
  suffix_find<16>(local, R, 0, lane, &cb, &above);
  cb = min(max(cb, 0), 1023);  // R <= d: always found
}

// Second part: waves 0 and 1 each find one boundary inside its coarse bin; every wave gets
// both (sel) and, for each, the number of channels whose key equals it (E).  Ends with a
// barrier.
template <int NT>
__device__ __forceinline__ void select_finish(KeyHist<NT>& h, const int (&R)[2],
                                              Select (&sel)[2], int (&E)[2]) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave < 2) {  // wave b finds boundary b
    const int b = wave;
    Select sb{0x8000, 0};
    int eb = 0;
    if (R[b] > 0) {
      int cb, above;
      coarse_find<NT>(h, R[b], lane, cb, above);
      const uint32_t dw = h.fine[16 * cb + ((lane & 31) >> 1)];
      const int cnt[1] = {lane < 32 ? (int)((dw >> ((lane & 1) << 4)) & 0xFFFFu) : 0};
      int v = 0, ab = 0;
      suffix_find<1>(cnt, R[b], above, lane, &v, &ab);
      v = min(max(v, 0), 31);
      sb = Select{32 * cb + v, R[b] - ab};
      eb = __builtin_amdgcn_readlane(cnt[0], v);
    }
    if (lane == 0) {
      h.sel[b] = sb;
      h.E[b] = eb;
    }
  }
  __syncthreads();
  sel[0] = h.sel[0];
  sel[1] = h.sel[1];
  E[0] = h.E[0];
  E[1] = h.E[1];
}

// Pass 3: FULL / APPROX channels go to emit_list(tier, rank, j, raw) with their rank in the
// ascending list; emit_tier(j, t_even, t_odd, n) sees each lane's pair of channels (j even,
// n = 2, or 1 when j + 1 is past the wave's range).  Only ranks in [f_lo, f_hi) (FULL) and
// [a_lo, a_hi) (APPROX) are wanted.  Unless every channel must reach emit_tier
// (all_channels), a wave whose rank ranges miss both windows does nothing, and a wave stops
// once it is past both (ranks grow with the channel index).  Uses build_plan's bases; no
// barrier.
template <int NT, class EmitList, class EmitTier>
__device__ __forceinline__ void emit(const Shared<NT>& sh, const Keys& k, const Plan& p,
                                     bool all_channels, int f_lo, int f_hi, int a_lo, int a_hi,
                                     EmitList emit_list, EmitTier emit_tier) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int fpos = sh.wave_base[wave][0], apos = sh.wave_base[wave][1];
  int eqb0 = sh.wave_base[wave][2], eqb1 = sh.wave_base[wave][3];
  const int f_end = sh.wave_base[wave + 1][0], a_end = sh.wave_base[wave + 1][1];
  const bool wantF = fpos < f_hi && f_end > f_lo && f_lo < f_hi;
  const bool wantA = apos < a_hi && a_end > a_lo && a_lo < a_hi;
  if (!all_channels && !wantF && !wantA) return;
  if (all_channels) f_hi = a_hi = INT_MAX;
  const Select s0 = p.s0, s1 = p.s1;
  // Within a step the order is lane-major: channel 2l, 2l+1, 2l+2, ...  so the channels before
  // (l, e) are both channels of lanes < l, plus the even channel of lane l if e = 1.
  for (int s = 0; s < k.steps && (fpos < f_hi || apos < a_hi); ++s) {
    const uint32_t wd = k.word(s, lane);
    const uint32_t raw0 = wd & 0xFFFFu, raw1 = wd >> 16;
    const bool v0 = k.valid(s, lane, 0), v1 = k.valid(s, lane, 1);
    const int key0 = v0 ? (int)(raw0 & 0x7FFFu) : -1;
    const int key1 = v1 ? (int)(raw1 & 0x7FFFu) : -1;
    bool f0, f1, a0, a1;
    const bool tie = key0 == s0.kb || key1 == s0.kb || key0 == s1.kb || key1 == s1.kb;
    if (__ballot(tie) == 0) {  // no boundary key in this step: plain comparisons
      f0 = key0 > s0.kb;
      f1 = key1 > s0.kb;
      a0 = !f0 && key0 > s1.kb;
      a1 = !f1 && key1 > s1.kb;
    } else {
      const uint64_t q0e = __ballot(key0 == s0.kb), q0o = __ballot(key1 == s0.kb);
      const uint64_t q1e = __ballot(key0 == s1.kb), q1o = __ballot(key1 == s1.kb);
      const int r0 = eqb0 + (int)lanes_below(q0e) + (int)lanes_below(q0o);  // ties before even
      const int r1 = eqb1 + (int)lanes_below(q1e) + (int)lanes_below(q1o);
      f0 = key0 > s0.kb || (key0 == s0.kb && r0 < s0.m);
      f1 = key1 > s0.kb || (key1 == s0.kb && r0 + (key0 == s0.kb) < s0.m);
      const bool k0 = key0 > s1.kb || (key0 == s1.kb && r1 < s1.m);
      const bool k1 = key1 > s1.kb || (key1 == s1.kb && r1 + (key0 == s1.kb) < s1.m);
      a0 = k0 && !f0;
      a1 = k1 && !f1;
      eqb0 += popc(q0e) + popc(q0o);
      eqb1 += popc(q1e) + popc(q1o);
    }
    const uint64_t bfe = __ballot(f0), bfo = __ballot(f1);
    const uint64_t bae = __ballot(a0), bao = __ballot(a1);
    const int fr = fpos + (int)lanes_below(bfe) + (int)lanes_below(bfo);
    const int ar = apos + (int)lanes_below(bae) + (int)lanes_below(bao);
    const int jb = k.j0 + k.off(s, lane, 0);
    if (f0) emit_list(SPAX_TIER_FULL, fr, jb, raw0);
    if (a0) emit_list(SPAX_TIER_APPROX, ar, jb, raw0);
    if (f1) emit_list(SPAX_TIER_FULL, fr + (int)f0, jb + 1, raw1);
    if (a1) emit_list(SPAX_TIER_APPROX, ar + (int)a0, jb + 1, raw1);
    if (v0) {
      const uint32_t t0 = f0 ? SPAX_TIER_FULL : a0 ? SPAX_TIER_APPROX : SPAX_TIER_SKIP;
      const uint32_t t1 = f1 ? SPAX_TIER_FULL : a1 ? SPAX_TIER_APPROX : SPAX_TIER_SKIP;
      emit_tier(jb, t0, t1, v1 ? 2 : 1);
    }
    fpos += popc(bfe) + popc(bfo);
    apos += popc(bae) + popc(bao);
  }
}

// A whole mask in one workgroup with its outputs in global memory: tier bytes (tier may be
// NULL), both ascending lists and the counts {n_full, n_approx, n_skip}.  Used by the
// stand-alone mask kernel, the writer workgroup of the fused decode kernel and the batched
// mask launch.  d <= MAXD.
template <int NT, int MAXD>
__device__ __forceinline__ void tiers_to_global(Shared<NT>& sh, uint32_t* xs32, const TierArgs& a,
                                                const uint16_t* __restrict__ x, uint8_t* tier,
                                                int32_t* full_idx, int32_t* approx_idx,
                                                int32_t* counts) {
  Keys k;
  const Plan p = build_plan<NT, MAXD>(sh, k, xs32, x, a);
  const bool tier_even = ((uintptr_t)tier & 1) == 0;  // channel pairs start at even j
  emit<NT>(
      sh, k, p, true, 0, INT_MAX, 0, INT_MAX,
      [&](int t, int rank, int j, uint32_t) {
        if (t == SPAX_TIER_FULL) full_idx[rank] = j;
        else approx_idx[rank] = j;
      },
      [&](int j, uint32_t t0, uint32_t t1, int n) {
        if (!tier) return;
        if (n == 2 && tier_even) *reinterpret_cast<uint16_t*>(tier + j) = (uint16_t)(t0 | t1 << 8);
        else {
          tier[j] = (uint8_t)t0;
          if (n == 2) tier[j + 1] = (uint8_t)t1;
        }
      });
  if (threadIdx.x == 0) {
    counts[0] = p.n_full;
    counts[1] = p.n_kept - p.n_full;
    counts[2] = a.d - p.n_kept;
  }
}

}  // namespace mask
}  // namespace spax
