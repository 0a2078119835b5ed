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
//   1. the per-key histogram (select_begin), after which two waves find the exact boundaries
//      (select_finish);
//   2. (tiers_to_global) per-wave counts of the keys above and equal to each boundary, from
//      which every wave derives its list and tie bases with scans over the waves;
//   3. emit: ranks from ballots plus those bases.
// The kernels are issue-bound inside one CU (every wave instruction competes with those of
// the other waves), so fixed per-wave work is kept small: two 16-bit counts share one 32-bit
// lane sum (a wave holds at most 2048 channels), and a step without boundary keys skips the
// tie ranking.
#pragma once

#include <climits>

#include "common.h"

namespace spax {
namespace mask {

struct Select {
  int32_t kb;  // boundary key
  int32_t m;   // channels with key == kb that are selected (lowest indices first)
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

// Workgroup barrier for LDS traffic: the fences order LDS operations only, so global loads
// still in flight stay in flight (a plain __syncthreads() also waits for every one of them).
// Every barrier of the mask code guards LDS data only.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

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

// Inclusive prefix sum within each row of 16 lanes (row shifts only).
__device__ __forceinline__ int row_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  return x;
}

// Largest value over the 64 lanes, as a wave-uniform value.
__device__ __forceinline__ int wave_max(int x) {
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x111, 0xF, 0xF, false));  // row_shr:1
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x112, 0xF, 0xF, false));  // row_shr:2
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x114, 0xF, 0xF, false));  // row_shr:4
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x118, 0xF, 0xF, false));  // row_shr:8
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x142, 0xA, 0xF, false));  // row_bcast:15
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return __builtin_amdgcn_readlane(x, 63);
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

// Exact selection: a radix select over the 15-bit keys with two digits (the high 10 bits,
// then the low 5), both digit histograms built in one pass of LDS atomics: 1024 counters of
// the high digit and 32768 16-bit per-key counters (two keys per dword; a count never exceeds
// 32768, so it cannot carry into its neighbour), the low-digit histogram of a high digit
// being its 32 key counters.  Then one wave finds each boundary with two suffix scans (high
// digit, then low digit).  Lanes collide in a per-key counter only on equal keys.
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
  // For tiers_to_global: per wave, (keys above | keys equal) << 16 for each boundary.
  int wave_cnt[W][2];
  Select sel[2];
  int E[2];
};

// Exact boundaries from a per-key histogram, in two parts (a caller may do other work in
// between).  select_begin loads x into LDS (xs32: roundup(d, 2) halves), sets k (the wave's
// channel range), builds the per-key histogram and the coarse one (32 keys per bin), and gives
// every wave the two target ranks R (FULL, kept; counted from the largest key).  For
// THRESHOLD the boundaries are the given keys: sel and E are set and false is returned.
// Both histograms are complete on return (its last barrier follows the last atomic).
// after_x(): called by every thread once x is in LDS, before the histogram pass; after_hist():
// once the thread has issued its histogram atomics, which the LDS then works through while the
// thread goes on (neither is called for THRESHOLD masks, whose boundaries are known at once).
struct NoHook {
  __device__ __forceinline__ void operator()() const {}
};
template <int NT, int MAXD, class AfterX = NoHook, class AfterHist = NoHook>
__device__ __forceinline__ bool select_begin(KeyHist<NT>& h, Keys& k, uint32_t* xs32,
                                             const uint16_t* __restrict__ x, const TierArgs& a,
                                             int (&R)[2], Select (&sel)[2], int (&E)[2],
                                             AfterX after_x = AfterX(),
                                             AfterHist after_hist = AfterHist()) {
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
    // Every load has landed: say so to the compiler's wait tracking, so that loads issued
    // after the mask passes are not made to wait for these conditional ones.
    __builtin_amdgcn_s_waitcnt(0);
  }
  lds_barrier();
  if (thresholds) {
    sel[0] = Select{a.k_full, d};
    sel[1] = Select{a.k_skip, d};
    E[0] = E[1] = 0;
    R[0] = R[1] = 0;
    return false;
  }
  after_x();
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
  after_hist();
  nat = wave_sum(nat);
  if (lane == 0) h.wave_nat[wave] = nat;
  lds_barrier();
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
// Lane l sums bins 16 l .. 16 l + 15; a scan over the lanes and one ballot find the lane whose
// bins hold rank R; then lanes 0..15 take that lane's bins, highest first, and a scan within
// the row of 16 and one more ballot find the bin.
template <int NT>
__device__ __forceinline__ void coarse_find(const KeyHist<NT>& h, int R, int lane, int& cb,
                                            int& above) {
  const int4* c4 = reinterpret_cast<const int4*>(h.coarse) + 4 * lane;
  int sum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int4 v = c4[q];
    sum += v.x + v.y + v.z + v.w;
  }
  const int pre = wave_scan(sum);
  const int run = __builtin_amdgcn_readlane(pre, 63) - pre;  // keys in the lanes above
  const uint64_t hit = __ballot(run < R && run + sum >= R);  // one lane: R <= d
  const int L = hit ? (int)__builtin_ctzll(hit) : 0;
  const int runL = __builtin_amdgcn_readlane(run, L);
  const int v = lane < 16 ? h.coarse[16 * L + 15 - lane] : 0;
  const int cum = row_scan(v);  // lane i: bins 16 L + 15 - i .. 16 L + 15
  const uint64_t in = __ballot(lane < 16 && runL + cum >= R);
  const int i = in ? (int)__builtin_ctzll(in) : 15;
  cb = 16 * L + 15 - i;
  above = runL + __builtin_amdgcn_readlane(cum - v, i);
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
  lds_barrier();
  sel[0] = h.sel[0];
  sel[1] = h.sel[1];
  E[0] = h.E[0];
  E[1] = h.E[1];
}

// A wave's first FULL and APPROX list positions, the ties at each boundary key before its
// first channel, and the end of its FULL and APPROX positions.
struct WaveBases {
  int fpos, apos, eqb0, eqb1, f_end, a_end;
};

// Pass 3: FULL / APPROX channels go to emit_list(tier, rank, j, raw) with their rank in the
// ascending list; emit_tier(j, t_even, t_odd, n) sees each lane's pair of channels (j even,
// n = 2, or 1 when j + 1 is past the wave's range).  Only ranks in [f_lo, f_hi) (FULL) and
// [a_lo, a_hi) (APPROX) are wanted.  Unless every channel must reach emit_tier
// (all_channels), a wave whose rank ranges miss both windows does nothing, and a wave stops
// once it is past both (ranks grow with the channel index).  No barrier.
template <class EmitList, class EmitTier>
__device__ __forceinline__ void emit(const WaveBases& b, const Keys& k, const Plan& p,
                                     bool all_channels, int f_lo, int f_hi, int a_lo, int a_hi,
                                     EmitList emit_list, EmitTier emit_tier) {
  const int lane = threadIdx.x & 63;
  int fpos = b.fpos, apos = b.apos, eqb0 = b.eqb0, eqb1 = b.eqb1;
  const int f_end = b.f_end, a_end = b.a_end;
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
// mask launch.  d <= MAXD.  The boundaries come from the per-key histogram (select_begin /
// select_finish); one counting pass gives every wave its keys above and equal to each
// boundary, one barrier publishes them, and every wave derives its list and tie bases with
// two scans over the waves before emit writes the lists.
template <int NT, int MAXD>
__device__ __forceinline__ void tiers_to_global(KeyHist<NT>& h, uint32_t* xs32, const TierArgs& a,
                                                const uint16_t* __restrict__ x, uint8_t* tier,
                                                int32_t* full_idx, int32_t* approx_idx,
                                                int32_t* counts) {
  constexpr int W = NT / 64;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  Keys k;
  int R[2], E[2];
  Select sel[2];
  if (select_begin<NT, MAXD>(h, k, xs32, x, a, R, sel, E)) select_finish<NT>(h, R, sel, E);
  const Select s0 = sel[0], s1 = sel[1];
  // counts of this wave's channels: (above | equal << 16) per boundary (a wave holds at most
  // 32768 / W channels, so each half fits 16 bits)
  uint32_t c0 = 0, c1 = 0;
  for (int s = 0; s < k.steps; ++s) {
    const uint32_t wd = k.word(s, lane);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int key = k.valid(s, lane, e) ? (int)((e ? wd >> 16 : wd) & 0x7FFFu) : -1;
      c0 += (key > s0.kb ? 1u : 0u) + (key == s0.kb ? 0x10000u : 0u);
      c1 += (key > s1.kb ? 1u : 0u) + (key == s1.kb ? 0x10000u : 0u);
    }
  }
  c0 = (uint32_t)wave_sum((int)c0);
  c1 = (uint32_t)wave_sum((int)c1);
  if (lane == 0) {
    h.wave_cnt[wave][0] = (int)c0;
    h.wave_cnt[wave][1] = (int)c1;
  }
  lds_barrier();
  // lane u < W holds wave u's counts; exclusive scans over the waves give the ties before
  // wave u, its FULL and kept counts, then its first list positions
  const uint32_t w0 = lane < W ? (uint32_t)h.wave_cnt[lane][0] : 0u;
  const uint32_t w1 = lane < W ? (uint32_t)h.wave_cnt[lane][1] : 0u;
  const int g0 = (int)(w0 & 0xFFFFu), e0 = (int)(w0 >> 16);
  const int g1 = (int)(w1 & 0xFFFFu), e1 = (int)(w1 >> 16);
  const int t0 = wave_scan(e0) - e0, t1 = wave_scan(e1) - e1;  // ties before wave u
  const int nf = g0 + min(max(s0.m - t0, 0), e0);
  const int nk = g1 + min(max(s1.m - t1, 0), e1);
  const int fb = wave_scan(nf) - nf, ab = wave_scan(nk - nf) - (nk - nf);
  WaveBases b;
  b.fpos = __builtin_amdgcn_readlane(fb, wave);
  b.apos = __builtin_amdgcn_readlane(ab, wave);
  b.eqb0 = __builtin_amdgcn_readlane(t0, wave);
  b.eqb1 = __builtin_amdgcn_readlane(t1, wave);
  b.f_end = b.fpos + __builtin_amdgcn_readlane(nf, wave);
  b.a_end = b.apos + __builtin_amdgcn_readlane(nk - nf, wave);
  Plan p;
  p.s0 = s0;
  p.s1 = s1;
  p.n_full = __builtin_amdgcn_readlane(fb + nf, W - 1);
  p.n_kept = p.n_full + __builtin_amdgcn_readlane(ab + nk - nf, W - 1);
  const bool tier_even = ((uintptr_t)tier & 1) == 0;  // channel pairs start at even j
  emit(
      b, k, p, true, 0, INT_MAX, 0, INT_MAX,
      [&](int t, int rank, int j, uint32_t) {
        if (t == SPAX_TIER_FULL) full_idx[rank] = j;
        else approx_idx[rank] = j;
      },
      [&](int j, uint32_t t0_, uint32_t t1_, int n) {
        if (!tier) return;
        if (n == 2 && tier_even) *reinterpret_cast<uint16_t*>(tier + j) = (uint16_t)(t0_ | t1_ << 8);
        else {
          tier[j] = (uint8_t)t0_;
          if (n == 2) tier[j + 1] = (uint8_t)t1_;
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
