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
// of 128.  Three passes over the wave's channels:
//   1. 256-bin histogram of the high key bits (LDS atomics), natural count;
//   2. (TopK boundaries) per-wave 128-bin histograms of the low bits inside the boundary
//      bucket, from which each wave gets its own "greater" / "equal" counts;
//   3. emit: ranks from ballots plus per-wave bases derived from those counts.
// One emit pass and no block-wide scan.
#pragma once

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
  // Level-1 histogram in 16 copies (one per lane & 15, odd stride so the copies of a bin
  // sit in different banks): lanes whose keys share a bin mostly hit different addresses.
  static constexpr int kCopies = 16, kStride = 257;
  int hist_rep[kCopies * kStride];
  int hist_hi[256];
  int wave_hist[2][W][128];
  int wave_cnt[W][6];  // natural, gt0, eq0, gt1, eq1, spare
  int sel_b[2], sel_above[2];
  Select sel[2];
};

// Channel layout: wave w owns channels [j0, j0 + n), j0 = w*C (C a multiple of 128); at step
// s, lane l handles the two adjacent channels j0 + 128 s + 2 l + {0, 1}, stored as one dword
// of raw fp16 bits (low half: even channel) in LDS, so every step is one conflict-free,
// coalesced 256-byte LDS read per wave.  The passes are rolled loops: the kernels run once per
// token, so their code is fetched cold and must stay small.
struct Keys {
  const uint32_t* xs32;  // LDS, d halves rounded up to dwords
  int C;                 // channels per wave (multiple of 128)
  int j0;                // first channel of this wave
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

// Load x into LDS (xs32: roundup(d, 2) halves), then passes 1 and 2 plus the selects.
// Leaves each wave's (gt, eq) counts against both boundaries in sh.wave_cnt.  Contains the
// barriers it needs and ends with one.  d <= MAXD.
template <int NT, int MAXD>
__device__ __forceinline__ Plan build_plan(Shared<NT>& sh, Keys& k, uint32_t* xs32,
                                           const uint16_t* __restrict__ x, const TierArgs& a) {
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

  // ---- x into LDS: every load of a thread in flight at once.  For odd d the last dword
  // also holds the two bytes past x (same dword, never used as a channel).
  {
    const uint32_t* x32 = reinterpret_cast<const uint32_t*>(x);
    const int ndw = (d + 1) >> 1;
    constexpr int PER = (MAXD / 2 + NT - 1) / NT;
    uint32_t v[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int i = tid + q * NT;
      v[q] = i < ndw ? x32[i] : 0u;
    }
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int i = tid + q * NT;
      if (i < ndw) xs32[i] = v[q];
    }
  }
  if (!thresholds) {
    for (int i = tid; i < Shared<NT>::kCopies * Shared<NT>::kStride; i += NT) sh.hist_rep[i] = 0;
    for (int i = tid; i < 2 * W * 128; i += NT) (&sh.wave_hist[0][0][0])[i] = 0;
  }
  __syncthreads();

  // ---- pass 1: high-bit histogram, natural count, threshold counts
  int nat = 0, gt0 = 0, eq0 = 0, gt1 = 0, eq1 = 0;
  for (int s = 0; s < k.steps; ++s) {
    const uint32_t wd = k.word(s, lane);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const bool valid = k.valid(s, lane, e);
      const int key = (int)((e ? wd >> 16 : wd) & 0x7FFFu);
      if (valid && !thresholds)
        atomicAdd(&sh.hist_rep[(lane & 15) * Shared<NT>::kStride + (key >> 7)], 1);
      nat += popc(__ballot(valid && key < a.k_tau));
      if (thresholds) {
        gt0 += popc(__ballot(valid && key > a.k_full));
        eq0 += popc(__ballot(valid && key == a.k_full));
        gt1 += popc(__ballot(valid && key > a.k_skip));
        eq1 += popc(__ballot(valid && key == a.k_skip));
      }
    }
  }
  if (lane == 0) {
    sh.wave_cnt[wave][0] = nat;
    sh.wave_cnt[wave][1] = gt0;
    sh.wave_cnt[wave][2] = eq0;
    sh.wave_cnt[wave][3] = gt1;
    sh.wave_cnt[wave][4] = eq1;
  }
  __syncthreads();

  Plan p;
  if (thresholds) {
    p.s0 = Select{a.k_full, d};
    p.s1 = Select{a.k_skip, d};
  } else {
    int natural = 0;
    for (int w = 0; w < W; ++w) natural += sh.wave_cnt[w][0];
    int R[2];
    if (a.mode == SPAX_MODE_TOPK) {
      R[0] = a.n_full;
      R[1] = a.n_full + a.n_approx;
    } else {
      const int n_skip = min(max(natural, a.n_lo), a.n_hi);
      const int kept = d - n_skip;
      // num <= den <= 65535 and kept <= 32768: fits 32 bits
      const int n_approx = (int)(((uint32_t)a.num * (uint32_t)kept + (uint32_t)(a.den / 2)) /
                                 (uint32_t)a.den);
      R[0] = kept - n_approx;
      R[1] = kept;
    }
    // ---- fold the histogram copies
    for (int b = tid; b < 256; b += NT) {
      int t = 0;
#pragma unroll
      for (int c = 0; c < Shared<NT>::kCopies; ++c) t += sh.hist_rep[c * Shared<NT>::kStride + b];
      sh.hist_hi[b] = t;
    }
    __syncthreads();
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
    const int b0 = sh.sel_b[0], b1 = sh.sel_b[1];
    // ---- pass 2: per-wave low-bit histograms inside the buckets; keys above the buckets
    int above0 = 0, above1 = 0;
    for (int s = 0; s < k.steps; ++s) {
      const uint32_t wd = k.word(s, lane);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const bool valid = k.valid(s, lane, e);
        const int key = (int)((e ? wd >> 16 : wd) & 0x7FFFu);
        const int hi = valid ? key >> 7 : -2;
        if (hi == b0) atomicAdd(&sh.wave_hist[0][wave][key & 127], 1);
        if (hi == b1) atomicAdd(&sh.wave_hist[1][wave][key & 127], 1);
        above0 += popc(__ballot(b0 >= 0 && hi > b0));
        above1 += popc(__ballot(b1 >= 0 && hi > b1));
      }
    }
    __syncthreads();
    // ---- level 2: exact boundary keys (waves 0 and 1 sum the per-wave histograms)
    if (wave < 2) {
      int local[2] = {0, 0};
      for (int w = 0; w < W; ++w) {
        local[0] += sh.wave_hist[wave][w][lane * 2];
        local[1] += sh.wave_hist[wave][w][lane * 2 + 1];
      }
      int v = -1, ab = 0;
      if (R[wave] > 0) suffix_find<2>(local, R[wave], sh.sel_above[wave], lane, &v, &ab);
      if (lane == 0)
        sh.sel[wave] =
            R[wave] > 0 ? Select{(sh.sel_b[wave] << 7) | v, R[wave] - ab} : Select{0x8000, 0};
    }
    __syncthreads();
    p.s0 = sh.sel[0];
    p.s1 = sh.sel[1];
    // ---- this wave's counts against the boundaries, from its own histograms
    const int low0 = p.s0.kb & 127, low1 = p.s1.kb & 127;
    const int c0a = sh.wave_hist[0][wave][lane * 2], c0b = sh.wave_hist[0][wave][lane * 2 + 1];
    const int c1a = sh.wave_hist[1][wave][lane * 2], c1b = sh.wave_hist[1][wave][lane * 2 + 1];
    const int G0 = wave_sum((lane * 2 > low0 ? c0a : 0) + (lane * 2 + 1 > low0 ? c0b : 0));
    const int E0 = wave_sum((lane * 2 == low0 ? c0a : 0) + (lane * 2 + 1 == low0 ? c0b : 0));
    const int G1 = wave_sum((lane * 2 > low1 ? c1a : 0) + (lane * 2 + 1 > low1 ? c1b : 0));
    const int E1 = wave_sum((lane * 2 == low1 ? c1a : 0) + (lane * 2 + 1 == low1 ? c1b : 0));
    if (lane == 0) {
      // R == 0: boundary above every key, nothing greater or equal
      sh.wave_cnt[wave][1] = R[0] > 0 ? above0 + G0 : 0;
      sh.wave_cnt[wave][2] = R[0] > 0 ? E0 : 0;
      sh.wave_cnt[wave][3] = R[1] > 0 ? above1 + G1 : 0;
      sh.wave_cnt[wave][4] = R[1] > 0 ? E1 : 0;
    }
    __syncthreads();
  }
  // totals: a wave's selected ties are clamp(m - ties before it, 0, its ties)
  int eqb0 = 0, eqb1 = 0;
  p.n_full = 0;
  p.n_kept = 0;
  for (int w = 0; w < W; ++w) {
    const int g0 = sh.wave_cnt[w][1], e0 = sh.wave_cnt[w][2];
    const int g1 = sh.wave_cnt[w][3], e1 = sh.wave_cnt[w][4];
    p.n_full += g0 + min(max(p.s0.m - eqb0, 0), e0);
    p.n_kept += g1 + min(max(p.s1.m - eqb1, 0), e1);
    eqb0 += e0;
    eqb1 += e1;
  }
  return p;
}

// Pass 3: every FULL / APPROX channel goes to emit_list(tier, rank, j, raw) with its rank
// in the ascending list; emit_tier(j, tier) sees every channel.  Uses the per-wave counts
// build_plan left in sh.wave_cnt; no barrier.
template <int NT, class EmitList, class EmitTier>
__device__ __forceinline__ void emit(const Shared<NT>& sh, const Keys& k, const Plan& p,
                                     EmitList emit_list, EmitTier emit_tier) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int eqb0 = 0, eqb1 = 0, fbase = 0, kbase = 0;
  for (int w = 0; w < wave; ++w) {
    const int g0 = sh.wave_cnt[w][1], e0 = sh.wave_cnt[w][2];
    const int g1 = sh.wave_cnt[w][3], e1 = sh.wave_cnt[w][4];
    fbase += g0 + min(max(p.s0.m - eqb0, 0), e0);
    kbase += g1 + min(max(p.s1.m - eqb1, 0), e1);
    eqb0 += e0;
    eqb1 += e1;
  }
  // FULL is a subset of kept, so APPROX before this wave = kept before - FULL before.
  // Within a step the order is lane-major: channel 2l, 2l+1, 2l+2, ...  so the channels
  // before (l, e) are both channels of lanes < l, plus the even channel of lane l if e = 1.
  int fpos = fbase, apos = kbase - fbase;
  const uint64_t lt = (1ull << lane) - 1ull;
  for (int s = 0; s < k.steps; ++s) {
    const uint32_t wd = k.word(s, lane);
    const uint32_t raw[2] = {wd & 0xFFFFu, wd >> 16};
    int key[2];
    bool val[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      val[e] = k.valid(s, lane, e);
      key[e] = val[e] ? (int)(raw[e] & 0x7FFFu) : -1;
    }
    const uint64_t q0e = __ballot(key[0] == p.s0.kb), q0o = __ballot(key[1] == p.s0.kb);
    const uint64_t q1e = __ballot(key[0] == p.s1.kb), q1o = __ballot(key[1] == p.s1.kb);
    const int r0 = eqb0 + popc(q0e & lt) + popc(q0o & lt);  // ties before the even channel
    const int r1 = eqb1 + popc(q1e & lt) + popc(q1o & lt);
    bool isF[2], isA[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int t0 = r0 + (e ? (key[0] == p.s0.kb) : 0);
      const int t1 = r1 + (e ? (key[0] == p.s1.kb) : 0);
      isF[e] = key[e] > p.s0.kb || (key[e] == p.s0.kb && t0 < p.s0.m);
      const bool kept = key[e] > p.s1.kb || (key[e] == p.s1.kb && t1 < p.s1.m);
      isA[e] = kept && !isF[e];
    }
    eqb0 += popc(q0e) + popc(q0o);
    eqb1 += popc(q1e) + popc(q1o);
    const uint64_t bfe = __ballot(isF[0]), bfo = __ballot(isF[1]);
    const uint64_t bae = __ballot(isA[0]), bao = __ballot(isA[1]);
    const int fr = fpos + popc(bfe & lt) + popc(bfo & lt);
    const int ar = apos + popc(bae & lt) + popc(bao & lt);
    const int jb = k.j0 + k.off(s, lane, 0);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int fe = fr + (e ? (int)isF[0] : 0);
      const int ae = ar + (e ? (int)isA[0] : 0);
      if (isF[e]) emit_list(SPAX_TIER_FULL, fe, jb + e, raw[e]);
      if (isA[e]) emit_list(SPAX_TIER_APPROX, ae, jb + e, raw[e]);
      if (val[e]) emit_tier(jb + e, isF[e] ? SPAX_TIER_FULL : isA[e] ? SPAX_TIER_APPROX : SPAX_TIER_SKIP);
    }
    fpos += popc(bfe) + popc(bfo);
    apos += popc(bae) + popc(bao);
  }
}

}  // namespace mask
}  // namespace spax
