// Decode step over a stack of projection groups.
//
// Pages: eigenradar commentary on SpAx, second and last paragraphs (selection per generated
// token during batch-one decoding); TopK-Guided (arXiv:2610.01763) section 2.1 (per-token
// mask, O(d)); ByteCross abstract (fixed kernel costs add to the byte account).
//
// Default: per group, the stand-alone mask kernel (tiers.hip, which also clears y) and then
// the stand-alone GEMV (gemv.hip).  With SPAX_STEP_FUSED_MASK, a group's mask and its GEMV
// run in one kernel of at most one 1024-thread workgroup per compute unit: every workgroup
// loads the activation vector into LDS, finds the two tier boundaries and ranks the channels
// (mask_core.h), keeps only the slice of the FULL / APPROX lists its column chunk needs
// (channel | fp16 x_j << 16 per LDS entry), then streams those columns for its 512-row tile
// (gemv_core.h).  One extra workgroup writes the tier bytes, the ascending lists and the
// counts, so the outputs equal those of spax_build_tiers.  The mask is repeated once per
// compute unit, in parallel, in place of a second launch and of the counts -> indices ->
// activations chain of dependent global loads; the rank pass runs only in the waves whose
// ranks meet the workgroup's slices.  The mask is bound by vector-instruction issue inside
// one CU (a wave64 instruction occupies a SIMD for 4 cycles), so skipped waves shorten it.
//
// y of a group is accumulated with fp32 atomics and must start at zero: the mask kernel (or,
// fused, the previous launch, spread over its workgroups) clears it; otherwise a small
// kernel does.
#include <climits>
#include <cstdlib>

#include "gemv_core.h"
#include "mask_core.h"

namespace spax {
namespace {

constexpr int kFusedThreads = 1024;
constexpr int kFusedWaves = kFusedThreads / 64;

struct FusedArgs {
  TierArgs ta;
  gemv::Shape sh;
  const uint8_t* packed;
  const uint16_t* x;
  uint8_t* tier;
  int32_t* full_idx;
  int32_t* approx_idx;
  int32_t* counts;
  float* y;
  float4* y_next;    // cleared as a side job (NULL: none)
  int32_t n_next4;   // float4s of y_next
  int32_t per_next;  // float4s cleared per workgroup
  int32_t wave_cap;  // LDS list entries per wave and tier (>= its channels)
  int32_t xs_bytes;  // LDS bytes of the activations (lists follow)
};

// Side job: clear this workgroup's slice of the next group's output.  Issued at the end, so
// that no wait for this kernel's loads includes these stores.
__device__ __forceinline__ void clear_next(const FusedArgs& a) {
  if (!a.y_next) return;
  const int b = (int)blockIdx.x * a.per_next;
  const int e = min(b + a.per_next, a.n_next4);
  for (int i = b + (int)threadIdx.x; i < e; i += kFusedThreads)
    a.y_next[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// Wave-local LDS ordering: lanes read entries that other lanes of the same wave wrote.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Tier decisions for one wave's candidate list (entries channel | x bits << 16, ascending
// channel).  `ties` counts the channels before the list's first channel whose key equals the
// boundary key (only needed when the boundary keeps some but not all of its ties).  The first
// kFirst entries get bit 15 set when used; the used entries after them are compacted to
// positions kFirst, kFirst + 1, ...  (in place: a write never passes the entries still to be
// read).  Returns the number of compacted entries.  FULL list: use = FULL; APPROX list:
// use = kept and not FULL.
#ifndef SPAX_FUSED_FIRST
#define SPAX_FUSED_FIRST 8
#endif
constexpr int kFirst = SPAX_FUSED_FIRST;

template <bool kApprox>
__device__ __forceinline__ int decide(uint32_t* list, int n, const mask::Plan& p, bool need0,
                                      bool need1, int ties0, int ties1, int lane) {
  int used = 0;
  for (int i0 = 0; i0 < n; i0 += 64) {
    const int i = i0 + lane;
    const bool v = i < n;
    const uint32_t e = v ? list[i] : 0u;
    const int key = (int)((e >> 16) & 0x7FFFu);
    const bool t0 = v && key == p.s0.kb, t1 = v && key == p.s1.kb;
    const uint64_t b0 = __ballot(t0), b1 = __ballot(t1);
    const int r0 = ties0 + (int)mask::lanes_below(b0), r1 = ties1 + (int)mask::lanes_below(b1);
    const bool full = key > p.s0.kb || (t0 && (!need0 || r0 < p.s0.m));
    bool use;
    if (kApprox) {
      const bool kept = key > p.s1.kb || (t1 && (!need1 || r1 < p.s1.m));
      use = v && kept && !full;
    } else {
      use = v && full;
    }
    ties0 += mask::popc(b0);
    ties1 += mask::popc(b1);
    const uint64_t bu = __ballot(use && i >= kFirst);
    if (v && i < kFirst) list[i] = e | (use ? 0x8000u : 0u);
    if (use && i >= kFirst) list[kFirst + used + (int)mask::lanes_below(bu)] = e;
    used += mask::popc(bu);
  }
  return used;
}

// One group: mask and GEMV.  Workgroup gridDim.x - 1 only writes the outputs of the mask
// (build_plan + emit, as the stand-alone mask kernel).  Every other workgroup owns one
// 512-row tile and one contiguous range of input channels, split over its 16 waves:
//   1. stage 1 of the mask (x to LDS, high-bit histogram, level-1 buckets);
//   2. each wave lists its channels that may still be FULL (key >= L0) or APPROX
//      (L1 <= key <= U0) and issues the loads of its first kFirst columns of each list;
//   3. stage 2 of the mask (exact boundaries) runs while those loads are in flight;
//   4. the tier decisions (ties by channel order) mark or compact the lists; the loaded
//      columns that are used are multiplied, the rest of the used columns streamed.
// A candidate that ends up unused costs its load but adds nothing.
template <int FMT, int MAXD>
__global__ __launch_bounds__(kFusedThreads) void fused_phase_kernel(FusedArgs a) {
  extern __shared__ __align__(16) uint8_t dyn[];
  // The mask's scratch and the GEMV's cross-wave reduction are never live together.
  __shared__ union {
    mask::Shared<kFusedThreads> msh;
    float red[kFusedWaves][kTileRows];
  } u;
  mask::Shared<kFusedThreads>& msh = u.msh;
  uint32_t* xs32 = reinterpret_cast<uint32_t*>(dyn);
  const uint16_t* xs16 = reinterpret_cast<const uint16_t*>(dyn);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const gemv::Shape& sh = a.sh;
  const int d = a.ta.d;
  mask::Keys k;

  if (blockIdx.x == gridDim.x - 1) {
    // ---- writer: tier bytes, ascending lists, counts
    const mask::Plan p = mask::build_plan<kFusedThreads, MAXD>(msh, k, xs32, a.x, a.ta);
    const bool tier_even = ((uintptr_t)a.tier & 1) == 0;  // channel pairs start at even j
    mask::emit<kFusedThreads>(
        msh, k, p, true, 0, INT_MAX, 0, INT_MAX,
        [&](int t, int rank, int j, uint32_t) {
          if (t == SPAX_TIER_FULL) a.full_idx[rank] = j;
          else a.approx_idx[rank] = j;
        },
        [&](int j, uint32_t t0, uint32_t t1, int n) {
          if (!a.tier) return;
          if (n == 2 && tier_even) *reinterpret_cast<uint16_t*>(a.tier + j) = (uint16_t)(t0 | t1 << 8);
          else {
            a.tier[j] = (uint8_t)t0;
            if (n == 2) a.tier[j + 1] = (uint8_t)t1;
          }
        });
    if (tid == 0) {
      a.counts[0] = p.n_full;
      a.counts[1] = p.n_kept - p.n_full;
      a.counts[2] = d - p.n_kept;
    }
    clear_next(a);
    return;
  }

  const int tile = (int)(blockIdx.x % (uint32_t)sh.n_tiles);
  const int chunk = (int)(blockIdx.x / (uint32_t)sh.n_tiles);
  const int c0 = gemv::split_at(d, chunk, sh.n_chunks);
  const int c1 = gemv::split_at(d, chunk + 1, sh.n_chunks);
  const int S = a.wave_cap;
  const int ws = min(c0 + wave * S, c1), we = min(ws + S, c1);  // this wave's channels
  uint32_t* lF = reinterpret_cast<uint32_t*>(dyn + a.xs_bytes) + wave * S;
  uint32_t* lA = lF + kFusedWaves * S;
  const int T = sh.T;
  const int row0 = tile * kTileRows;
  const int row = row0 + lane * 8 < T ? row0 + lane * 8 : 0;
  const uint32_t jmax = (uint32_t)d - 1u;

  // ---- 1. mask stage 1
  mask::plan_stage1<kFusedThreads, MAXD>(msh, k, xs32, a.x, a.ta);
  const mask::Interval iv = mask::intervals(msh, a.ta);

  // ---- 2. candidate lists and the first loads
  int nFc = 0, nAc = 0;
  for (int j0 = ws; j0 < we; j0 += 64) {
    const int j = j0 + lane;
    const bool v = j < we;
    const uint32_t raw = v ? (uint32_t)xs16[j] : 0u;
    const int key = (int)(raw & 0x7FFFu);
    const bool fc = v && key >= iv.L0;
    const bool ac = v && key >= iv.L1 && key <= iv.U0;
    const uint64_t bf = __ballot(fc), ba = __ballot(ac);
    const uint32_t e = (uint32_t)j | (raw << 16);
    if (fc) lF[nFc + (int)mask::lanes_below(bf)] = e;
    if (ac) lA[nAc + (int)mask::lanes_below(ba)] = e;
    nFc += mask::popc(bf);
    nAc += mask::popc(ba);
  }
  wave_lds_fence();
  const int nf1 = min(nFc, kFirst), na1 = min(nAc, kFirst);
  float xf[kFirst], xa[kFirst];
  uint4 vf[kFirst];
  uint32_t cf[kFirst], sf[kFirst], ca[kFirst], sa[kFirst];
  {
    const gemv::LdsList LF{lF, 0, jmax}, LA{lA, 0, jmax};
    const uint8_t* regionA = a.packed + sh.off_A;
    const uint32_t loffF = FMT == SPAX_FMT_FP16 ? (uint32_t)row * 2u : (uint32_t)row / 2u;
    const uint32_t szoffF = (uint32_t)(T / 2) + (uint32_t)(row / sh.base_group) * 4u;
    const uint32_t loffA4 = ((uint32_t)row / 4u) & ~3u;
    const uint32_t szoffA = (uint32_t)(T / 4) + (uint32_t)(row / sh.approx_group) * 4u;
#pragma unroll
    for (int q = 0; q < kFirst; ++q) {
      if (q < nf1) {
        int j;
        LF.get(q, j, xf[q]);
        const uint8_t* col = a.packed + (int64_t)j * sh.stride_F;
        if (FMT == SPAX_FMT_FP16) {
          vf[q] = *reinterpret_cast<const uint4*>(col + loffF);
        } else {
          cf[q] = *reinterpret_cast<const uint32_t*>(col + loffF);
          sf[q] = *reinterpret_cast<const uint32_t*>(col + szoffF);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kFirst; ++q) {
      if (q < na1) {
        int j;
        LA.get(q, j, xa[q]);
        const uint8_t* col = regionA + (int64_t)j * sh.stride_A;
        ca[q] = *reinterpret_cast<const uint32_t*>(col + loffA4);
        sa[q] = *reinterpret_cast<const uint32_t*>(col + szoffA);
      }
    }
  }

  // ---- 3. mask stage 2 (exact boundaries, tie bases)
  const mask::Plan p = mask::plan_stage2<kFusedThreads>(msh, k, a.ta);

  // ---- 4. decisions.  Ties before this wave's first channel: the tie count before its
  // mask wave (layout of the mask passes) plus a count up to ws.
  constexpr int kW = kFusedWaves;
  const bool need0 = p.s0.m < msh.wave_base[kW][2];  // the FULL boundary splits its ties
  const bool need1 = p.s1.m < msh.wave_base[kW][3];
  int ties0 = 0, ties1 = 0;
  if ((need0 || need1) && ws < we) {
    const int gw = ws / k.C;
    ties0 = msh.wave_base[gw][2];
    ties1 = msh.wave_base[gw][3];
    for (int j0 = gw * k.C; j0 < ws; j0 += 64) {
      const int j = j0 + lane;
      const int key = j < ws ? (int)(xs16[j] & 0x7FFFu) : -1;
      ties0 += mask::popc(__ballot(key == p.s0.kb));
      ties1 += mask::popc(__ballot(key == p.s1.kb));
    }
  }
  const int nUF = decide<false>(lF, nFc, p, need0, need1, ties0, ties1, lane);
  const int nUA = decide<true>(lA, nAc, p, need0, need1, ties0, ties1, lane);
  wave_lds_fence();

  // ---- 5. GEMV: the columns already loaded, then the remaining used ones
  float acc[8];
#pragma unroll
  for (int h = 0; h < 8; ++h) acc[h] = 0.0f;
  float zsum = 0.0f;
  const uint32_t shA = (((uint32_t)row / 4u) & 2u) * 8u;
#pragma unroll
  for (int q = 0; q < kFirst; ++q) {
    if (q < nf1 && (__builtin_amdgcn_readfirstlane(lF[q]) & 0x8000u)) {
      if (FMT == SPAX_FMT_FP16) {
        gemv::fma_fp16x8(acc, xf[q], vf[q]);
      } else {
        gemv::fma_int4x8(acc, xf[q] * gemv::half_lo(sf[q]), cf[q]);
        zsum = fmaf(xf[q], gemv::half_hi(sf[q]), zsum);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < kFirst; ++q) {
    if (q < na1 && (__builtin_amdgcn_readfirstlane(lA[q]) & 0x8000u)) {
      gemv::fma_int2x8(acc, xa[q] * gemv::half_lo(sa[q]), ca[q] >> shA);
      zsum = fmaf(xa[q], gemv::half_hi(sa[q]), zsum);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // the first loads are all consumed or dropped
  gemv::stream_columns<FMT>(sh, a.packed, row, kFirst, kFirst + nUF, gemv::LdsList{lF, 0, jmax},
                            kFirst, kFirst + nUA, gemv::LdsList{lA, 0, jmax}, acc, zsum);
  __syncthreads();  // every wave is done with the mask scratch that `red` overlays
  gemv::finish_tile<kFusedWaves>(u.red, acc, zsum, wave, lane, row0, T, sh.n_chunks, a.y);
  clear_next(a);
}

struct FusedLds {
  int32_t wave_cap, xs_bytes;
  size_t bytes;
};

// Compute units of the current device (cached per device).
int cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// Fused grid: the 512-row tiles times as many column chunks as fill one workgroup per
// compute unit (at least 16 input channels per chunk), plus the writer workgroup.
GemvPlan fused_plan(const spax_layout* L) {
  GemvPlan p{};
  const int64_t T = L->d_out_total;
  p.n_tiles = (int32_t)((T + kTileRows - 1) / kTileRows);
  static const int target = [] {
    const char* v = getenv("SPAX_FUSED_WGS");
    return v ? atoi(v) : 0;
  }();
  const int wgs = (target > 1 ? target : cu_count()) - 1;  // one more writes the mask outputs
  int k = wgs / p.n_tiles;
  const int kmax = L->d_in / 16 > 1 ? L->d_in / 16 : 1;
  if (k > kmax) k = kmax;
  if (k < 1) k = 1;
  p.n_chunks = k;
  p.ws_bytes = 0;
  return p;
}

// Dynamic LDS: the activations (d_in halves rounded up to whole dwords, in bytes, rounded
// to 16), then per wave a FULL and an APPROX candidate list of wave_cap entries each
// (wave_cap * 16 >= the channels of one chunk).
FusedLds fused_lds(const spax_layout* L, const GemvPlan& plan) {
  FusedLds f;
  const int range = (L->d_in + plan.n_chunks - 1) / plan.n_chunks;
  f.wave_cap = (range + kFusedWaves - 1) / kFusedWaves;
  f.xs_bytes = (4 * ((L->d_in + 1) / 2) + 15) / 16 * 16;
  f.bytes = (size_t)f.xs_bytes + 2 * kFusedWaves * 4 * (size_t)f.wave_cap;
  return f;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
  return pa < pb + nb && pb < pa + na;
}

}  // namespace

bool fused_phase_ok(const spax_layout* L) {
  if (L->d_in > kFusedMaxDin) return false;
  return fused_lds(L, fused_plan(L)).bytes <= kFusedMaxDynLds;
}

int launch_decode_step(const spax_step* st, hipStream_t s) {
  const int n = st->n_phases;
  const bool separate = (st->flags & SPAX_STEP_FUSED_MASK) == 0;
  auto fused_phase_ok = [&](const spax_layout* L) { return !separate && spax::fused_phase_ok(L); };
  for (int i = 0; i < n; ++i) {
    const spax_phase& ph = st->phases[i];
    const spax_layout* L = ph.layout;
    TierArgs ta;
    tier_args_from_params(&ph.params, L->d_in, &ta);
    const GemvPlan plan = fused_phase_ok(L) ? fused_plan(L) : gemv_plan(L);
    const size_t ybytes = (size_t)L->d_out_total * 4;
    // Was this group's y cleared by the previous launch?
    bool cleared = false;
    if (i > 0) {
      const spax_phase& pp = st->phases[i - 1];
      cleared = fused_phase_ok(pp.layout) && plan.n_chunks > 1 &&
                !overlaps(pp.y, (size_t)pp.layout->d_out_total * 4, ph.y, ybytes);
    }
    if (!fused_phase_ok(L)) {
      // Large input vectors: stand-alone mask kernel (which clears y) + GEMV.
      const bool clear_in_mask = plan.n_chunks > 1 && L->d_out_total <= kMaskClearMax && !cleared;
      if (plan.n_chunks > 1 && !cleared && !clear_in_mask) {
        int rc = launch_zero_f32(ph.y, L->d_out_total, s);
        if (rc) return rc;
        cleared = true;
      }
      int rc = launch_build_tiers(ta, ph.x, ph.tier, ph.full_idx, ph.approx_idx, ph.counts,
                                  clear_in_mask ? ph.y : nullptr,
                                  clear_in_mask ? L->d_out_total : 0, s);
      if (rc) return rc;
      if (st->events) SPAX_HIP_CHECK(hipEventRecord(st->events[2 * i], s));
      rc = launch_tiered_gemv(L, plan, ph.packed, ph.x, ph.full_idx, ph.approx_idx, ph.counts,
                              ph.y, cleared || clear_in_mask, s);
      if (rc) return rc;
      if (st->events) SPAX_HIP_CHECK(hipEventRecord(st->events[2 * i + 1], s));
      continue;
    }
    if (plan.n_chunks > 1 && !cleared) {
      int rc = launch_zero_f32(ph.y, L->d_out_total, s);
      if (rc) return rc;
    }
    if (st->events) SPAX_HIP_CHECK(hipEventRecord(st->events[2 * i], s));
    FusedArgs a{};
    a.ta = ta;
    a.sh = gemv_shape(L, plan);
    a.packed = static_cast<const uint8_t*>(ph.packed);
    a.x = ph.x;
    a.tier = ph.tier;
    a.full_idx = ph.full_idx;
    a.approx_idx = ph.approx_idx;
    a.counts = ph.counts;
    a.y = ph.y;
    a.y_next = nullptr;
    a.n_next4 = 0;
    if (i + 1 < n) {
      const spax_phase& nx = st->phases[i + 1];
      const GemvPlan np = fused_phase_ok(nx.layout) ? fused_plan(nx.layout) : gemv_plan(nx.layout);
      if (np.n_chunks > 1 && !overlaps(ph.y, ybytes, nx.y, (size_t)nx.layout->d_out_total * 4)) {
        a.y_next = reinterpret_cast<float4*>(nx.y);
        a.n_next4 = (int32_t)((nx.layout->d_out_total + 3) / 4);  // rows <= 2^24
      }
    }
    const FusedLds f = fused_lds(L, plan);
    a.wave_cap = f.wave_cap;
    a.xs_bytes = f.xs_bytes;
    const dim3 grid((unsigned)(plan.n_tiles * plan.n_chunks + 1));  // + the writer
    a.per_next = (a.n_next4 + (int32_t)grid.x - 1) / (int32_t)grid.x;
    const dim3 blk(kFusedThreads);
    if (L->base_fmt == SPAX_FMT_FP16)
      hipLaunchKernelGGL((fused_phase_kernel<SPAX_FMT_FP16, kFusedMaxDin>), grid, blk, f.bytes, s, a);
    else
      hipLaunchKernelGGL((fused_phase_kernel<SPAX_FMT_INT4, kFusedMaxDin>), grid, blk, f.bytes, s, a);
    SPAX_HIP_CHECK(hipGetLastError());
    if (st->events) SPAX_HIP_CHECK(hipEventRecord(st->events[2 * i + 1], s));
  }
  return SPAX_OK;
}

}  // namespace spax
