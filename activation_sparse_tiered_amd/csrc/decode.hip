// Decode step over a stack of projection groups.
//
// Pages: eigenradar commentary on SpAx, second and last paragraphs (selection per generated
// token during batch-one decoding); TopK-Guided (arXiv:2610.01763) section 2.1 (per-token
// mask, O(d)); ByteCross abstract (fixed kernel costs add to the byte account).
//
// Default: one fused kernel per group, at most one 1024-thread workgroup per compute unit.
// Every workgroup loads the activation vector into LDS and finds the two tier boundaries
// from a per-key histogram (mask_core.h, select_begin / select_finish), decides the tiers of
// its own range of input channels, lists those columns in LDS (channel | fp16 x_j << 16 per
// entry, one list per wave and tier, shared out among the waves) and streams them for its
// 512-row tile (gemv_core.h).  One extra workgroup writes the tier bytes, the ascending
// lists and the counts with the rank-producing mask code, so the outputs equal
// those of spax_build_tiers.  Repeating the boundary search in every workgroup costs no time
// (it runs in parallel on separate compute units) and removes the second launch and the
// counts -> indices -> activations chain of dependent global loads.  With
// SPAX_STEP_SEPARATE (and for inputs too wide for the fused kernel) a group takes the
// stand-alone mask kernel (tiers.hip, which also clears y) and the stand-alone GEMV
// (gemv.hip).
//
// y of a group is accumulated with fp32 atomics and must start at zero: the mask kernel (or,
// fused, the previous launch, spread over its workgroups) clears it; otherwise a small
// kernel does.
#include <atomic>
#include <climits>
#include <cstdlib>

#include "gemv_core.h"
#include "mask_core.h"

namespace spax {
namespace {

constexpr int kFusedThreads = 1024;
constexpr int kFusedWaves = kFusedThreads / 64;
// FULL fp16 columns per wave whose loads are issued before the mask completes (0: none).
// Not done for int4 columns: a quarter of the bytes per load did not repay the extra work
// on the mask's path (measured slower).
#ifndef SPAX_EARLY
#define SPAX_EARLY 4
#endif
template <int FMT>
struct Early {
  static constexpr bool use = FMT == SPAX_FMT_FP16 && SPAX_EARLY > 0;
  static constexpr int n = SPAX_EARLY > 0 ? SPAX_EARLY : 1;
};

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

// The next up to kUnroll entries of tier t (0 FULL, 1 APPROX) for this wave from the column
// lists of its workgroup: from its own list while that has entries left, else from the next
// wave's list (in wave order) that has.  q = KeyHist::lists_q; lane v reads wave v's counter
// and published length, so one look costs one LDS round trip.  A list not yet published
// looks used up (its owner streams it).  A claim is one LDS atomic on the list's counter, so
// every entry goes to exactly one wave; a claim that comes too late leaves that counter at
// or past the length, so the list drops out of the next look, and the loop ends after at
// most kFusedWaves such misses.  Returns the count (0: no work left) and sets `base`, the
// entry's index from the start of the lists (wave v's FULL list at 2 v S, its APPROX list at
// 2 v S + S).  Wave-uniform.
__device__ __forceinline__ int claim_entries(int (*q)[kFusedWaves], int t, int wave, int S,
                                             int lane, int& base) {
#pragma unroll 1
  for (int miss = 0; miss <= kFusedWaves; ++miss) {
    const int v_l = lane & (kFusedWaves - 1);
    const int c = __hip_atomic_load(&q[2 + t][v_l], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    const int seen = __hip_atomic_load(&q[t][v_l], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    const uint32_t m = (uint32_t)__ballot(lane < kFusedWaves && seen < c);  // wave v: bit v
    if (m == 0u) return 0;
    const uint32_t rot = ((m >> wave) | (m << (kFusedWaves - wave))) & 0xFFFFu;  // own wave first
    const int v = (wave + (int)__builtin_ctz(rot)) & (kFusedWaves - 1);
    const int cv = __builtin_amdgcn_readlane(c, v);
    int st = 0;
    if (lane == 0)
      st = __hip_atomic_fetch_add(&q[t][v], gemv::kUnroll, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_WORKGROUP);
    st = __builtin_amdgcn_readfirstlane(st);
    if (st < cv) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");  // the entries before the count
      base = v * 2 * S + t * S + st;
      return min(gemv::kUnroll, cv - st);
    }
  }
  return 0;
}

// How many of the two fp16 halves of an LDS word of x have key (bits & 0x7FFF) kb, where
// kb2 = kb in both halves; only the first nv (0, 1 or 2) halves count.  XOR with kb2 leaves
// a half zero exactly where the key equals kb (a key never has its top bit set).
__device__ __forceinline__ int equal_halves(uint32_t wd, uint32_t kb2, int nv) {
  const uint32_t t = (wd & 0x7FFF7FFFu) ^ kb2;
  return (nv > 0 && (t & 0xFFFFu) == 0u ? 1 : 0) + (nv > 1 && t < 0x10000u ? 1 : 0);
}

// Channels j in [begin, end) whose key is kb (begin even; eight keys per lane and LDS read).
// One wave; the result is wave-uniform.
__device__ __forceinline__ int ties_between(const uint32_t* xs32, int begin, int end, int kb,
                                            int lane) {
  const uint32_t kb2 = (uint32_t)kb * 0x10001u;
  int c = 0;
  const uint4* x4 = reinterpret_cast<const uint4*>(xs32);
  for (int base = begin; base < end; base += 512) {
    const int j = base + 8 * lane;
    if (j < end) {
      const uint4 v = x4[j >> 3];
      c += equal_halves(v.x, kb2, end - j) + equal_halves(v.y, kb2, end - j - 2) +
           equal_halves(v.z, kb2, end - j - 4) + equal_halves(v.w, kb2, end - j - 6);
    }
  }
  return mask::wave_sum(c);
}

// One group: mask and GEMV.  Workgroup gridDim.x - 1 only writes the outputs of the mask
// (build_plan + emit, as the stand-alone mask kernel).  Every other workgroup owns one
// 512-row tile and one contiguous range of input channels, split over its 16 waves:
//   1. the exact boundaries from a per-key histogram (select_begin / select_finish: one pass
//      over the keys); as soon as the coarse bin of the FULL boundary is known, the loads of
//      the wave's first few columns above that bin (FULL whatever the exact boundary) are
//      issued, so they are in flight while the boundaries are completed (fp16 columns);
//   2. each wave decides the tiers of its channels (ties at a boundary key by channel order,
//      counting the equal keys before its first channel only when it holds such a tie) and
//      lists its FULL and APPROX columns in LDS;
//   3. each wave multiplies its early columns, streams its own list and then takes columns
//      from the other waves' lists until all are done (claim_entries); the tile is reduced
//      across waves and added to y.
template <int FMT, int MAXD>
__global__ __launch_bounds__(kFusedThreads) void fused_phase_kernel(FusedArgs a) {
  extern __shared__ __align__(16) uint8_t dyn[];
  // The mask's scratch and the GEMV's cross-wave reduction are never live together.
  __shared__ union {
    mask::Shared<kFusedThreads> msh;
    mask::KeyHist<kFusedThreads> kh;
    float red[kFusedWaves][kTileRows];
  } u;
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
    mask::tiers_to_global<kFusedThreads, MAXD>(u.msh, xs32, a.ta, a.x, a.tier, a.full_idx,
                                               a.approx_idx, a.counts);
    clear_next(a);
    return;
  }

  const int item = gemv::xcd_order((int)blockIdx.x, (int)gridDim.x - 1);
  const int tile = (int)((uint32_t)item % (uint32_t)sh.n_tiles);
  const int chunk = (int)((uint32_t)item / (uint32_t)sh.n_tiles);
  const int c0 = gemv::split_at(d, chunk, sh.n_chunks);
  const int c1 = gemv::split_at(d, chunk + 1, sh.n_chunks);
  const int S = a.wave_cap;  // channels per wave
  const int ws = min(c0 + wave * S, c1), we = min(ws + S, c1);
  uint32_t* lF = reinterpret_cast<uint32_t*>(dyn + a.xs_bytes) + wave * 2 * S;
  uint32_t* lA = lF + S;
  const int T = sh.T;
  const int row0 = tile * kTileRows;
  const int row = row0 + lane * 8 < T ? row0 + lane * 8 : 0;
  const uint32_t jmax = (uint32_t)d - 1u;

  // ---- 1. boundaries, with the first FULL columns already on their way
  mask::Select sel[2];
  int E[2], R[2];
  const bool search = mask::select_begin<kFusedThreads, MAXD>(u.kh, k, xs32, a.x, a.ta, R, sel, E);
  // Keys >= kc are FULL wherever the exact boundary falls inside its coarse bin (THRESHOLD:
  // the boundary itself).  The loads of this wave's first kEarly such columns (channel order)
  // are issued now and stay in flight through the rest of the mask work.
  int kc = 0x8000;
  constexpr bool kUseEarly = Early<FMT>::use;
  constexpr int kEarly = Early<FMT>::n;
  if (!kUseEarly) {
  } else if (!search) {
    kc = sel[0].kb;
  } else if (R[0] > 0) {
    int cb, above;
    mask::coarse_find<kFusedThreads>(u.kh, R[0], lane, cb, above);
    kc = 32 * (cb + 1);
  }
  uint32_t pe[kEarly];
#pragma unroll
  for (int q = 0; q < kEarly; ++q) pe[q] = 0u;
  int np = 0;
  for (int j0 = ws; kUseEarly && j0 < we && np < kEarly; j0 += 64) {
    const int j = j0 + lane;
    const uint32_t raw = j < we ? (uint32_t)xs16[j] : 0u;
    uint64_t b = __ballot(j < we && (int)(raw & 0x7FFFu) >= kc);
    const uint32_t e = (uint32_t)j | (raw << 16);
    int taken = 0;
#pragma unroll
    for (int q = 0; q < kEarly; ++q) {
      if (q >= np && b != 0) {
        pe[q] = (uint32_t)__builtin_amdgcn_readlane((int)e, (int)__builtin_ctzll(b));
        b &= b - 1;
        ++taken;
      }
    }
    np += taken;
  }
#pragma unroll
  for (int q = 1; q < kEarly; ++q)
    if (q >= np) pe[q] = pe[q - 1];  // unused slots repeat a used column (or column 0)
  gemv::EarlyColumns<FMT, kEarly> early;
  if (kUseEarly) early.issue(sh, a.packed, row, pe, np, jmax);
  if (search) mask::select_finish<kFusedThreads>(u.kh, R, sel, E);
  const mask::Select s0 = sel[0], s1 = sel[1];

  // ---- 2. this wave's tiers and column lists
  bool need0 = s0.m < E[0], need1 = s1.m < E[1];  // the boundary keeps some of its ties only
  if (need0 || need1) {
    bool here0 = false, here1 = false;  // this wave holds a channel at that boundary key
    for (int j0 = ws; j0 < we; j0 += 64) {
      const int j = j0 + lane;
      const int key = j < we ? (int)(xs16[j] & 0x7FFFu) : -1;
      here0 |= __ballot(key == s0.kb) != 0;
      here1 |= __ballot(key == s1.kb) != 0;
    }
    need0 = need0 && here0;
    need1 = need1 && here1;
  }
  // Channels before ws at a split boundary key: counted by the few waves that hold such a
  // channel, each over x[0, ws) in LDS, so the others go on with no barrier.
  int ties0 = need0 ? ties_between(xs32, 0, ws, s0.kb, lane) : 0;
  int ties1 = need1 ? ties_between(xs32, 0, ws, s1.kb, lane) : 0;
  int nF = 0, nA = 0, ne = 0;
  for (int j0 = ws; j0 < we; j0 += 64) {
    const int j = j0 + lane;
    const bool v = j < we;
    const uint32_t raw = v ? (uint32_t)xs16[j] : 0u;
    const int key = v ? (int)(raw & 0x7FFFu) : -1;
    const bool t0 = key == s0.kb, t1 = key == s1.kb;
    const uint64_t b0 = __ballot(t0), b1 = __ballot(t1);
    const int r0 = ties0 + (int)mask::lanes_below(b0), r1 = ties1 + (int)mask::lanes_below(b1);
    // the early columns are the wave's first np channels with key >= kc
    const bool cand = key >= kc;
    const uint64_t bc = __ballot(cand);
    const bool is_early = cand && ne + (int)mask::lanes_below(bc) < np;
    ne += mask::popc(bc);
    const bool full = !is_early && (key > s0.kb || (t0 && (!need0 || r0 < s0.m)));
    const bool kept = key > s1.kb || (t1 && (!need1 || r1 < s1.m));
    const bool apx = kept && !full && !is_early;
    ties0 += mask::popc(b0);
    ties1 += mask::popc(b1);
    const uint32_t e = (uint32_t)j | (raw << 16);
    const uint64_t bf = __ballot(full), ba = __ballot(apx);
    if (full) lF[nF + (int)mask::lanes_below(bf)] = e;
    if (apx) lA[nA + (int)mask::lanes_below(ba)] = e;
    nF += mask::popc(bf);
    nA += mask::popc(ba);
  }
  wave_lds_fence();

  // ---- 3. stream, reduce
  float acc[8];
#pragma unroll
  for (int h = 0; h < 8; ++h) acc[h] = 0.0f;
  float zsum = 0.0f;
  if (kUseEarly) early.multiply(acc, zsum);
  // The waves' lists are shared out: a wave streams its own list and then helps the others,
  // so the workgroup ends with its average wave rather than its longest list.  A wave keeps
  // its first round for itself: its counters start past those entries and are set before
  // the lengths are published, so no claim is needed to start.  The entries are written
  // before the lengths (release); a claim reads a length before the entries (acquire).
  int nf = min(nF, gemv::kUnroll), na = min(nA, gemv::kUnroll);
  int bF = wave * 2 * S, bA = wave * 2 * S + S;
  if (lane == 0) {
    __hip_atomic_store(&u.kh.lists_q[0][wave], nf, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __hip_atomic_store(&u.kh.lists_q[1][wave], na, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  if (lane == 0) {
    __hip_atomic_store(&u.kh.lists_q[2][wave], nF, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __hip_atomic_store(&u.kh.lists_q[3][wave], nA, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  const uint32_t* lists = reinterpret_cast<const uint32_t*>(dyn + a.xs_bytes);
  const gemv::TileOffsets<FMT> g(sh, row);
  while (nf > 0 || na > 0) {
    gemv::RoundLoads<FMT> r;
    gemv::issue_round<FMT>(sh, a.packed, g, gemv::LdsBlock(lists + bF, nf, jmax), 0, nf,
                           gemv::LdsBlock(lists + bA, na, jmax), 0, na, r);
    // the next claims overlap this round's loads
    int nbF = bF, nbA = bA;
    const int nf2 = claim_entries(u.kh.lists_q, 0, wave, S, lane, nbF);
    const int na2 = claim_entries(u.kh.lists_q, 1, wave, S, lane, nbA);
    gemv::finish_round<FMT>(r, g, nf, na, acc, zsum);
    nf = nf2;
    na = na2;
    bF = nbF;
    bA = nbA;
  }
  __syncthreads();  // every wave is done with the mask scratch that `red` overlays
  gemv::finish_tile<kFusedWaves>(u.red, acc, zsum, wave, lane, row0, T, sh.n_chunks, a.y);
  clear_next(a);
}

struct FusedLds {
  int32_t wave_cap, xs_bytes;
  size_t bytes;
};

// Compute units of the current device (cached per device; calls from several host threads
// may fill an entry at once, with the same value).
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
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
// to 16), then for each wave a FULL and an APPROX list of wave_cap entries; wave_cap * 16 >=
// the channels of one chunk.
FusedLds fused_lds(const spax_layout* L, const GemvPlan& plan) {
  FusedLds f;
  const int range = (L->d_in + plan.n_chunks - 1) / plan.n_chunks;
  f.wave_cap = (range + kFusedWaves - 1) / kFusedWaves;
  f.xs_bytes = (4 * ((L->d_in + 1) / 2) + 15) / 16 * 16;
  f.bytes = (size_t)f.xs_bytes + kFusedWaves * 2 * 4 * (size_t)f.wave_cap;
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
  if (st->flags & SPAX_STEP_BATCHED) return launch_decode_step_batched(st, cu_count(), s);
  const int n = st->n_phases;
  const bool separate = (st->flags & SPAX_STEP_SEPARATE) != 0;
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
