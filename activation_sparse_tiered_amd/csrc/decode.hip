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
// 512-row tile (gemv_core.h).  With fp16 bases each wave also loads the FULL records of its
// largest-key channels while the histogram is being built, and multiplies them only if the
// mask makes them FULL.  One extra workgroup writes the tier bytes, the ascending
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
  float* partials;   // deterministic mode: chunk c's tile goes to partials[c][...] (NULL: atomics)
  int32_t own_only;  // deterministic mode: each wave streams only its own lists
  float4* y_next;    // cleared as a side job (NULL: none)
  int32_t n_next4;   // float4s of y_next
  int32_t per_next;  // float4s cleared per workgroup
  int32_t n_spec;    // FULL columns per wave loaded before the mask is known (0..kUnroll)
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
// 2 v S + S).  Wave-uniform.  own_only: only the wave's own list is looked at, so which
// wave adds which column (and so the rounding of the tile) does not depend on timing.
__device__ __forceinline__ int claim_entries(int (*q)[kFusedWaves], int t, int wave, int S,
                                             int lane, int& base, bool own_only) {
#pragma unroll 1
  for (int miss = 0; miss <= kFusedWaves; ++miss) {
    const int v_l = lane & (kFusedWaves - 1);
    const int c = __hip_atomic_load(&q[2 + t][v_l], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    const int seen = __hip_atomic_load(&q[t][v_l], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    uint32_t m = (uint32_t)__ballot(lane < kFusedWaves && seen < c);  // wave v: bit v
    if (own_only) m &= 1u << wave;
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

// Bit 15 of each half of the result set where that half of w (two fp16 activations) has key
// (bits & 0x7FFF) kb, with kb2 = kb in both halves.  t = key ^ kb leaves a half zero exactly
// where the key equals kb, and since both lie below 0x8000 a half h of t is zero exactly when
// h - 1 (a packed 16-bit subtract: no borrow between the halves) has bit 15 set.
__device__ __forceinline__ uint32_t equal_bits(uint32_t w, uint32_t kb2) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  const uint32_t t = (w & 0x7FFF7FFFu) ^ kb2;
  const u16x2 one = {1, 1};
  const uint32_t dm = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, t) - one);
  return dm & ~t & 0x80008000u;
}

// Eight activations (a 16-byte LDS read): how many have key kb0 (bits 0..15 of the result)
// and kb1 (bits 16..31).  keep: the halves that count (bit 15 of each).
__device__ __forceinline__ uint32_t equal8(const uint4& v, uint32_t kb2_0, uint32_t kb2_1,
                                           const uint4& keep) {
  return (uint32_t)(__builtin_popcount(equal_bits(v.x, kb2_0) & keep.x) +
                    __builtin_popcount(equal_bits(v.y, kb2_0) & keep.y) +
                    __builtin_popcount(equal_bits(v.z, kb2_0) & keep.z) +
                    __builtin_popcount(equal_bits(v.w, kb2_0) & keep.w)) +
         ((uint32_t)(__builtin_popcount(equal_bits(v.x, kb2_1) & keep.x) +
                     __builtin_popcount(equal_bits(v.y, kb2_1) & keep.y) +
                     __builtin_popcount(equal_bits(v.z, kb2_1) & keep.z) +
                     __builtin_popcount(equal_bits(v.w, kb2_1) & keep.w))
          << 16);
}

// Channels j in [0, end) whose key is kb0, and those whose key is kb1 (eight keys per lane and
// LDS read; whole 512-channel blocks read four at a time with no bounds, so four reads are
// in flight).  One wave; the results are wave-uniform.
__device__ __forceinline__ void ties_before(const uint32_t* xs32, int end, int kb0, int kb1,
                                            int lane, int& t0, int& t1) {
  const uint32_t k0 = (uint32_t)kb0 * 0x10001u, k1 = (uint32_t)kb1 * 0x10001u;
  const uint4 all = make_uint4(0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u);
  const uint4* x4 = reinterpret_cast<const uint4*>(xs32);
  const int full = end & ~511;
  uint32_t c = 0;  // kb0 in bits 0..15, kb1 in 16..31: each count is at most 16384
  int base = 0;
  for (; base + 2048 <= full; base += 2048) {
    uint4 v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = x4[(base >> 3) + 64 * q + lane];
#pragma unroll
    for (int q = 0; q < 4; ++q) c += equal8(v[q], k0, k1, all);
  }
  for (; base < full; base += 512) c += equal8(x4[(base >> 3) + lane], k0, k1, all);
  const int j = base + 8 * lane;
  if (j < end) {  // the last, partial block: only the first end - j halves count
    const int n = end - j;
    const uint4 keep = make_uint4((n > 0 ? 0x8000u : 0u) | (n > 1 ? 0x80000000u : 0u),
                                  (n > 2 ? 0x8000u : 0u) | (n > 3 ? 0x80000000u : 0u),
                                  (n > 4 ? 0x8000u : 0u) | (n > 5 ? 0x80000000u : 0u),
                                  (n > 6 ? 0x8000u : 0u) | (n > 7 ? 0x80000000u : 0u));
    c += equal8(x4[j >> 3], k0, k1, keep);
  }
  c = (uint32_t)mask::wave_sum((int)c);
  t0 = (int)(c & 0xFFFFu);
  t1 = (int)(c >> 16);
}

// Multiplies the speculatively loaded FULL fp16 columns of r whose slot bit is set in ok (the
// others proved not to be FULL and are dropped unread).  Waits for every load first.
template <int FMT>
__device__ __forceinline__ void finish_spec(const gemv::RoundLoads<FMT>& r, uint32_t ok,
                                            float (&acc)[8]) {
  __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
  for (int u = 0; u < gemv::kUnroll; ++u)
    if ((ok >> u) & 1u) gemv::fma_fp16x8(acc, r.xf[u], r.vf[u]);
}

// One group: mask and GEMV.  Workgroup gridDim.x - 1 only writes the outputs of the mask
// (tiers_to_global, as the stand-alone mask kernel).  Every other workgroup owns one
// 512-row tile and one contiguous range of input channels, split over its 16 waves:
//   1. the exact boundaries from a per-key histogram (select_begin / select_finish: one pass
//      over the keys);
//   1a. (fp16 bases) while the histogram is built, each wave already loads the FULL records
//      of the n_spec largest keys among its first 64 channels (the memory system is otherwise
//      idle until the boundaries are known); they are multiplied only once the mask confirms
//      them FULL;
//   2. each wave decides the tiers of its channels (ties at a boundary key by channel order,
//      counting the equal keys before its first channel only when it holds such a tie) and
//      lists its FULL and APPROX columns in LDS, leaving out the confirmed speculative ones;
//   3. each wave streams its own list and then takes columns from the other waves' lists
//      until all are done (claim_entries; in deterministic mode a wave keeps to its own
//      list); the tile is reduced across waves and added to y (deterministic mode: stored
//      as the chunk's partial sums).
// (Issuing each wave's first FULL columns as soon as the FULL boundary's coarse bin was known,
// before the exact boundaries, measured 0.55% slower per token: the selection and the issue
// lengthened every wave's path to the boundary search more than the early bytes saved.)
template <int FMT, int MAXD, class Blob>
__global__ __launch_bounds__(kFusedThreads) void fused_phase_kernel(FusedArgs a) {
  extern __shared__ __align__(16) uint8_t dyn[];
  // The mask's scratch and the GEMV's cross-wave reduction are never live together.
  __shared__ union {
    mask::KeyHist<kFusedThreads> kh;
    float red[kFusedWaves][kTileRows];
  } u;
  static_assert(sizeof(float) * kFusedWaves * kTileRows <= sizeof(u.kh.fine),
                "the reduction buffer must lie inside the per-key counters");
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
    mask::tiers_to_global<kFusedThreads, MAXD>(u.kh, xs32, a.ta, a.x, a.tier, a.full_idx,
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
  const gemv::TileOffsets<FMT> g(sh, row);
  const Blob blob(sh, a.packed);

  // ---- 1. boundaries
  mask::Select sel[2];
  int E[2], R[2];
  // ---- 1a. speculative FULL columns: slot i holds channel ws + sl[i]
  gemv::RoundLoads<FMT> r0;
  int sl[gemv::kUnroll] = {};
  int n_sp = 0;
  uint64_t picked = 0;  // lanes of the first 64 channels whose column was loaded
  // this lane's channel of the wave's first 64, read before the histogram pass (LDS reads
  // after it would queue behind the atomics)
  int key = -1;
  uint32_t raw = 0;
  auto spec_keys = [&]() {
    if (FMT != SPAX_FMT_FP16 || a.n_spec <= 0) return;
    const int j = ws + lane;
    raw = j < we ? (uint32_t)xs16[j] : 0u;
    key = j < we ? (int)(raw & 0x7FFFu) : -1;
  };
  // Chosen and issued once the wave's histogram atomics are issued: the LDS works through
  // those meanwhile.
  auto speculate = [&]() {
    if (FMT != SPAX_FMT_FP16 || a.n_spec <= 0 || ws >= we) return;
#pragma unroll
    for (int i = 0; i < gemv::kUnroll; ++i) {
      sl[i] = 0;
      r0.xf[i] = 0.0f;
      if (i >= a.n_spec) continue;
      const int m = mask::wave_max(key);
      if (m < 0) continue;
      const int l = (int)__builtin_ctzll(__ballot(key == m));
      if (lane == l) key = -1;
      sl[i] = l;
      picked |= 1ull << l;
      n_sp = i + 1;
      const int jc = ws + l;
      r0.xf[i] = gemv::half_lo((uint32_t)__builtin_amdgcn_readlane((int)raw, l));
      r0.vf[i] = blob.full(jc).stream128(g.loffF);
    }
  };
  const bool search =
      mask::select_begin<kFusedThreads, MAXD>(u.kh, k, xs32, a.x, a.ta, R, sel, E, spec_keys,
                                              speculate);
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
  int ties0 = 0, ties1 = 0;
  if (need0 || need1) ties_before(xs32, ws, s0.kb, s1.kb, lane, ties0, ties1);
  int nF = 0, nA = 0;
  uint64_t spec_full = 0;  // lanes whose speculatively loaded column is FULL
  for (int j0 = ws; j0 < we; j0 += 64) {
    const int j = j0 + lane;
    const bool v = j < we;
    const uint32_t raw = v ? (uint32_t)xs16[j] : 0u;
    const int key = v ? (int)(raw & 0x7FFFu) : -1;
    const bool t0 = key == s0.kb, t1 = key == s1.kb;
    const uint64_t b0 = __ballot(t0), b1 = __ballot(t1);
    const int rk0 = ties0 + (int)mask::lanes_below(b0), rk1 = ties1 + (int)mask::lanes_below(b1);
    const bool full = key > s0.kb || (t0 && (!need0 || rk0 < s0.m));
    const bool kept = key > s1.kb || (t1 && (!need1 || rk1 < s1.m));
    const bool apx = kept && !full;
    const bool sp = j0 == ws && ((picked >> lane) & 1u);
    if (j0 == ws) spec_full = __ballot(sp && full);
    const bool listF = full && !sp;
    ties0 += mask::popc(b0);
    ties1 += mask::popc(b1);
    const uint32_t e = (uint32_t)j | (raw << 16);
    const uint64_t bf = __ballot(listF), ba = __ballot(apx);
    if (listF) lF[nF + (int)mask::lanes_below(bf)] = e;
    if (apx) lA[nA + (int)mask::lanes_below(ba)] = e;
    nF += mask::popc(bf);
    nA += mask::popc(ba);
  }
  uint32_t spec_ok = 0;  // slots to multiply
#pragma unroll
  for (int i = 0; i < gemv::kUnroll; ++i)
    if (i < n_sp && ((spec_full >> sl[i]) & 1u)) spec_ok |= 1u << i;
  wave_lds_fence();

  // ---- 3. stream, reduce
  float acc[8];
#pragma unroll
  for (int h = 0; h < 8; ++h) acc[h] = 0.0f;
  float zsum = 0.0f;
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
  const bool own_only = a.own_only != 0;
  bool spec_pending = n_sp > 0;
  while (nf > 0 || na > 0) {
    gemv::RoundLoads<FMT> r;
    gemv::issue_round<FMT>(blob, g, gemv::LdsBlock(lists + bF, nf, jmax), 0, nf,
                           gemv::LdsBlock(lists + bA, na, jmax), 0, na, r);
    // the next claims overlap this round's loads
    int nbF = bF, nbA = bA;
    const int nf2 = claim_entries(u.kh.lists_q, 0, wave, S, lane, nbF, own_only);
    const int na2 = claim_entries(u.kh.lists_q, 1, wave, S, lane, nbA, own_only);
    gemv::finish_round<FMT>(r, g, nf, na, acc, zsum);
    if (spec_pending) {  // landed long ago; multiplied after the first round's wait
      finish_spec<FMT>(r0, spec_ok, acc);
      spec_pending = false;
    }
    nf = nf2;
    na = na2;
    bF = nbF;
    bA = nbA;
  }
  if (spec_pending) finish_spec<FMT>(r0, spec_ok, acc);
  // `red` overlays only the per-key counters, which no wave reads after select_finish's last
  // barrier (the claim counters lie past them), so no barrier is needed before it is written.
  gemv::finish_tile<kFusedWaves>(u.red, acc, zsum, wave, lane, row0, T, sh.n_chunks, a.y,
                                 a.partials, chunk);
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
  // More workgroups than compute units measured slower (a second resident workgroup per CU
  // shares its LDS and issue slots with the first).
  const int wgs = cu_count() - 1;  // one more writes the mask outputs
  int k = wgs / p.n_tiles;
  const int kmax = L->d_in / 16 > 1 ? L->d_in / 16 : 1;
  if (k > kmax) k = kmax;
  if (k < 1) k = 1;
  p.n_chunks = k;
  p.ws_bytes = 0;
  return p;
}

// Speculative FULL columns per wave: half the FULL channels the fewest a mask can select would
// put among a wave's first 64 channels, at most kUnroll (so the largest keys there are almost
// always FULL); none for threshold masks, whose boundaries need no search, and none for int4
// bases, whose 4-byte code loads per lane save less time than choosing the columns costs
// (measured 4.9% slower per token).
int spec_columns(const TierArgs& ta, int wave_cap, int32_t base_fmt) {
  if (base_fmt != SPAX_FMT_FP16) return 0;
  int64_t fmin = 0;
  if (ta.mode == SPAX_MODE_TOPK) {
    fmin = ta.n_full;
  } else if (ta.mode == SPAX_MODE_TOPK_GUIDED) {
    const int64_t kept = (int64_t)ta.d - ta.n_hi;
    fmin = kept - ((int64_t)ta.num * kept + ta.den / 2) / ta.den;
  } else {
    return 0;
  }
  const int64_t n = fmin * (wave_cap < 64 ? wave_cap : 64) / (2 * (int64_t)ta.d);
  return n < 0 ? 0 : (n > gemv::kUnroll ? gemv::kUnroll : (int)n);
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

}  // namespace

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || !na || !nb) return false;
  const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
  return pa < pb + nb && pb < pa + na;
}

bool phase_touches(const spax_phase& ph, const void* p, size_t n) {
  const spax_layout* L = ph.layout;
  const size_t d = (size_t)L->d_in;
  return overlaps(ph.x, 4 * ((d + 1) / 2), p, n) || overlaps(ph.tier, d, p, n) ||
         overlaps(ph.full_idx, 4 * d, p, n) || overlaps(ph.approx_idx, 4 * d, p, n) ||
         overlaps(ph.counts, 12, p, n) || overlaps(ph.packed, (size_t)L->total_bytes, p, n) ||
         overlaps(ph.y, 4 * (size_t)L->d_out_total, p, n);
}

bool fused_phase_ok(const spax_layout* L) {
  if (L->d_in > kFusedMaxDin) return false;
  return fused_lds(L, fused_plan(L)).bytes <= kFusedMaxDynLds;
}

size_t deterministic_workspace_bytes(const spax_phase* phases, int32_t n_phases) {
  size_t mx = 0;
  for (int i = 0; i < n_phases; ++i) {
    const spax_layout* L = phases[i].layout;
    // either launch form may run the phase
    for (const GemvPlan& p : {gemv_plan(L), fused_phase_ok(L) ? fused_plan(L) : gemv_plan(L)}) {
      if (p.n_chunks < 2) continue;
      const size_t b = (size_t)p.n_chunks * (size_t)L->d_out_total * 4;
      if (b > mx) mx = b;
    }
  }
  return mx;
}

int launch_decode_step(const spax_step* st, hipStream_t s, bool noalloc) {
  if (st->flags & SPAX_STEP_BATCHED)
    return noalloc ? launch_decode_step_batched_static(st, cu_count(), s)
                   : launch_decode_step_batched(st, cu_count(), s);
  const int n = st->n_phases;
  const bool separate = (st->flags & SPAX_STEP_SEPARATE) != 0;
  // Deterministic mode: every phase's column chunks store their partial sums in the workspace
  // (reused phase after phase in stream order) and one more launch adds them in chunk order;
  // y is then never cleared or added to atomically.
  float* partials =
      (st->flags & SPAX_STEP_DETERMINISTIC) ? static_cast<float*>(st->ws) : nullptr;
  auto fused_phase_ok = [&](const spax_layout* L) { return !separate && spax::fused_phase_ok(L); };
  auto plan_of = [&](const spax_layout* L) { return fused_phase_ok(L) ? fused_plan(L) : gemv_plan(L); };
  // Launch i clears the y of phase i + 1 as a side job only when phase i is one fused launch,
  // phase i + 1 accumulates through atomics, and that y shares no byte with anything phase i
  // reads or writes: under stream order phase i + 1 may reuse phase i's buffers, and its y
  // must not be zeroed while launch i still uses them.  Otherwise phase i + 1 clears its own
  // y with a kernel right before its launch.
  auto clears_next = [&](int i) {
    if (i + 1 >= n || partials) return false;
    const spax_phase& nx = st->phases[i + 1];
    return fused_phase_ok(st->phases[i].layout) && plan_of(nx.layout).n_chunks > 1 &&
           !phase_touches(st->phases[i], nx.y, 4 * (size_t)nx.layout->d_out_total);
  };
  for (int i = 0; i < n; ++i) {
    const spax_phase& ph = st->phases[i];
    const spax_layout* L = ph.layout;
    TierArgs ta;
    tier_args_from_params(&ph.params, L->d_in, &ta);
    const GemvPlan plan = plan_of(L);
    // Was this group's y cleared by the previous launch?
    bool cleared = i > 0 && clears_next(i - 1);
    if (!fused_phase_ok(L)) {
      // Large input vectors: stand-alone mask kernel (which clears y) + GEMV.
      const bool clear_in_mask =
          plan.n_chunks > 1 && L->d_out_total <= kMaskClearMax && !cleared && !partials;
      if (plan.n_chunks > 1 && !cleared && !clear_in_mask && !partials) {
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
                              ph.y, cleared || clear_in_mask, s, false, partials);
      if (rc) return rc;
      if (st->events) SPAX_HIP_CHECK(hipEventRecord(st->events[2 * i + 1], s));
      continue;
    }
    if (plan.n_chunks > 1 && !cleared && !partials) {
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
    a.partials = plan.n_chunks > 1 ? partials : nullptr;
    a.own_only = partials != nullptr;
    a.y_next = nullptr;
    a.n_next4 = 0;
    if (clears_next(i)) {
      const spax_phase& nx = st->phases[i + 1];
      a.y_next = reinterpret_cast<float4*>(nx.y);
      a.n_next4 = (int32_t)((nx.layout->d_out_total + 3) / 4);  // rows <= 2^24
    }
    const FusedLds f = fused_lds(L, plan);
    a.wave_cap = f.wave_cap;
    a.xs_bytes = f.xs_bytes;
    a.n_spec = spec_columns(ta, f.wave_cap, L->base_fmt);
    const dim3 grid((unsigned)(plan.n_tiles * plan.n_chunks + 1));  // + the writer
    a.per_next = (a.n_next4 + (int32_t)grid.x - 1) / (int32_t)grid.x;
    const dim3 blk(kFusedThreads);
    const bool fp16 = L->base_fmt == SPAX_FMT_FP16;
    if (narrow_regions(L)) {
      if (fp16)
        hipLaunchKernelGGL((fused_phase_kernel<SPAX_FMT_FP16, kFusedMaxDin, gemv::RegionBlob>),
                           grid, blk, f.bytes, s, a);
      else
        hipLaunchKernelGGL((fused_phase_kernel<SPAX_FMT_INT4, kFusedMaxDin, gemv::RegionBlob>),
                           grid, blk, f.bytes, s, a);
    } else {
      if (fp16)
        hipLaunchKernelGGL((fused_phase_kernel<SPAX_FMT_FP16, kFusedMaxDin, gemv::RecordBlob>),
                           grid, blk, f.bytes, s, a);
      else
        hipLaunchKernelGGL((fused_phase_kernel<SPAX_FMT_INT4, kFusedMaxDin, gemv::RecordBlob>),
                           grid, blk, f.bytes, s, a);
    }
    SPAX_HIP_CHECK(hipGetLastError());
    if (st->events) SPAX_HIP_CHECK(hipEventRecord(st->events[2 * i + 1], s));
    if (a.partials) {
      int rc = launch_reduce_chunks(partials, plan.n_chunks, L->d_out_total, ph.y, s);
      if (rc) return rc;
    }
  }
  return SPAX_OK;
}

}  // namespace spax
