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
  int32_t cap;       // LDS list entries per tier
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
  uint32_t* lF = reinterpret_cast<uint32_t*>(dyn + a.xs_bytes);
  uint32_t* lA = lF + a.cap;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const gemv::Shape& sh = a.sh;
  const int d = a.ta.d;
  // The last workgroup only writes the outputs of the mask; the others each own one
  // (row tile, column chunk) of the GEMV.
  const bool writer = blockIdx.x == gridDim.x - 1;

  // ---- mask (every workgroup)
  mask::Keys k;
  const mask::Plan p = mask::build_plan<kFusedThreads, MAXD>(msh, k, xs32, a.x, a.ta);
  const int nF = p.n_full, nA = p.n_kept - p.n_full;
  if (writer) {
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
      a.counts[0] = nF;
      a.counts[1] = nA;
      a.counts[2] = d - p.n_kept;
    }
    clear_next(a);
    return;
  }
  const int tile = (int)(blockIdx.x % (uint32_t)sh.n_tiles);
  const int chunk = (int)(blockIdx.x / (uint32_t)sh.n_tiles);
  const int fb = gemv::split_at(nF, chunk, sh.n_chunks);
  const int fe = gemv::split_at(nF, chunk + 1, sh.n_chunks);
  const int ab = gemv::split_at(nA, chunk, sh.n_chunks);
  const int ae = gemv::split_at(nA, chunk + 1, sh.n_chunks);
  // Only the waves whose ranks meet this chunk's slices take part.
  mask::emit<kFusedThreads>(
      msh, k, p, false, fb, fe, ab, ae,
      [&](int t, int rank, int j, uint32_t raw) {
        const uint32_t e = (uint32_t)j | (raw << 16);
        if (t == SPAX_TIER_FULL) {
          if (rank >= fb && rank < fe) lF[rank - fb] = e;
        } else {
          if (rank >= ab && rank < ae) lA[rank - ab] = e;
        }
      },
      [](int, uint32_t, uint32_t, int) {});
  __syncthreads();  // list slices complete; the mask scratch is dead from here on

  // ---- GEMV over this workgroup's slice
  const int T = sh.T;
  const int row0 = tile * kTileRows;
  const int row = row0 + lane * 8 < T ? row0 + lane * 8 : 0;
  int wfb, wfe, wab, wae;
  gemv::wave_range<kFusedWaves>(fb, fe, wave, wfb, wfe);
  gemv::wave_range<kFusedWaves>(ab, ae, wave, wab, wae);
  float acc[8];
#pragma unroll
  for (int h = 0; h < 8; ++h) acc[h] = 0.0f;
  float zsum = 0.0f;
  const uint32_t jmax = (uint32_t)d - 1u;
  gemv::stream_columns<FMT>(sh, a.packed, row, wfb, wfe, gemv::LdsList{lF, fb, jmax}, wab, wae,
                            gemv::LdsList{lA, ab, jmax}, acc, zsum);
  gemv::finish_tile<kFusedWaves>(u.red, acc, zsum, wave, lane, row0, T, sh.n_chunks, a.y);
  clear_next(a);
}

struct FusedLds {
  int32_t cap, xs_bytes;
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
// to 16), then the workgroup's two list slices.
FusedLds fused_lds(const spax_layout* L, const GemvPlan& plan) {
  FusedLds f;
  f.cap = (L->d_in + plan.n_chunks - 1) / plan.n_chunks;
  f.xs_bytes = (4 * ((L->d_in + 1) / 2) + 15) / 16 * 16;
  f.bytes = (size_t)f.xs_bytes + 8 * (size_t)f.cap;
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
    a.cap = f.cap;
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
