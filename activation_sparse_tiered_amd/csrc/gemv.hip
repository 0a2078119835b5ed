// Tiered gather-GEMV: y = sum_{j in FULL} x_j W[:, j] + sum_{j in APPROX} x_j What[:, j].
//
// Pages: SpAx Abstract (arXiv:2610.02598) -- three read options per weight; eigenradar
// commentary on SpAx, "The route outside GPU memory" -- per-column tiers, two-bit
// approximations reconstructed on the GPU ("reconstructing two-bit approximations also
// consumes GPU time", third paragraph).  This is a batch-one GEMV: every selected byte is
// used for exactly one multiply-add, so the kernel is bound by HBM bandwidth and does not
// use MFMA.
//
// Work decomposition.  Rows are cut into tiles of 512 (one 64-lane wavefront, 8 rows per
// lane).  A workgroup of 8 wavefronts owns one row tile and one chunk of each selected-
// column list (split-K); its waves split the chunk and stream their columns:
//   FULL fp16  : one 16-byte load per lane per column (8 halves), fp32 FMA;
//   FULL int4  : one 4-byte load of 8 nibbles + the group's (s, z) word;
//   APPROX 2b  : one 2-byte load of 8 two-bit codes + the group's (s, z) word.
// The zero-point term of a quantized column is the same for the lane's 8 rows (a group is
// at least 64 rows), so it is accumulated once per column into `zsum` and added at the end:
//   x_j (s q + z) = (x_j s) q + x_j z.
// Column indices and activations are wave-uniform scalar loads; column bases are formed in
// scalar registers and the lane offset rides in a vector register.
//
// Reduction.  Waves add through LDS; the chunks of one tile meet in y through hardware fp32
// atomic adds at device scope (y is zeroed first, in stream order).  A fence-based "last
// workgroup reduces" scheme was measured slower by two orders of magnitude: a device-scope
// fence writes back and invalidates the L2 of the caller's XCD.  The order in which chunks
// land is not fixed, so y may differ in the last bits between runs; masks and lists are
// bit-exact.
#include "common.h"

namespace spax {
namespace {

constexpr int kWaves = kGemvThreads / 64;
constexpr int kUnroll = 8;

__device__ __forceinline__ float half_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float half_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Activation j as fp32 from a wave-uniform index (scalar dword load + half select).
__device__ __forceinline__ float load_x(const uint32_t* __restrict__ x32, int j) {
  const uint32_t w = x32[j >> 1];
  return (j & 1) ? half_hi(w) : half_lo(w);
}

__device__ __forceinline__ void fma_fp16x8(float (&acc)[8], float xv, const uint4& v) {
  acc[0] = fmaf(xv, half_lo(v.x), acc[0]);
  acc[1] = fmaf(xv, half_hi(v.x), acc[1]);
  acc[2] = fmaf(xv, half_lo(v.y), acc[2]);
  acc[3] = fmaf(xv, half_hi(v.y), acc[3]);
  acc[4] = fmaf(xv, half_lo(v.z), acc[4]);
  acc[5] = fmaf(xv, half_hi(v.z), acc[5]);
  acc[6] = fmaf(xv, half_lo(v.w), acc[6]);
  acc[7] = fmaf(xv, half_hi(v.w), acc[7]);
}

// 8 int4 codes (row 2k low nibble) scaled by a.
__device__ __forceinline__ void fma_int4x8(float (&acc)[8], float a, uint32_t c) {
  const uint32_t lo = c & 0x0F0F0F0Fu;          // rows 0,2,4,6 in bytes 0..3
  const uint32_t hi = (c >> 4) & 0x0F0F0F0Fu;   // rows 1,3,5,7
  acc[0] = fmaf(a, (float)(lo & 0xFFu), acc[0]);
  acc[1] = fmaf(a, (float)(hi & 0xFFu), acc[1]);
  acc[2] = fmaf(a, (float)((lo >> 8) & 0xFFu), acc[2]);
  acc[3] = fmaf(a, (float)((hi >> 8) & 0xFFu), acc[3]);
  acc[4] = fmaf(a, (float)((lo >> 16) & 0xFFu), acc[4]);
  acc[5] = fmaf(a, (float)((hi >> 16) & 0xFFu), acc[5]);
  acc[6] = fmaf(a, (float)(lo >> 24), acc[6]);
  acc[7] = fmaf(a, (float)(hi >> 24), acc[7]);
}

// 8 two-bit codes (row 4k+i in bits [2i+1:2i] of byte k) scaled by a.
__device__ __forceinline__ void fma_int2x8(float (&acc)[8], float a, uint32_t c) {
  const uint32_t t0 = c & 0x0303u;          // rows 0 (byte 0) and 4 (byte 1)
  const uint32_t t1 = (c >> 2) & 0x0303u;   // rows 1, 5
  const uint32_t t2 = (c >> 4) & 0x0303u;   // rows 2, 6
  const uint32_t t3 = (c >> 6) & 0x0303u;   // rows 3, 7
  acc[0] = fmaf(a, (float)(t0 & 0xFFu), acc[0]);
  acc[4] = fmaf(a, (float)(t0 >> 8), acc[4]);
  acc[1] = fmaf(a, (float)(t1 & 0xFFu), acc[1]);
  acc[5] = fmaf(a, (float)(t1 >> 8), acc[5]);
  acc[2] = fmaf(a, (float)(t2 & 0xFFu), acc[2]);
  acc[6] = fmaf(a, (float)(t2 >> 8), acc[6]);
  acc[3] = fmaf(a, (float)(t3 & 0xFFu), acc[3]);
  acc[7] = fmaf(a, (float)(t3 >> 8), acc[7]);
}

struct GemvShape {
  int64_t stride_F, stride_A, off_A;
  int32_t T, n_tiles, n_chunks;
  int32_t approx_group, base_group;
  int32_t d_in;
};

template <int FMT>
__global__ __launch_bounds__(kGemvThreads) void tiered_gemv_kernel(
    GemvShape sh, const uint8_t* __restrict__ packed, const uint32_t* __restrict__ x32,
    const int32_t* __restrict__ full_idx, const int32_t* __restrict__ approx_idx,
    const int32_t* __restrict__ counts, float* __restrict__ y) {
  __shared__ float red[kWaves][kTileRows];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile = blockIdx.x % sh.n_tiles;
  const int chunk = blockIdx.x / sh.n_tiles;
  const int T = sh.T;
  const int row0 = tile * kTileRows;
  // Lanes past the last row (ragged last tile) read the record's first rows instead, which
  // is always in bounds; their sums land in rows >= T and are never stored.
  const int row = row0 + lane * 8 < T ? row0 + lane * 8 : 0;

  // Counts and indices come from device memory; they are clamped so that even malformed
  // lists cannot address outside the blob (the result is then unspecified).
  const int nF = min(max(counts[0], 0), sh.d_in);
  const int nA = min(max(counts[1], 0), sh.d_in);
  const uint32_t jmax = (uint32_t)sh.d_in - 1u;
  const int fb = (int)((int64_t)nF * chunk / sh.n_chunks);
  const int fe = (int)((int64_t)nF * (chunk + 1) / sh.n_chunks);
  const int ab = (int)((int64_t)nA * chunk / sh.n_chunks);
  const int ae = (int)((int64_t)nA * (chunk + 1) / sh.n_chunks);
  const int wfb = fb + (fe - fb) * wave / kWaves;
  const int wfe = fb + (fe - fb) * (wave + 1) / kWaves;
  const int wab = ab + (ae - ab) * wave / kWaves;
  const int wae = ab + (ae - ab) * (wave + 1) / kWaves;

  float acc[8];
#pragma unroll
  for (int h = 0; h < 8; ++h) acc[h] = 0.0f;
  float zsum = 0.0f;

  // ------------------------------------------------------------ FULL tier
  if (FMT == SPAX_FMT_FP16) {
    const uint32_t loff = (uint32_t)row * 2u;
    int i = wfb;
    for (; i + kUnroll <= wfe; i += kUnroll) {
      int idx[kUnroll];
      float xv[kUnroll];
      uint4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) idx[u] = (int)min((uint32_t)full_idx[i + u], jmax);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const uint8_t* col = packed + (int64_t)idx[u] * sh.stride_F;
        v[u] = *reinterpret_cast<const uint4*>(col + loff);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) xv[u] = load_x(x32, idx[u]);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) fma_fp16x8(acc, xv[u], v[u]);
    }
    for (; i < wfe; ++i) {
      const int j = (int)min((uint32_t)full_idx[i], jmax);
      const uint8_t* col = packed + (int64_t)j * sh.stride_F;
      const uint4 v = *reinterpret_cast<const uint4*>(col + loff);
      fma_fp16x8(acc, load_x(x32, j), v);
    }
  } else {
    const uint32_t loff = (uint32_t)row / 2u;
    const uint32_t szoff = (uint32_t)(T / 2) + (uint32_t)(row / sh.base_group) * 4u;
    int i = wfb;
    for (; i + kUnroll <= wfe; i += kUnroll) {
      int idx[kUnroll];
      uint32_t c[kUnroll], sz[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) idx[u] = (int)min((uint32_t)full_idx[i + u], jmax);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const uint8_t* col = packed + (int64_t)idx[u] * sh.stride_F;
        c[u] = *reinterpret_cast<const uint32_t*>(col + loff);
        sz[u] = *reinterpret_cast<const uint32_t*>(col + szoff);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const float xv = load_x(x32, idx[u]);
        fma_int4x8(acc, xv * half_lo(sz[u]), c[u]);
        zsum = fmaf(xv, half_hi(sz[u]), zsum);
      }
    }
    for (; i < wfe; ++i) {
      const int j = (int)min((uint32_t)full_idx[i], jmax);
      const uint8_t* col = packed + (int64_t)j * sh.stride_F;
      const uint32_t c = *reinterpret_cast<const uint32_t*>(col + loff);
      const uint32_t sz = *reinterpret_cast<const uint32_t*>(col + szoff);
      const float xv = load_x(x32, j);
      fma_int4x8(acc, xv * half_lo(sz), c);
      zsum = fmaf(xv, half_hi(sz), zsum);
    }
  }

  // ------------------------------------------------------------ APPROX tier (two-bit)
  {
    const uint8_t* regionA = packed + sh.off_A;
    const uint32_t loff = (uint32_t)row / 4u;
    const uint32_t szoff = (uint32_t)(T / 4) + (uint32_t)(row / sh.approx_group) * 4u;
    int i = wab;
    for (; i + kUnroll <= wae; i += kUnroll) {
      int idx[kUnroll];
      uint32_t c[kUnroll], sz[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) idx[u] = (int)min((uint32_t)approx_idx[i + u], jmax);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const uint8_t* col = regionA + (int64_t)idx[u] * sh.stride_A;
        c[u] = (uint32_t)*reinterpret_cast<const uint16_t*>(col + loff);
        sz[u] = *reinterpret_cast<const uint32_t*>(col + szoff);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const float xv = load_x(x32, idx[u]);
        fma_int2x8(acc, xv * half_lo(sz[u]), c[u]);
        zsum = fmaf(xv, half_hi(sz[u]), zsum);
      }
    }
    for (; i < wae; ++i) {
      const int j = (int)min((uint32_t)approx_idx[i], jmax);
      const uint8_t* col = regionA + (int64_t)j * sh.stride_A;
      const uint32_t c = (uint32_t)*reinterpret_cast<const uint16_t*>(col + loff);
      const uint32_t sz = *reinterpret_cast<const uint32_t*>(col + szoff);
      const float xv = load_x(x32, j);
      fma_int2x8(acc, xv * half_lo(sz), c);
      zsum = fmaf(xv, half_hi(sz), zsum);
    }
  }

  // ------------------------------------------------------------ reduce across waves
  {
    float4* dst = reinterpret_cast<float4*>(&red[wave][lane * 8]);
    dst[0] = make_float4(acc[0] + zsum, acc[1] + zsum, acc[2] + zsum, acc[3] + zsum);
    dst[1] = make_float4(acc[4] + zsum, acc[5] + zsum, acc[6] + zsum, acc[7] + zsum);
  }
  __syncthreads();
  float sum = 0.0f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) sum += red[w][tid];
  const int grow = row0 + tid;
  if (grow >= T) return;
  // ------------------------------------------------------------ reduce across chunks
  // One chunk: plain store.  Several: hardware fp32 atomic add at device scope into a y that
  // was zeroed earlier in stream order.  No device-scope fence is needed because y is only
  // read after the kernel has finished.
  if (sh.n_chunks == 1) y[grow] = sum;
  else unsafeAtomicAdd(&y[grow], sum);
}

__global__ __launch_bounds__(256) void zero_f32_kernel(float4* __restrict__ p, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n4) p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  if (!v || !*v) return dflt;
  return atoi(v);
}

}  // namespace

GemvPlan gemv_plan(const spax_layout* L) {
  GemvPlan p{};
  const int64_t T = L->d_out_total;
  p.n_tiles = (int32_t)((T + kTileRows - 1) / kTileRows);
  // Split-K: aim for about `target` resident workgroups, but keep >= 16 input channels per
  // chunk.
  static const int target = env_int("SPAX_GEMV_TARGET_WGS", 1024);
  int k = (target + p.n_tiles / 2) / p.n_tiles;
  const int kmax = L->d_in / 16 > 1 ? L->d_in / 16 : 1;
  if (k > kmax) k = kmax;
  if (k < 1) k = 1;
  p.n_chunks = k;
  p.ws_bytes = 0;
  return p;
}

int launch_zero_f32(float* y, int64_t n, hipStream_t s) {
  const int64_t n4 = (n + 3) / 4;
  const int threads = 256;
  hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)((n4 + threads - 1) / threads)), dim3(threads),
                     0, s, reinterpret_cast<float4*>(y), n4);
  SPAX_HIP_CHECK(hipGetLastError());
  return SPAX_OK;
}

int launch_tiered_gemv(const spax_layout* L, const GemvPlan& plan, const void* packed,
                       const uint16_t* x, const int32_t* full_idx, const int32_t* approx_idx,
                       const int32_t* counts, float* y, bool y_zeroed, hipStream_t s) {
  if (plan.n_chunks > 1 && !y_zeroed) {
    int st = launch_zero_f32(y, L->d_out_total, s);
    if (st) return st;
  }
  GemvShape sh{};
  sh.stride_F = L->stride_F;
  sh.stride_A = L->stride_A;
  sh.off_A = L->off_A;
  sh.T = (int32_t)L->d_out_total;
  sh.n_tiles = plan.n_tiles;
  sh.n_chunks = plan.n_chunks;
  sh.approx_group = L->approx_group;
  sh.base_group = L->base_group;
  sh.d_in = L->d_in;
  const dim3 grid((unsigned)(plan.n_tiles * plan.n_chunks));
  const auto* pk = static_cast<const uint8_t*>(packed);
  const auto* x32 = reinterpret_cast<const uint32_t*>(x);
  if (L->base_fmt == SPAX_FMT_FP16)
    hipLaunchKernelGGL(tiered_gemv_kernel<SPAX_FMT_FP16>, grid, dim3(kGemvThreads), 0, s, sh, pk,
                       x32, full_idx, approx_idx, counts, y);
  else
    hipLaunchKernelGGL(tiered_gemv_kernel<SPAX_FMT_INT4>, grid, dim3(kGemvThreads), 0, s, sh, pk,
                       x32, full_idx, approx_idx, counts, y);
  SPAX_HIP_CHECK(hipGetLastError());
  return SPAX_OK;
}

}  // namespace spax
