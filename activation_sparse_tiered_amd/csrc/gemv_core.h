// Column streaming of the tiered GEMV, shared by the stand-alone GEMV kernel (column lists
// in global memory) and the fused mask+GEMV kernel of the decode step (lists in LDS).
//
// Pages: SpAx Abstract (arXiv:2610.02598) -- per input channel the column is read in full,
// read as a compressed approximation, or skipped; eigenradar commentary on SpAx, "The route
// outside GPU memory", third paragraph -- the two-bit approximation is reconstructed on the
// GPU.  Every selected byte feeds exactly one multiply-add, so the loops are built to keep
// many 16-byte loads in flight, not to reuse data; MFMA does not apply.
//
// Lane mapping: a row tile is 512 rows; lane l of a wavefront owns rows [8l, 8l+8) of it.
//   FULL fp16 : one 16-byte load per column (8 halves), fp32 FMA with fp16 operands;
//   FULL int4 : 4 bytes of codes (8 nibbles) + the (s, z) word of the lane's group;
//   APPROX 2b : 2 bytes of codes (8 two-bit codes) + the (s, z) word of the lane's group.
// A group spans >= 64 rows, so the zero-point term x_j * z is the same for a lane's 8 rows
// and is summed once per column into zsum: x_j (s q + z) = (x_j s) q + x_j z.
#pragma once

#include "common.h"

namespace spax {
namespace gemv {

constexpr int kWaves = kGemvThreads / 64;
constexpr int kUnroll = 8;

struct Shape {
  int64_t stride_F, stride_A, off_A;
  int32_t T, n_tiles, n_chunks;
  int32_t approx_group, base_group;
  int32_t d_in;
};

}  // namespace gemv

gemv::Shape gemv_shape(const spax_layout* L, const GemvPlan& plan);

namespace gemv {

__device__ __forceinline__ float half_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float half_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
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

// 8 int4 codes (row 2k in the low nibble of byte k/2) scaled by a.
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

// Column lists in global memory (stand-alone GEMV): indices clamped to [0, d_in), the
// activation read with a wave-uniform scalar dword load.
struct GlobalList {
  const int32_t* __restrict__ idx;
  const uint32_t* __restrict__ x32;
  uint32_t jmax;
  __device__ __forceinline__ void get(int i, int& j, float& xv) const {
    j = (int)min((uint32_t)idx[i], jmax);
    const uint32_t w = x32[j >> 1];
    xv = (j & 1) ? half_hi(w) : half_lo(w);
  }
};

// Column lists in LDS (fused kernel): entry = channel | (fp16 bits of x_j) << 16, indexed
// from the workgroup's first rank `base`.  The channel is clamped to [0, d_in) like the
// global lists, so a corrupted entry can never address outside the blob.
struct LdsList {
  const uint32_t* e;
  int base;
  uint32_t jmax;
  __device__ __forceinline__ void get(int i, int& j, float& xv) const {
    const uint32_t v = __builtin_amdgcn_readfirstlane(e[i - base]);
    j = (int)min(v & 0xFFFFu, jmax);
    xv = half_hi(v);
  }
};

// FULL columns [b, e) of `src` into acc / zsum.  `row` is the lane's first row (or 0 for
// lanes past the last row, which read valid memory and are never stored).
template <int FMT, class Src>
__device__ __forceinline__ void stream_full(const Shape& sh, const uint8_t* __restrict__ packed,
                                            int row, int b, int e, const Src& src,
                                            float (&acc)[8], float& zsum) {
  if (FMT == SPAX_FMT_FP16) {
    const uint32_t loff = (uint32_t)row * 2u;
    int i = b;
    for (; i + kUnroll <= e; i += kUnroll) {
      int j[kUnroll];
      float xv[kUnroll];
      uint4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) src.get(i + u, j[u], xv[u]);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        v[u] = *reinterpret_cast<const uint4*>(packed + (int64_t)j[u] * sh.stride_F + loff);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) fma_fp16x8(acc, xv[u], v[u]);
    }
    for (; i < e; ++i) {
      int j;
      float xv;
      src.get(i, j, xv);
      const uint4 v = *reinterpret_cast<const uint4*>(packed + (int64_t)j * sh.stride_F + loff);
      fma_fp16x8(acc, xv, v);
    }
  } else {
    const uint32_t loff = (uint32_t)row / 2u;
    const uint32_t szoff = (uint32_t)(sh.T / 2) + (uint32_t)(row / sh.base_group) * 4u;
    int i = b;
    for (; i + kUnroll <= e; i += kUnroll) {
      int j[kUnroll];
      float xv[kUnroll];
      uint32_t c[kUnroll], sz[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) src.get(i + u, j[u], xv[u]);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const uint8_t* col = packed + (int64_t)j[u] * sh.stride_F;
        c[u] = *reinterpret_cast<const uint32_t*>(col + loff);
        sz[u] = *reinterpret_cast<const uint32_t*>(col + szoff);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        fma_int4x8(acc, xv[u] * half_lo(sz[u]), c[u]);
        zsum = fmaf(xv[u], half_hi(sz[u]), zsum);
      }
    }
    for (; i < e; ++i) {
      int j;
      float xv;
      src.get(i, j, xv);
      const uint8_t* col = packed + (int64_t)j * sh.stride_F;
      const uint32_t c = *reinterpret_cast<const uint32_t*>(col + loff);
      const uint32_t sz = *reinterpret_cast<const uint32_t*>(col + szoff);
      fma_int4x8(acc, xv * half_lo(sz), c);
      zsum = fmaf(xv, half_hi(sz), zsum);
    }
  }
}

// APPROX (two-bit) columns [b, e) of `src`.
template <class Src>
__device__ __forceinline__ void stream_approx(const Shape& sh, const uint8_t* __restrict__ packed,
                                              int row, int b, int e, const Src& src,
                                              float (&acc)[8], float& zsum) {
  const uint8_t* regionA = packed + sh.off_A;
  const uint32_t loff = (uint32_t)row / 4u;
  const uint32_t szoff = (uint32_t)(sh.T / 4) + (uint32_t)(row / sh.approx_group) * 4u;
  int i = b;
  for (; i + kUnroll <= e; i += kUnroll) {
    int j[kUnroll];
    float xv[kUnroll];
    uint32_t c[kUnroll], sz[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) src.get(i + u, j[u], xv[u]);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint8_t* col = regionA + (int64_t)j[u] * sh.stride_A;
      c[u] = (uint32_t)*reinterpret_cast<const uint16_t*>(col + loff);
      sz[u] = *reinterpret_cast<const uint32_t*>(col + szoff);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      fma_int2x8(acc, xv[u] * half_lo(sz[u]), c[u]);
      zsum = fmaf(xv[u], half_hi(sz[u]), zsum);
    }
  }
  for (; i < e; ++i) {
    int j;
    float xv;
    src.get(i, j, xv);
    const uint8_t* col = regionA + (int64_t)j * sh.stride_A;
    const uint32_t c = (uint32_t)*reinterpret_cast<const uint16_t*>(col + loff);
    const uint32_t sz = *reinterpret_cast<const uint32_t*>(col + szoff);
    fma_int2x8(acc, xv * half_lo(sz), c);
    zsum = fmaf(xv, half_hi(sz), zsum);
  }
}

// Split [b, e) evenly over the workgroup's waves.
__device__ __forceinline__ void wave_range(int b, int e, int wave, int& wb, int& we) {
  wb = b + (e - b) * wave / kWaves;
  we = b + (e - b) * (wave + 1) / kWaves;
}

// Reduce the waves' partial rows through LDS, then write (one chunk) or atomically add
// (several chunks, y zeroed beforehand in stream order) the tile into y.
__device__ __forceinline__ void finish_tile(float (*red)[kTileRows], const float (&acc)[8],
                                            float zsum, int wave, int lane, int row0, int T,
                                            int n_chunks, float* __restrict__ y) {
  const int tid = threadIdx.x;
  float4* dst = reinterpret_cast<float4*>(&red[wave][lane * 8]);
  dst[0] = make_float4(acc[0] + zsum, acc[1] + zsum, acc[2] + zsum, acc[3] + zsum);
  dst[1] = make_float4(acc[4] + zsum, acc[5] + zsum, acc[6] + zsum, acc[7] + zsum);
  __syncthreads();
  float sum = 0.0f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) sum += red[w][tid];
  const int grow = row0 + tid;
  if (grow >= T) return;
  // Several chunks meet through hardware fp32 atomics at device scope; y is read only after
  // the kernel ends, so no device-scope fence is needed.
  if (n_chunks == 1) y[grow] = sum;
  else unsafeAtomicAdd(&y[grow], sum);
}

}  // namespace gemv
}  // namespace spax
