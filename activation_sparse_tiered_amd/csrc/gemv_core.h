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
// A group spans >= 64 rows, so the zero-point term is the same for a lane's 8 rows and is
// summed once per column into zsum (see fma_int4x8 for the form the codes take).
#pragma once

#include "common.h"

namespace spax {
namespace gemv {

constexpr int kWaves = kGemvThreads / 64;
#ifndef SPAX_UNROLL
#define SPAX_UNROLL 4
#endif
constexpr int kUnroll = SPAX_UNROLL;  // columns per tier whose loads are in flight together

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

// Codes enter the multiply-adds as fp16 operands of v_fma_mix_f32 (an fp32 FMA that reads one
// half of a packed register), with no integer-to-float conversion: a code q placed in the top
// mantissa bits under the exponent of 1.0 reads as h = 1 + q / 2^b (b = 4 for int4, 2 for
// two-bit codes).  Two rows share a register, one per half, so each pair of rows costs one
// shift and one and-or.  The caller scales by 2^b and removes the constant part:
// x (s q + z) = (2^b x s) h + x (z - 2^b s).
constexpr uint32_t kOne16x2 = 0x3C003C00u;  // fp16 1.0 in both halves

// (x & m) | k in one instruction.  Written out because the compiler splits it into two
// (the three-operand form takes no literal constants, so m and k are passed in registers).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t k) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(m), "v"(k));
  return r;
}

// 8 int4 codes (row n in bits [4n+3:4n]) times a = 16 x s: acc[r] += a (1 + q_r / 16).
__device__ __forceinline__ void fma_int4x8(float (&acc)[8], float a, uint32_t c) {
  const uint32_t m = 0x03C003C0u;  // mantissa bits 6..9 of both halves
  const uint32_t h0 = and_or(c << 6, m, kOne16x2);  // rows 0, 4
  const uint32_t h1 = and_or(c << 2, m, kOne16x2);  // rows 1, 5
  const uint32_t h2 = and_or(c >> 2, m, kOne16x2);  // rows 2, 6
  const uint32_t h3 = and_or(c >> 6, m, kOne16x2);  // rows 3, 7
  acc[0] = fmaf(a, half_lo(h0), acc[0]);
  acc[4] = fmaf(a, half_hi(h0), acc[4]);
  acc[1] = fmaf(a, half_lo(h1), acc[1]);
  acc[5] = fmaf(a, half_hi(h1), acc[5]);
  acc[2] = fmaf(a, half_lo(h2), acc[2]);
  acc[6] = fmaf(a, half_hi(h2), acc[6]);
  acc[3] = fmaf(a, half_lo(h3), acc[3]);
  acc[7] = fmaf(a, half_hi(h3), acc[7]);
}

// A column's group terms for codes read as h = 1 + q / 2^B: returns the multiplier
// a = 2^B x s and adds x z - a to zsum, with s and z the fp16 halves of the group's (s, z)
// word read by v_fma_mix_f32 (no separate conversions).  The zero addend keeps the first
// product a fused multiply-add, which can read an fp16 operand.
template <int B>
__device__ __forceinline__ float group_terms(float x, uint32_t sz, float& zsum) {
  const float a = fmaf(x * (float)(1 << B), half_lo(sz), 0.0f);
  zsum = fmaf(x, half_hi(sz), zsum) - a;
  return a;
}

// Byte selector that moves bytes k0 and k0 + 1 of a dword to bytes 1 and 3 (zeros elsewhere).
__device__ __forceinline__ uint32_t spread_sel(uint32_t k0) {
  return 0x000C000Cu | (k0 << 8) | ((k0 + 1u) << 24);
}

// 8 two-bit codes (row 4k+i in bits [2i+1:2i] of byte k0+k of w, k0 given through sel) times
// a = 4 x s: acc[r] += a (1 + q_r / 4).
__device__ __forceinline__ void fma_int2x8(float (&acc)[8], float a, uint32_t w, uint32_t sel) {
  const uint32_t p = __builtin_amdgcn_perm(0u, w, sel);  // rows 0..3 at bits 8.., 4..7 at 24..
  const uint32_t m = 0x03000300u;  // mantissa bits 8..9 of both halves
  const uint32_t h0 = and_or(p, m, kOne16x2);        // rows 0, 4
  const uint32_t h1 = and_or(p >> 2, m, kOne16x2);   // rows 1, 5
  const uint32_t h2 = and_or(p >> 4, m, kOne16x2);   // rows 2, 6
  const uint32_t h3 = and_or(p >> 6, m, kOne16x2);   // rows 3, 7
  acc[0] = fmaf(a, half_lo(h0), acc[0]);
  acc[4] = fmaf(a, half_hi(h0), acc[4]);
  acc[1] = fmaf(a, half_lo(h1), acc[1]);
  acc[5] = fmaf(a, half_hi(h1), acc[5]);
  acc[2] = fmaf(a, half_lo(h2), acc[2]);
  acc[6] = fmaf(a, half_hi(h2), acc[6]);
  acc[3] = fmaf(a, half_lo(h3), acc[3]);
  acc[7] = fmaf(a, half_hi(h3), acc[7]);
}

// Every pointer here points to device (global) memory.  Loads through a pointer that reaches
// the kernel inside a descriptor in memory are compiled as flat loads unless the address
// space is stated; flat loads also count as LDS operations for the wait counters.
template <class T>
using global_ptr = const __attribute__((address_space(1))) T*;
template <class T>
__device__ __forceinline__ T load_global(const void* p) {
  return *(global_ptr<T>)p;  // a C-style cast: reinterpret_cast cannot change address space
}

// A wave-uniform value moved to a scalar register, so that the compiler treats what depends
// on it (loop bounds, branches, addresses) as uniform: values loaded from memory after the
// kernel has stored to memory are otherwise kept per lane.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uniform(int64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
template <class T>
__device__ __forceinline__ T* uniform(T* p) {
  return reinterpret_cast<T*>(uniform((int64_t)reinterpret_cast<uintptr_t>(p)));
}

// Weight codes are read once per token: optionally as non-temporal loads.
#ifndef SPAX_NT_LOADS
#define SPAX_NT_LOADS 1
#endif

// Loads from one column record through a buffer descriptor built on the record's (uniform)
// base: the record base stays in scalar registers and the lane's byte offset, the same for
// every column, is the only vector operand, so no 64-bit address is added per column and
// load.  The descriptor's size is the record's, so a load past it reads zero.
struct Record {
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ Record(const uint8_t* base, int64_t bytes)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, (int)bytes,
                                            0x00020000)) {}
  // cache policy 2: non-temporal (weight codes are read once per token)
  __device__ __forceinline__ uint32_t stream32(uint32_t off) const {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, SPAX_NT_LOADS ? 2 : 0);
  }
  __device__ __forceinline__ uint32_t word(uint32_t off) const {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  }
  __device__ __forceinline__ uint4 stream128(uint32_t off) const {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, SPAX_NT_LOADS ? 2 : 0);
    return make_uint4(v.x, v.y, v.z, v.w);
  }
};

// A block of up to 64 entries of a column list held in registers, one per lane: entry =
// channel | (fp16 bits of x_j) << 16, for list positions [base, base + 64).  Loaded with one
// vector load of the indices and one gather of the activations (load_blocks: two dependent
// round trips per 64 columns instead of two per column); get() broadcasts one entry with
// readlane.  Indices are clamped to [0, d_in), so malformed lists cannot address outside the
// blob.
struct RegBlock {
  uint32_t e;
  int base;
  __device__ __forceinline__ void get(int i, int& j, float& xv) const {
    const uint32_t v = (uint32_t)__builtin_amdgcn_readlane((int)e, i - base);
    j = (int)(v & 0xFFFFu);
    xv = half_hi(v);
  }
};

// The FULL and the APPROX block of one step of 64 list positions, [fi, fend) and [ai, aend),
// with their loads overlapped: both index loads, then both activation gathers (two dependent
// round trips for the pair instead of four).  The loads are unconditional: a lane past its
// tier's end reads the tier's last entry (or entry 0 of an empty list, whose buffer still
// holds d_in entries) and keeps a zero entry.  kCompact: the lists hold staging slot |
// channel << 16 (pinned-host path) and the returned entry holds the slot and x of the
// channel.
template <bool kCompact>
__device__ __forceinline__ void load_blocks(const void* __restrict__ idxF,
                                            const void* __restrict__ idxA,
                                            const uint16_t* __restrict__ x16, int fi, int fend,
                                            int ai, int aend, uint32_t jmax, RegBlock& bf,
                                            RegBlock& ba) {
  const int lane = threadIdx.x & 63;
  const int iF = fi + lane, iA = ai + lane;
  const uint32_t rF =
      load_global<uint32_t>(reinterpret_cast<const uint32_t*>(idxF) + min(iF, max(fend - 1, 0)));
  const uint32_t rA =
      load_global<uint32_t>(reinterpret_cast<const uint32_t*>(idxA) + min(iA, max(aend - 1, 0)));
  const uint32_t jF = min(kCompact ? rF >> 16 : rF, jmax), jA = min(kCompact ? rA >> 16 : rA, jmax);
  const uint32_t sF = kCompact ? min(rF & 0xFFFFu, jmax) : jF;
  const uint32_t sA = kCompact ? min(rA & 0xFFFFu, jmax) : jA;
  const uint32_t xF = load_global<uint16_t>(x16 + jF), xA = load_global<uint16_t>(x16 + jA);
  bf = RegBlock{iF < fend ? sF | (xF << 16) : 0u, fi};
  ba = RegBlock{iA < aend ? sA | (xA << 16) : 0u, ai};
}

// Column lists in LDS (fused kernel): entry = channel | (fp16 bits of x_j) << 16.  Up to 64
// consecutive entries are held one per lane: one LDS read for the wave instead of one read
// and wait per column; get() broadcasts entry i with readlane.  Lanes past n read entry n - 1
// (entry 0 when n <= 0), so p must hold at least one entry.  The channel is clamped to
// [0, d_in) like the global lists, so a corrupted entry can never address outside the blob.
struct LdsBlock {
  uint32_t e;
  uint32_t jmax;
  __device__ __forceinline__ LdsBlock(const uint32_t* p, int n, uint32_t jmax_) : jmax(jmax_) {
    const int lane = threadIdx.x & 63;
    e = p[min(lane, max(n - 1, 0))];
  }
  __device__ __forceinline__ void get(int i, int& j, float& xv) const {
    const uint32_t v = (uint32_t)__builtin_amdgcn_readlane((int)e, i);
    j = (int)min(v & 0xFFFFu, jmax);
    xv = half_hi(v);
  }
};

// Up to P FULL columns whose loads are issued ahead of the rest of the work and multiplied
// later (the fused decode kernel issues them while its mask is still being completed, so
// their memory latency overlaps that work).  Entries as in LdsBlock.  All P loads are issued
// (a conditional load would make the compiler copy its result right away, which waits for
// it): slots past n load the entry the caller put there (a repeat of a used column, which
// costs no extra HBM traffic, or column 0) and are multiplied by a zero activation.
template <int FMT, int P>
struct EarlyColumns {
  float xv[P];
  uint4 v[P];
  uint32_t c[P], sz[P];
  __device__ __forceinline__ void issue(const Shape& sh, const uint8_t* __restrict__ packed,
                                        int row, const uint32_t (&e)[P], int n, uint32_t jmax) {
    const uint32_t loffF = FMT == SPAX_FMT_FP16 ? (uint32_t)row * 2u : (uint32_t)row / 2u;
    const uint32_t szoffF = (uint32_t)(sh.T / 2) + (uint32_t)(row / sh.base_group) * 4u;
#pragma unroll
    for (int u = 0; u < P; ++u) {
      const uint32_t j = min(e[u] & 0xFFFFu, jmax);
      xv[u] = u < n ? half_hi(e[u]) : 0.0f;
      const Record rec(packed + (int64_t)j * sh.stride_F, sh.stride_F);
      if (FMT == SPAX_FMT_FP16) {
        v[u] = rec.stream128(loffF);
      } else {
        c[u] = rec.stream32(loffF);
        sz[u] = rec.word(szoffF);
      }
    }
  }
  __device__ __forceinline__ void multiply(float (&acc)[8], float& zsum) const {
#pragma unroll
    for (int u = 0; u < P; ++u) {
      if (FMT == SPAX_FMT_FP16) {
        fma_fp16x8(acc, xv[u], v[u]);
      } else {
        fma_int4x8(acc, group_terms<4>(xv[u], sz[u], zsum), c[u]);
      }
    }
  }
};

// A lane's byte offsets inside a column record for its rows of the tile.
template <int FMT>
struct TileOffsets {
  uint32_t loffA4;  // two-bit codes: the aligned dword that holds the lane's 2 bytes (a 16-bit
                    // load would be widened right after it is issued, which makes it wait)
  uint32_t selA;    // byte selector for those 2 bytes
  uint32_t szoffA;  // (s, z) word of the lane's two-bit group
  uint32_t loffF;   // FULL codes (fp16 rows or int4 codes)
  uint32_t szoffF;  // (s, z) word of the lane's int4 group
  __device__ __forceinline__ TileOffsets(const Shape& sh, int row)
      : loffA4(((uint32_t)row / 4u) & ~3u),
        selA(spread_sel(((uint32_t)row / 4u) & 2u)),
        szoffA((uint32_t)(sh.T / 4) + (uint32_t)(row / sh.approx_group) * 4u),
        loffF(FMT == SPAX_FMT_FP16 ? (uint32_t)row * 2u : (uint32_t)row / 2u),
        szoffF((uint32_t)(sh.T / 2) + (uint32_t)(row / sh.base_group) * 4u) {}
};

// The registers of one round: up to kUnroll FULL and kUnroll APPROX columns.
template <int FMT>
struct RoundLoads {
  float xf[kUnroll], xa[kUnroll];
  uint4 vf[kUnroll];
  uint32_t cf[kUnroll], sf[kUnroll], ca[kUnroll], sa[kUnroll];
};

// Issues the loads of FULL columns [fi, fi + nf) of srcF and APPROX columns [ai, ai + na) of
// srcA (counts wave-uniform, at most kUnroll, may be <= 0).  Slots past a count keep zero
// data and a zero activation.
template <int FMT, class SrcF, class SrcA>
__device__ __forceinline__ void issue_round(const Shape& sh, const uint8_t* __restrict__ packed,
                                            const TileOffsets<FMT>& g, const SrcF& srcF, int fi,
                                            int nf, const SrcA& srcA, int ai, int na,
                                            RoundLoads<FMT>& r) {
  const uint8_t* regionA = packed + sh.off_A;
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    r.xf[u] = 0.0f;
    r.xa[u] = 0.0f;
    r.vf[u] = make_uint4(0u, 0u, 0u, 0u);
    r.cf[u] = r.sf[u] = r.ca[u] = r.sa[u] = 0u;
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    if (u < nf) {
      int j;
      srcF.get(fi + u, j, r.xf[u]);
      const Record rec(packed + (int64_t)j * sh.stride_F, sh.stride_F);
      if (FMT == SPAX_FMT_FP16) {
        r.vf[u] = rec.stream128(g.loffF);
      } else {
        r.cf[u] = rec.stream32(g.loffF);
        r.sf[u] = rec.word(g.szoffF);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    if (u < na) {
      int j;
      srcA.get(ai + u, j, r.xa[u]);
      const Record rec(regionA + (int64_t)j * sh.stride_A, sh.stride_A);
      r.ca[u] = rec.stream32(g.loffA4);
      r.sa[u] = rec.word(g.szoffA);
    }
  }
}

// Waits for every load of the round and multiplies.  A tier with no column in the round
// skips its multiplies (a wave-uniform branch around whole blocks).  The explicit wait for
// every load makes the branches visible as complete to the compiler's wait tracking, which
// otherwise assumes loads of a skipped block are still in flight in the next round and waits
// for each of them there.
template <int FMT>
__device__ __forceinline__ void finish_round(const RoundLoads<FMT>& r, const TileOffsets<FMT>& g,
                                             int nf, int na, float (&acc)[8], float& zsum) {
  __builtin_amdgcn_s_waitcnt(0);
  if (nf > 0) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (FMT == SPAX_FMT_FP16) {
        fma_fp16x8(acc, r.xf[u], r.vf[u]);
      } else {
        fma_int4x8(acc, group_terms<4>(r.xf[u], r.sf[u], zsum), r.cf[u]);
      }
    }
  }
  if (na > 0) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      fma_int2x8(acc, group_terms<2>(r.xa[u], r.sa[u], zsum), r.ca[u], g.selA);
    }
  }
}

// FULL columns [fb, fe) of `srcF` and APPROX (two-bit) columns [ab, ae) of `srcA` into
// acc / zsum.  Each round issues the loads of up to kUnroll FULL and kUnroll APPROX columns
// back to back (the counts are wave-uniform, so the guards are scalar branches) and only then
// waits and multiplies: a wave's few columns cost one or two memory round trips, not one per
// column.  Slots past the end keep zero data and a zero activation and are multiplied
// anyway: with conditional multiplies the compiler's wait tracking cannot tell which loads of
// the previous round are still in flight and makes every load wait for all earlier ones.
// `row` is the lane's first row (or 0 for lanes past the last row, which read valid memory
// and are never stored).
template <int FMT, class SrcF, class SrcA>
__device__ __forceinline__ void stream_columns(const Shape& sh, const uint8_t* __restrict__ packed,
                                               int row, int fb, int fe, const SrcF& srcF, int ab,
                                               int ae, const SrcA& srcA, float (&acc)[8],
                                               float& zsum) {
  const TileOffsets<FMT> g(sh, row);
  int fi = fb, ai = ab;
  while (fi < fe || ai < ae) {
    const int nf = min(fe - fi, kUnroll), na = min(ae - ai, kUnroll);  // may be <= 0
    RoundLoads<FMT> r;
    issue_round<FMT>(sh, packed, g, srcF, fi, nf, srcA, ai, na, r);
    finish_round<FMT>(r, g, nf, na, acc, zsum);
    fi += max(nf, 0);
    ai += max(na, 0);
  }
}

// First item of part c when n items are split into `parts` contiguous parts.  n <= 32768
// and parts <= 2048, so 32-bit unsigned arithmetic suffices (a 64-bit division costs a
// wavefront ~130 scalar instructions, and every wave of the CU shares one scalar unit).
__device__ __forceinline__ int split_at(int n, int c, int parts) {
  return (int)((uint32_t)n * (uint32_t)c / (uint32_t)parts);
}

// Work-item order for the chip's 8 XCDs.  Workgroups are dispatched to the XCDs round-robin
// (workgroup b runs on XCD b % 8), and each XCD has its own L2.  Item b is mapped to
// (b % 8) * (n / 8) + b / 8, so each XCD takes one contiguous run of items: whole column
// chunks with all their row tiles, and the lines that the tiles of one column share (its
// (s, z) words) are fetched into one L2 instead of several.  A bijection on [0, n); items past
// the last multiple of 8 keep their index.
__device__ __forceinline__ int xcd_order(int b, int n) {
  const int n8 = n >> 3;
  return b < (n8 << 3) ? (b & 7) * n8 + (b >> 3) : b;
}

// Split [b, e) evenly over the workgroup's NW waves.
template <int NW>
__device__ __forceinline__ void wave_range(int b, int e, int wave, int& wb, int& we) {
  wb = b + (e - b) * wave / NW;
  we = b + (e - b) * (wave + 1) / NW;
}

// Reduce the NW waves' partial rows through LDS, then write (one chunk) or atomically add
// (several chunks, y zeroed beforehand in stream order) the tile into y.
template <int NW>
__device__ __forceinline__ void finish_tile(float (*red)[kTileRows], const float (&acc)[8],
                                            float zsum, int wave, int lane, int row0, int T,
                                            int n_chunks, float* __restrict__ y) {
  const int tid = threadIdx.x;
  float4* dst = reinterpret_cast<float4*>(&red[wave][lane * 8]);
  dst[0] = make_float4(acc[0] + zsum, acc[1] + zsum, acc[2] + zsum, acc[3] + zsum);
  dst[1] = make_float4(acc[4] + zsum, acc[5] + zsum, acc[6] + zsum, acc[7] + zsum);
  __syncthreads();
  const int grow = row0 + tid;
  if (tid < kTileRows && grow < T) {
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) sum += red[w][tid];
    // Several chunks meet through hardware fp32 atomics at device scope; y is read only after
    // the kernel ends, so no device-scope fence is needed.
    if (n_chunks == 1) y[grow] = sum;
    else unsafeAtomicAdd(&y[grow], sum);
  }
}

// One work item of the stand-alone GEMV: row tile `tile`, column chunk `chunk` of the lists
// in global memory (counts and indices clamped to [0, d_in], so malformed lists cannot
// address outside the blob).  kCompact: the lists hold slot | channel << 16 entries into a
// compacted staging copy of the records (`packed` is then the staging buffer).  A workgroup
// of kWaves waves; ends after the tile's atomics.
template <int FMT, bool kCompact = false>
__device__ __forceinline__ void gemv_item(const Shape& sh, const uint8_t* __restrict__ packed,
                                          const uint32_t* __restrict__ x32,
                                          const int32_t* __restrict__ full_idx,
                                          const int32_t* __restrict__ approx_idx,
                                          const int32_t* __restrict__ counts,
                                          float* __restrict__ y, int tile, int chunk,
                                          float (*red)[kTileRows]) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int T = sh.T;
  const int row0 = tile * kTileRows;
  // Lanes past the last row (ragged last tile) read the record's first rows instead, which
  // is always in bounds; their sums land in rows >= T and are never stored.
  const int row = row0 + lane * 8 < T ? row0 + lane * 8 : 0;
  const int nF = uniform(min(max(load_global<int32_t>(counts), 0), sh.d_in));
  const int nA = uniform(min(max(load_global<int32_t>(counts + 1), 0), sh.d_in));
  const uint32_t jmax = (uint32_t)sh.d_in - 1u;
  const int fb = split_at(nF, chunk, sh.n_chunks);
  const int fe = split_at(nF, chunk + 1, sh.n_chunks);
  const int ab = split_at(nA, chunk, sh.n_chunks);
  const int ae = split_at(nA, chunk + 1, sh.n_chunks);
  int wfb, wfe, wab, wae;
  wave_range<kWaves>(fb, fe, wave, wfb, wfe);
  wave_range<kWaves>(ab, ae, wave, wab, wae);
  float acc[8];
#pragma unroll
  for (int h = 0; h < 8; ++h) acc[h] = 0.0f;
  float zsum = 0.0f;
  const uint16_t* x16 = reinterpret_cast<const uint16_t*>(x32);
  // 64 list entries per tier and block; the channels fit the 16-bit entry field (d_in <= 32768)
  for (int fi = wfb, ai = wab; fi < wfe || ai < wae; fi += 64, ai += 64) {
    const int fend = min(fi + 64, wfe), aend = min(ai + 64, wae);
    RegBlock bf, ba;
    load_blocks<kCompact>(full_idx, approx_idx, x16, fi, fend, ai, aend, jmax, bf, ba);
    stream_columns<FMT>(sh, packed, row, fi, max(fi, fend), bf, ai, max(ai, aend), ba, acc, zsum);
  }
  finish_tile<kWaves>(red, acc, zsum, wave, lane, row0, T, sh.n_chunks, y);
}

}  // namespace gemv
}  // namespace spax
