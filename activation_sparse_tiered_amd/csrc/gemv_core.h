// Column streaming of the tiered GEMV, shared by the stand-alone GEMV kernel (column lists
// in global memory) and the fused mask+GEMV kernel of the decode step (lists in LDS).
//
// Pages: SpAx Abstract (arXiv:2610.02598) -- per input channel the column is read in full,
// read as a compressed approximation, or skipped; eigenradar commentary on SpAx, "The route
// outside GPU memory", third paragraph -- the two-bit approximation is reconstructed on the
// GPU.  Every selected byte feeds exactly one multiply-add, so the loops are built to keep
// many 16-byte loads in flight, not to reuse data; MFMA does not apply.
//
// Lane mapping: lane l of a wavefront owns RPL consecutive rows [RPL l, RPL l + RPL) of a
// 64 RPL-row tile.  RPL = 8 (fp16 layouts, and the fused decode kernel):
//   FULL fp16 : one 16-byte load per column (8 halves), fp32 FMA with fp16 operands;
//   FULL int4 : 4 bytes of codes (8 nibbles) + the (s, z) word of the lane's group;
//   APPROX 2b : 2 bytes of codes (8 two-bit codes) + the (s, z) word of the lane's group.
// RPL = 32 (int4 layouts in the batched GEMV): one 16-byte load of 32 int4
// codes, or one 8-byte load of 32 two-bit codes, plus the group's (s, z) word per column, so a
// wave keeps as many bytes in flight per column as an fp16 wave.
// A group spans >= 64 rows, so the zero-point term is the same for all of a lane's rows and
// is summed once per column into zsum (see fma_int4x8 for the form the codes take).
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

__device__ __forceinline__ void fma_fp16x8(float* acc, float xv, const uint4& v) {
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
__device__ __forceinline__ void fma_int4x8(float* acc, float a, uint32_t c) {
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
__device__ __forceinline__ void fma_int2x8(float* acc, float a, uint32_t w, uint32_t sel) {
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

// Loads from one column record: a buffer descriptor in scalar registers plus a scalar byte
// offset, so the lane's byte offset inside the record, the same for every column, is the only
// vector operand and no 64-bit address is formed per load.  Callers keep every offset inside
// the record (lanes past a tile's last row read row 0), so no load relies on the hardware's
// range check.
struct Column {
  __amdgpu_buffer_rsrc_t r;
  uint32_t so;
  // cache policy 2: non-temporal (weight codes are read once per token)
  __device__ __forceinline__ uint32_t stream32(uint32_t off) const {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, (int)so, SPAX_NT_LOADS ? 2 : 0);
  }
  __device__ __forceinline__ uint32_t word(uint32_t off) const {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, (int)so, 0);
  }
  __device__ __forceinline__ uint2 stream64(uint32_t off) const {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, (int)so, SPAX_NT_LOADS ? 2 : 0);
    return make_uint2(v.x, v.y);
  }
  __device__ __forceinline__ uint4 stream128(uint32_t off) const {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, (int)so, SPAX_NT_LOADS ? 2 : 0);
    return make_uint4(v.x, v.y, v.z, v.w);
  }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const uint8_t* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Column records of a blob through one descriptor per region (the FULL records, then the
// APPROX records): record j lies at scalar offset j * stride, one scalar multiply per column.
// Only for blobs whose two regions are each below 2 GiB (narrow_regions on the host), so every
// offset fits 32 bits.
struct RegionBlob {
  __amdgpu_buffer_rsrc_t rF, rA;
  uint32_t sF, sA;
  __device__ __forceinline__ RegionBlob(const Shape& sh, const uint8_t* packed)
      : rF(buffer_rsrc(packed, sh.off_A)),
        rA(buffer_rsrc(packed + sh.off_A, (int64_t)sh.d_in * sh.stride_A)),
        sF((uint32_t)sh.stride_F),
        sA((uint32_t)sh.stride_A) {}
  __device__ __forceinline__ Column full(int j) const { return Column{rF, (uint32_t)j * sF}; }
  __device__ __forceinline__ Column approx(int j) const { return Column{rA, (uint32_t)j * sA}; }
};

// Any blob size: a descriptor built per column record on its 64-bit base (five more scalar
// instructions per column).
struct RecordBlob {
  const uint8_t* packed;
  int64_t sF, sA, offA;
  __device__ __forceinline__ RecordBlob(const Shape& sh, const uint8_t* p)
      : packed(p), sF(sh.stride_F), sA(sh.stride_A), offA(sh.off_A) {}
  __device__ __forceinline__ Column full(int j) const {
    return Column{buffer_rsrc(packed + (int64_t)j * sF, sF), 0u};
  }
  __device__ __forceinline__ Column approx(int j) const {
    return Column{buffer_rsrc(packed + offA + (int64_t)j * sA, sA), 0u};
  }
};

// A block of up to 64 entries of a column list held in registers, one per lane: entry =
// channel | (fp16 bits of x_j) << 16, for a wave's list positions [base, base + 64).  Loaded
// with one vector load of the indices and one gather of the activations (load_index,
// finish_blocks: two dependent round trips per 64 columns instead of two per column); get()
// broadcasts one entry with readlane.  Indices are clamped to [0, d_in), so malformed lists cannot address outside the
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

// Strided list blocks (stand-alone and batched GEMV): a wave's list entries are
// first + stride * p for p = 0, 1, ...; lane l of block p0 holds p = p0 + l.  The entry
// indices are fixed before the counts are known, so a block's index loads can be issued
// before (or with) the counts load; an entry index is clamped into the list's capacity
// (d_in entries), so a lane past the wave's count reads a stale but in-bounds entry, which
// finish_blocks drops.
__device__ __forceinline__ uint32_t load_index(const void* __restrict__ idx, int first,
                                               int stride, int p, uint32_t jmax) {
  const int entry = min(first + stride * p, (int)jmax);  // < 2^31: stride * p <= 2^29
  return load_global<uint32_t>(reinterpret_cast<const uint32_t*>(idx) + entry);
}

// The FULL and APPROX blocks from raw index words rF / rA: lanes below nf / na (wave-uniform,
// may be <= 0) keep their entry and gather their activation; the others hold a zero entry.
// kCompact: the words are staging slot | channel << 16.
template <bool kCompact>
__device__ __forceinline__ void finish_blocks(uint32_t rF, uint32_t rA,
                                              const uint16_t* __restrict__ x16, int nf, int na,
                                              uint32_t jmax, int p0, RegBlock& bf,
                                              RegBlock& ba) {
  const int lane = threadIdx.x & 63;
  const uint32_t jF = min(kCompact ? rF >> 16 : rF, jmax), jA = min(kCompact ? rA >> 16 : rA, jmax);
  const uint32_t sF = kCompact ? min(rF & 0xFFFFu, jmax) : jF;
  const uint32_t sA = kCompact ? min(rA & 0xFFFFu, jmax) : jA;
  const uint32_t xF = load_global<uint16_t>(x16 + jF), xA = load_global<uint16_t>(x16 + jA);
  bf = RegBlock{lane < nf ? sF | (xF << 16) : 0u, p0};
  ba = RegBlock{lane < na ? sA | (xA << 16) : 0u, p0};
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

// log2 of a group size (a power of two: 64 or 128 rows), so that a row's group is a shift
// rather than a division by a runtime value (some forty instructions on the path to the first
// column loads).
__device__ __forceinline__ uint32_t log2_group(int32_t g) { return (uint32_t)__builtin_ctz((uint32_t)g); }

// A lane's byte offsets inside a column record for its rows of the tile.
template <int FMT, int RPL = 8>
struct TileOffsets {
  static_assert(RPL == 8 || (RPL == 32 && FMT == SPAX_FMT_INT4), "rows per lane: 8, or 32 for int4");
  uint32_t loffA;   // two-bit codes.  RPL 8: the aligned dword that holds the lane's 2 bytes (a
                    // 16-bit load would be widened right after it is issued, which makes it
                    // wait); RPL 32: the lane's 8 bytes
  uint32_t selA;    // RPL 8: byte selector for those 2 bytes
  uint32_t szoffA;  // (s, z) word of the lane's two-bit group
  uint32_t loffF;   // FULL codes (fp16 rows or int4 codes)
  uint32_t szoffF;  // (s, z) word of the lane's int4 group
  __device__ __forceinline__ TileOffsets(const Shape& sh, int row)
      : loffA(RPL == 8 ? (((uint32_t)row / 4u) & ~3u) : (uint32_t)row / 4u),
        selA(spread_sel(((uint32_t)row / 4u) & 2u)),
        szoffA((uint32_t)sh.T / 4u + ((uint32_t)row >> log2_group(sh.approx_group)) * 4u),
        loffF(FMT == SPAX_FMT_FP16 ? (uint32_t)row * 2u : (uint32_t)row / 2u),
        szoffF((uint32_t)sh.T / 2u + ((uint32_t)row >> log2_group(sh.base_group)) * 4u) {}
};

// The registers of one round: up to U FULL and U APPROX columns.  RPL 8: vf holds a fp16
// column's 8 halves, cf / ca a dword of int4 / two-bit codes.  RPL 32: vf holds 32 int4 codes,
// va 32 two-bit codes (in .x, .y).
template <int FMT, int RPL = 8, int U = kUnroll>
struct RoundLoads {
  float xf[U], xa[U];
  uint4 vf[U];
  uint2 va[U];
  uint32_t cf[U], sf[U], ca[U], sa[U];
};

// Issues the loads of FULL columns [fi, fi + nf) of srcF and APPROX columns [ai, ai + na) of
// srcA (counts wave-uniform, at most U, may be <= 0) from blob b (RegionBlob or RecordBlob).
// Slots past a count keep zero data and a zero activation.
template <int FMT, int RPL = 8, int U = kUnroll, class Blob, class SrcF, class SrcA>
__device__ __forceinline__ void issue_round(const Blob& b, const TileOffsets<FMT, RPL>& g,
                                            const SrcF& srcF, int fi, int nf, const SrcA& srcA,
                                            int ai, int na, RoundLoads<FMT, RPL, U>& r) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    r.xf[u] = 0.0f;
    r.xa[u] = 0.0f;
    r.vf[u] = make_uint4(0u, 0u, 0u, 0u);
    r.va[u] = make_uint2(0u, 0u);
    r.cf[u] = r.sf[u] = r.ca[u] = r.sa[u] = 0u;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (u < nf) {
      int j;
      srcF.get(fi + u, j, r.xf[u]);
      const Column rec = b.full(j);
      if (FMT == SPAX_FMT_FP16 || RPL == 32) {
        r.vf[u] = rec.stream128(g.loffF);
      } else {
        r.cf[u] = rec.stream32(g.loffF);
      }
      if (FMT == SPAX_FMT_INT4) r.sf[u] = rec.word(g.szoffF);
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (u < na) {
      int j;
      srcA.get(ai + u, j, r.xa[u]);
      const Column rec = b.approx(j);
      if (RPL == 32) r.va[u] = rec.stream64(g.loffA);
      else r.ca[u] = rec.stream32(g.loffA);
      r.sa[u] = rec.word(g.szoffA);
    }
  }
}

// Waits for every load of the round and multiplies.  A tier with no column in the round
// skips its multiplies (a wave-uniform branch around whole blocks).  The explicit wait for
// every load makes the branches visible as complete to the compiler's wait tracking, which
// otherwise assumes loads of a skipped block are still in flight in the next round and waits
// for each of them there.
template <int FMT, int RPL = 8, int U = kUnroll>
__device__ __forceinline__ void finish_round(const RoundLoads<FMT, RPL, U>& r,
                                             const TileOffsets<FMT, RPL>& g, int nf, int na,
                                             float (&acc)[RPL], float& zsum) {
  __builtin_amdgcn_s_waitcnt(0);
  if (nf > 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (FMT == SPAX_FMT_FP16) {
        fma_fp16x8(acc, r.xf[u], r.vf[u]);
      } else if (RPL == 8) {
        fma_int4x8(acc, group_terms<4>(r.xf[u], r.sf[u], zsum), r.cf[u]);
      } else {  // 32 rows: dword k of the 16 bytes holds rows 8k .. 8k + 7
        const float a = group_terms<4>(r.xf[u], r.sf[u], zsum);
        fma_int4x8(acc, a, r.vf[u].x);
        fma_int4x8(acc + 8, a, r.vf[u].y);
        fma_int4x8(acc + 16, a, r.vf[u].z);
        fma_int4x8(acc + 24, a, r.vf[u].w);
      }
    }
  }
  if (na > 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (RPL == 8) {
        fma_int2x8(acc, group_terms<2>(r.xa[u], r.sa[u], zsum), r.ca[u], g.selA);
      } else {  // 32 rows: bytes 2k, 2k + 1 of the 8 bytes hold rows 8k .. 8k + 7
        const float a = group_terms<2>(r.xa[u], r.sa[u], zsum);
        fma_int2x8(acc, a, r.va[u].x, spread_sel(0u));
        fma_int2x8(acc + 8, a, r.va[u].x, spread_sel(2u));
        fma_int2x8(acc + 16, a, r.va[u].y, spread_sel(0u));
        fma_int2x8(acc + 24, a, r.va[u].y, spread_sel(2u));
      }
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
template <int FMT, int RPL = 8, int U = kUnroll, class Blob, class SrcF, class SrcA>
__device__ __forceinline__ void stream_columns(const Shape& sh, const Blob& b, int row, int fb,
                                               int fe, const SrcF& srcF, int ab, int ae,
                                               const SrcA& srcA, float (&acc)[RPL],
                                               float& zsum) {
  const TileOffsets<FMT, RPL> g(sh, row);
  int fi = fb, ai = ab;
  while (fi < fe || ai < ae) {
    const int nf = min(fe - fi, U), na = min(ae - ai, U);  // may be <= 0
    RoundLoads<FMT, RPL, U> r;
    issue_round<FMT, RPL, U>(b, g, srcF, fi, nf, srcA, ai, na, r);
    finish_round<FMT, RPL, U>(r, g, nf, na, acc, zsum);
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

// Reduce the NW waves' partial rows through LDS, then write (one chunk) or atomically add
// (several chunks, y zeroed beforehand in stream order) the 64 RPL-row tile into y.  With
// `partials` (deterministic mode, several chunks) the tile is stored as row block `chunk` of
// partials[n_chunks][T] instead, for a later pass that adds the chunks in a fixed order.
template <int NW, int RPL = 8>
__device__ __forceinline__ void finish_tile(float (*red)[64 * RPL], const float (&acc)[RPL],
                                            float zsum, int wave, int lane, int row0, int T,
                                            int n_chunks, float* __restrict__ y,
                                            float* __restrict__ partials = nullptr,
                                            int chunk = 0) {
  constexpr int kRows = 64 * RPL;
  float4* dst = reinterpret_cast<float4*>(&red[wave][lane * RPL]);
#pragma unroll
  for (int q = 0; q < RPL / 4; ++q)
    dst[q] = make_float4(acc[4 * q] + zsum, acc[4 * q + 1] + zsum, acc[4 * q + 2] + zsum,
                         acc[4 * q + 3] + zsum);
  __syncthreads();
  for (int r = (int)threadIdx.x; r < kRows; r += NW * 64) {
    const int grow = row0 + r;
    if (grow < T) {
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) sum += red[w][r];
      // Several chunks meet through hardware fp32 atomics at device scope; y is read only
      // after the kernel ends, so no device-scope fence is needed.
      if (n_chunks == 1) y[grow] = sum;
      else if (partials) partials[(size_t)chunk * (size_t)T + (size_t)grow] = sum;
      else unsafeAtomicAdd(&y[grow], sum);
    }
  }
}

// Rows per lane and columns per round of the batched GEMV for a base format (tile = 64 RPL
// rows; the host's batched_tile_rows gives the same tile).  int4: 32 rows per lane, so a wave
// keeps four times the bytes in flight per column; 4 columns per round (6 and 8 measured
// slower: more registers, fewer resident waves).
template <int FMT>
struct ItemRows {
  static constexpr int rpl = FMT == SPAX_FMT_INT4 ? 32 : 8;
  static constexpr int tile = 64 * rpl;
  static constexpr int unroll = kUnroll;
};

// One work item of the stand-alone (and batched) GEMV: row tile `tile`, column chunk `chunk`
// of the lists in global memory -- the entries chunk, chunk + n_chunks, ... -- (counts
// clamped to [0, d_in] and channels to [0, d_in), so malformed lists cannot address outside
// the blob).  kCompact: the lists hold slot | channel << 16 entries into a compacted
// staging copy of the records (`packed` is then the staging buffer).  A workgroup
// of kWaves waves; RPL rows per lane (a 64 RPL-row tile), U columns per round; ends after the
// tile's atomics.  red: kWaves x 64 RPL floats.  Blob: RegionBlob or RecordBlob.
template <int FMT, class Blob, bool kCompact = false, int RPL = 8, int U = kUnroll>
__device__ __forceinline__ void gemv_item(const Shape& sh, const uint8_t* __restrict__ packed,
                                          const uint32_t* __restrict__ x32,
                                          const int32_t* __restrict__ full_idx,
                                          const int32_t* __restrict__ approx_idx,
                                          const int32_t* __restrict__ counts,
                                          float* __restrict__ y, int tile, int chunk,
                                          float* red, float* __restrict__ partials = nullptr) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int T = sh.T;
  const int row0 = tile * 64 * RPL;
  // Lanes past the last row (ragged last tile) read the record's first rows instead, which
  // is always in bounds; their sums land in rows >= T and are never stored.  Every matrix
  // height is a multiple of 64, so a lane's rows are all inside or all past T.
  const int row = row0 + lane * RPL < T ? row0 + lane * RPL : 0;
  const uint32_t jmax = (uint32_t)sh.d_in - 1u;
  // Chunk c takes the list entries c, c + n_chunks, c + 2 n_chunks, ... and wave w of the
  // workgroup every kWaves-th of those, so this wave's entries are first + stride * p.  The
  // first block's index loads go out with the counts load; the counts only fix how many of
  // the entries are valid.  Every chunk and every wave gets the same count within one.
  const int stride = sh.n_chunks * kWaves;
  const int first = chunk + sh.n_chunks * wave;
  uint32_t rF = load_index(full_idx, first, stride, lane, jmax);
  uint32_t rA = load_index(approx_idx, first, stride, lane, jmax);
  const int nF = uniform(min(max(load_global<int32_t>(counts), 0), sh.d_in));
  const int nA = uniform(min(max(load_global<int32_t>(counts + 1), 0), sh.d_in));
  const int cF = nF > first ? (nF - first + stride - 1) / stride : 0;  // this wave's entries
  const int cA = nA > first ? (nA - first + stride - 1) / stride : 0;
  float acc[RPL];
#pragma unroll
  for (int h = 0; h < RPL; ++h) acc[h] = 0.0f;
  float zsum = 0.0f;
  const uint16_t* x16 = reinterpret_cast<const uint16_t*>(x32);
  const Blob b(sh, packed);
  // 64 list entries per tier and block; the channels fit the 16-bit entry field (d_in <= 32768)
  for (int p0 = 0; p0 < cF || p0 < cA; p0 += 64) {
    if (p0 > 0) {
      rF = load_index(full_idx, first, stride, p0 + lane, jmax);
      rA = load_index(approx_idx, first, stride, p0 + lane, jmax);
    }
    const int nf = min(cF - p0, 64), na = min(cA - p0, 64);  // may be <= 0
    RegBlock bf, ba;
    finish_blocks<kCompact>(rF, rA, x16, nf, na, jmax, p0, bf, ba);
    stream_columns<FMT, RPL, U>(sh, b, row, p0, p0 + max(nf, 0), bf, p0, p0 + max(na, 0), ba,
                                acc, zsum);
  }
  finish_tile<kWaves, RPL>(reinterpret_cast<float(*)[64 * RPL]>(red), acc, zsum, wave, lane,
                           row0, T, sh.n_chunks, y, partials, chunk);
}

}  // namespace gemv
}  // namespace spax
