// Packing of fp16 weight columns into the column-major blob (original tier + two-bit
// approximation), one pass over the weights.
//
// Pages: eigenradar commentary on SpAx, "The route outside GPU memory", first paragraph
// (original and two-bit approximate form of every column) and third paragraph (jointly
// accessed columns stored together).  Quantizer: per group of G rows, z = min, s =
// (max-min)/L rounded to fp16, q = round-half-even((w - z)/s) clamped to [0, L]; every step
// fp32 with round-to-nearest-even and a correctly rounded division, so that the codes are
// a deterministic function of the weights.
//
// Placement (optional): record j may hold column perm[j], so that columns used together by
// the same tokens sit next to each other (eigenradar commentary, third paragraph).
//
// Thread mapping: one lane per (column j, 8 consecutive fused rows).  A quantization group
// of G rows is G/8 consecutive lanes; since every matrix height is a multiple of G, the
// lanes of one group are aligned inside the wavefront and reduce min/max with xor
// shuffles over G/8 lanes.
#include "common.h"

namespace spax {
namespace {

struct PackArgs {
  const uint16_t* W[SPAX_MAX_MATS];
  const int32_t* perm;  // record j packs column perm[j] (NULL: column j)
  uint8_t* packed;
  int32_t row_off[SPAX_MAX_MATS + 1];  // fused row where matrix m starts
  int32_t n_mats;
  int32_t d_in;
  int32_t T;             // d_out_total
  int32_t base_fmt;
  int32_t base_group;    // int4 group rows
  int32_t approx_group;  // two-bit group rows
  int64_t stride_F, stride_A, off_A;
  int32_t rec_F, rec_A;  // unpadded record bytes (multiples of 4)
};

// min/max over `lanes` aligned lanes (8 or 16); every lane of the wave takes part.
__device__ __forceinline__ void group_minmax(float& lo, float& hi, int lanes) {
  for (int m = 1; m < lanes; m <<= 1) {
    lo = fminf(lo, __shfl_xor(lo, m, 64));
    hi = fmaxf(hi, __shfl_xor(hi, m, 64));
  }
}

struct Quant {
  float s, z;      // fp16-rounded scale and zero, as fp32
  uint32_t word;   // fp16 s in [15:0], fp16 z in [31:16]
};

__device__ __forceinline__ Quant make_quant(float lo, float hi, float levels) {
  Quant q;
  float z32 = lo + 0.0f;          // -0 becomes +0
  float rng = hi - lo;
  float s32 = rng / levels;       // correctly rounded fp32 division
  _Float16 s16 = (_Float16)s32;   // round to nearest even
  _Float16 z16 = (_Float16)z32;   // exact: lo is an fp16 value
  q.s = (float)s16;
  q.z = (float)z16;
  q.word = (uint32_t)__builtin_bit_cast(uint16_t, s16) |
           ((uint32_t)__builtin_bit_cast(uint16_t, z16) << 16);
  return q;
}

__device__ __forceinline__ uint32_t code_of(float w, const Quant& q, float levels) {
  if (q.s == 0.0f) return 0u;
  float t = (w - q.z) / q.s;
  float r = rintf(t);
  r = fminf(fmaxf(r, 0.0f), levels);
  return (uint32_t)r;
}

__global__ __launch_bounds__(256) void pack_columns_kernel(PackArgs a) {
  const int64_t T8 = a.T / 8;
  const int64_t total = (int64_t)a.d_in * T8;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool active = gid < total;
  const int64_t j = active ? gid / T8 : 0;
  const int32_t c = active ? (int32_t)(gid - j * T8) : 0;
  const int32_t r0 = c * 8;

  int m = 0;
  while (m + 1 < a.n_mats && r0 >= a.row_off[m + 1]) ++m;
  const int64_t rows_m = a.row_off[m + 1] - a.row_off[m];
  const int64_t lr = r0 - a.row_off[m];

  // the source column of record j; clamped so that a malformed permutation stays in bounds
  const int64_t src = a.perm ? (int64_t)min(max(a.perm[j], 0), a.d_in - 1) : j;
  uint4 raw = make_uint4(0, 0, 0, 0);
  if (active) raw = *reinterpret_cast<const uint4*>(a.W[m] + src * rows_m + lr);
  const uint32_t words[4] = {raw.x, raw.y, raw.z, raw.w};
  float w[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    w[2 * k] = (float)__builtin_bit_cast(_Float16, (uint16_t)(words[k] & 0xFFFFu));
    w[2 * k + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(words[k] >> 16));
  }
  float lo = w[0], hi = w[0];
#pragma unroll
  for (int k = 1; k < 8; ++k) {
    lo = fminf(lo, w[k]);
    hi = fmaxf(hi, w[k]);
  }

  uint8_t* recF = a.packed + j * a.stride_F;
  uint8_t* recA = a.packed + a.off_A + j * a.stride_A;

  // ---------------- region F: the original column
  if (a.base_fmt == SPAX_FMT_FP16) {
    if (active) *reinterpret_cast<uint4*>(recF + (int64_t)r0 * 2) = raw;
  } else {
    float glo = lo, ghi = hi;
    group_minmax(glo, ghi, a.base_group / 8);
    const Quant q = make_quant(glo, ghi, 15.0f);
    uint32_t packed4 = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) packed4 |= code_of(w[k], q, 15.0f) << (4 * k);
    if (active) {
      *reinterpret_cast<uint32_t*>(recF + r0 / 2) = packed4;
      if ((r0 % a.base_group) == 0)
        *reinterpret_cast<uint32_t*>(recF + a.T / 2 + (r0 / a.base_group) * 4) = q.word;
    }
  }

  // ---------------- region A: the two-bit approximation of the fp16 column
  {
    float glo = lo, ghi = hi;
    group_minmax(glo, ghi, a.approx_group / 8);
    const Quant q = make_quant(glo, ghi, 3.0f);
    uint32_t packed2 = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) packed2 |= code_of(w[k], q, 3.0f) << (2 * k);
    if (active) {
      *reinterpret_cast<uint16_t*>(recA + r0 / 4) = (uint16_t)packed2;
      if ((r0 % a.approx_group) == 0)
        *reinterpret_cast<uint32_t*>(recA + a.T / 4 + (r0 / a.approx_group) * 4) = q.word;
    }
  }

  // ---------------- zero padding after each record (dword granularity)
  if (active) {
    const int32_t padF = (int32_t)((a.stride_F - a.rec_F) / 4);
    const int32_t padA = (int32_t)((a.stride_A - a.rec_A) / 4);
    for (int32_t k = c; k < padF; k += (int32_t)T8)
      *reinterpret_cast<uint32_t*>(recF + a.rec_F + 4 * k) = 0u;
    for (int32_t k = c; k < padA; k += (int32_t)T8)
      *reinterpret_cast<uint32_t*>(recA + a.rec_A + 4 * k) = 0u;
  }
}

}  // namespace

int launch_pack(const spax_layout* L, const uint16_t* const* W, const int32_t* perm,
                void* packed, hipStream_t s) {
  PackArgs a{};
  a.perm = perm;
  a.packed = static_cast<uint8_t*>(packed);
  a.n_mats = L->n_mats;
  a.d_in = L->d_in;
  a.T = (int32_t)L->d_out_total;
  a.base_fmt = L->base_fmt;
  a.base_group = L->base_group;
  a.approx_group = L->approx_group;
  a.stride_F = L->stride_F;
  a.stride_A = L->stride_A;
  a.off_A = L->off_A;
  a.rec_F = (int32_t)L->rec_F;
  a.rec_A = (int32_t)L->rec_A;
  int32_t off = 0;
  for (int m = 0; m < SPAX_MAX_MATS; ++m) {
    a.W[m] = m < L->n_mats ? W[m] : nullptr;
    a.row_off[m] = off;
    if (m < L->n_mats) off += L->d_out[m];
  }
  a.row_off[SPAX_MAX_MATS] = off;
  for (int m = L->n_mats; m <= SPAX_MAX_MATS; ++m) a.row_off[m] = off;

  const int64_t total = (int64_t)L->d_in * (L->d_out_total / 8);
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(pack_columns_kernel, dim3((unsigned)blocks), dim3(threads), 0, s, a);
  SPAX_HIP_CHECK(hipGetLastError());
  return SPAX_OK;
}

}  // namespace spax
