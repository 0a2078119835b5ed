// A plain streaming read over the whole GPU (spax_read_probe): a measuring stick for the
// kernels of the method, not a step of it.  Threads read 16-byte words with non-temporal
// loads, several in flight per round, and XOR them together; every wave stores its XOR in
// its own word of `out` (no atomics), so the reads cannot be dropped and the result can be
// checked.  Two launch shapes, picked by size (measured on MI355X): a large read goes best
// as one contiguous chunk per workgroup, one workgroup per compute unit; a read of tens of
// MB, as one launch among many, ends soonest grid-stride over four workgroups per unit.
#include <atomic>

#include "common.h"

namespace spax {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 512;
constexpr int kProbeWaves = kProbeThreads / 64;
constexpr int kProbeMaxDevices = 64;
constexpr size_t kProbeChunkedFrom = size_t(1) << 30;  // bytes

template <int U, bool CHUNKED>
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4* __restrict__ p,
                                                                   int64_t n, uint32_t* out) {
  // CHUNKED: workgroup b owns elements [b * per, (b + 1) * per); rounds of U * 512 elements.
  // Otherwise: element i, i + stride, ... over the whole grid.
  int64_t i, step, end;
  if (CHUNKED) {
    const int64_t per = (n + gridDim.x - 1) / gridDim.x;
    const int64_t b0 = (int64_t)blockIdx.x * per;
    end = b0 + per < n ? b0 + per : n;
    i = b0 + threadIdx.x;
    step = kProbeThreads;
  } else {
    end = n;
    i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
    step = (int64_t)gridDim.x * kProbeThreads;
  }
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (U - 1) * step < end; i += U * step) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * step);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  for (; i < end; i += step) acc ^= __builtin_nontemporal_load(p + i);
  uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
  for (int o = 32; o > 0; o >>= 1) r ^= (uint32_t)__shfl_xor((int)r, o);
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * kProbeWaves + (threadIdx.x >> 6)] = r;
}

int probe_cus() {
  static std::atomic<int> cache[kProbeMaxDevices];  // filled once per device, same value
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  int cus = dev < kProbeMaxDevices ? cache[dev].load(std::memory_order_relaxed) : 0;
  if (cus <= 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
      cus = 256;
    if (dev < kProbeMaxDevices) cache[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

}  // namespace
}  // namespace spax

extern "C" int spax_read_probe(const void* p, size_t bytes, uint32_t* out, int32_t out_words,
                               int32_t* n_written, hipStream_t stream) {
  using namespace spax;
  clear_error();
  if (n_written) *n_written = 0;
  if (bytes == 0) return SPAX_OK;
  if (!p || !out) return fail(SPAX_ERR_NULL, "p and out are required");
  if ((reinterpret_cast<uintptr_t>(p) & 15u) != 0 || (bytes & 15u) != 0)
    return fail(SPAX_ERR_ALIGN, "p and bytes must be multiples of 16");
  if ((reinterpret_cast<uintptr_t>(out) & 3u) != 0)
    return fail(SPAX_ERR_ALIGN, "out must be 4-byte aligned");
  if (out_words < kProbeWaves)
    return fail(SPAX_ERR_PARAM, "out_words %d < %d (one workgroup's waves)", out_words,
                kProbeWaves);
  const int64_t n16 = (int64_t)(bytes / 16);
  const bool chunked = bytes >= kProbeChunkedFrom;
  const int64_t want = (int64_t)probe_cus() * (chunked ? 1 : 4);
  const int64_t need = (n16 + kProbeThreads - 1) / kProbeThreads;
  int64_t grid = want < need ? want : need;
  if (grid > out_words / kProbeWaves) grid = out_words / kProbeWaves;
  if (grid < 1) grid = 1;
  const dim3 g((unsigned)grid), b(kProbeThreads);
  const u32x4* src = reinterpret_cast<const u32x4*>(p);
  if (chunked)
    hipLaunchKernelGGL((read_probe_kernel<4, true>), g, b, 0, stream, src, n16, out);
  else
    hipLaunchKernelGGL((read_probe_kernel<8, false>), g, b, 0, stream, src, n16, out);
  SPAX_HIP_CHECK(hipGetLastError());
  if (n_written) *n_written = (int32_t)(grid * kProbeWaves);
  return SPAX_OK;
}
