// A read-bandwidth probe for the benchmark (include/pa_profile.h): every
// byte of a buffer is read once with non-temporal 16-byte loads, as the
// decode kernels read K/V, and nothing is written. It measures what this GPU
// sustains for a plain read stream, the practical ceiling of a read-bound
// kernel, beside the 8 TB/s of the data sheet.
#include <algorithm>

#include "pa_profile.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;  // 16-byte loads in flight per lane

// `never` is 0 at every call; the store it guards keeps the loads from being
// removed and is never executed.
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4* __restrict__ p, uint64_t n16,
                                                                   uint32_t* sink, int never) {
  uint32_t acc = 0;
  const uint64_t step = uint64_t(gridDim.x) * kProbeThreads * kProbeUnroll;
  for (uint64_t base = uint64_t(blockIdx.x) * kProbeThreads * kProbeUnroll + threadIdx.x; base < n16; base += step) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int j = 0; j < kProbeUnroll; ++j) {
      const uint64_t i = base + uint64_t(j) * kProbeThreads;
      v[j] = i < n16 ? __builtin_nontemporal_load(p + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < kProbeUnroll; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
  }
  if (never) sink[uint64_t(blockIdx.x) * kProbeThreads + threadIdx.x] = acc;
}

}  // namespace
}  // namespace pa

extern "C" int pa_profile_read_probe(const void* buf, uint64_t bytes, void* stream) {
  if (!buf || bytes < 16 || bytes % 16 || reinterpret_cast<uintptr_t>(buf) % 16) return PA_ERR_SHAPE;
  const uint64_t n16 = bytes / 16;
  // enough workgroups to keep every CU busy several times over
  const uint64_t per_wg = uint64_t(pa::kProbeThreads) * pa::kProbeUnroll;
  const unsigned grid = static_cast<unsigned>(std::min<uint64_t>((n16 + per_wg - 1) / per_wg, 256 * 32));
  hipLaunchKernelGGL(pa::read_probe_kernel, dim3(grid), dim3(pa::kProbeThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const pa::u32x4*>(buf), n16, const_cast<uint32_t*>(static_cast<const uint32_t*>(buf)), 0);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}
