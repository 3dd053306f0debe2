// The HBM read ceiling that the weight streams are measured against: a plain
// read of a device buffer with 16-byte loads, ordinary or non-temporal.
// Each thread keeps four loads in flight per iteration of a grid-stride loop
// (a 256-thread workgroup reads 16 KB contiguous per iteration; consecutive
// workgroups read neighbouring blocks) and folds them into one word, which
// goes to `sink` only if it equals a value no input makes (so the loads stay
// and nothing is written).
#include "smoe_internal.h"

namespace smoe {

template <bool NT>
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4* __restrict__ p, size_t n,
                                                         u32x4* __restrict__ sink) {
  constexpr int U = 4;
  const size_t stride = (size_t)gridDim.x * 256 * U;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t i = (size_t)blockIdx.x * 256 * U + threadIdx.x; i + 256 * (U - 1) < n; i += stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = NT ? __builtin_nontemporal_load(p + i + 256 * u) : p[i + 256 * u];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  if (acc[0] == 0x9e3779b9u && acc[1] == 0x7f4a7c15u && acc[2] == 0xf39cc060u &&
      acc[3] == 0x5cedc834u)
    sink[0] = acc;
}

// two workgroups per CU
hipError_t launch_read_probe(const void* buf, size_t bytes, bool nontemporal, void* sink,
                             hipStream_t s) {
  int dev = 0, cus = 256;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const size_t n = bytes / 16;
  const auto* p = static_cast<const u32x4*>(buf);
  auto* out = static_cast<u32x4*>(sink);
  if (nontemporal)
    hipLaunchKernelGGL(read_probe_kernel<true>, dim3(2 * cus), dim3(256), 0, s, p, n, out);
  else
    hipLaunchKernelGGL(read_probe_kernel<false>, dim3(2 * cus), dim3(256), 0, s, p, n, out);
  return hipGetLastError();
}

}  // namespace smoe
