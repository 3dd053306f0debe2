// The bf16 matrix-core rate the chip sustains, the practical ceiling the
// grouped GEMMs' MFMA figures are read against next to the nominal peak:
// v_mfma_f32_32x32x16_bf16 on register operands, with no memory traffic in
// the timed loop.  One workgroup of 8 waves per CU (two per SIMD, as in the
// LDS-pipelined GEMM; 96 KB of dynamic LDS keep a second workgroup off the
// CU), each wave four independent accumulator chains.  Wave 0 of each
// workgroup records the shader-clock counter (s_memtime) and the 100 MHz
// real-time counter (s_memrealtime) around its loop, so the clock the
// matrix cores ran at follows from their ratio.  The accumulators go to
// `sink` only if their sum equals a value these operands never give.
#include "smoe_internal.h"

namespace smoe {

typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(512) void mfma_probe_kernel(int iters, unsigned long long* clocks,
                                                         float* sink) {
  const int lane = threadIdx.x & 63;
  // operands of small exact bf16 values: 2^-8 * (1 + lane % 8 / 8)
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.00390625f * (1.0f + (float)((lane + i) & 7) * 0.125f));
    b[i] = (__bf16)(0.00390625f * (1.0f + (float)((lane * 3 + i) & 7) * 0.125f));
  }
  f32x16 acc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[k][j] = 0.f;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[k][j];
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = t1 - t0;
    clocks[2 * blockIdx.x + 1] = r1 - r0;
  }
  if (s == -1.0f) sink[threadIdx.x & 3] = s;   // the sum is positive
}

hipError_t launch_mfma_probe(int iters, int grid, unsigned long long* clocks, void* sink,
                             hipStream_t s) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(grid), dim3(512), 96 * 1024, s, iters, clocks,
                     static_cast<float*>(sink));
  return hipGetLastError();
}

}  // namespace smoe
