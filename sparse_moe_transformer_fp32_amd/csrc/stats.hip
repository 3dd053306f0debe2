// Per-expert activation statistics of the SwiGLU output h.
//
// Sources: paperlayer.ai summary, §4.1.2 (monitor per-expert activation
// norms; a falling minimum-to-median ratio warns of expert death) and §4.1.3
// (the maximum-to-median activation-norm ratio exposes localized blow-up
// that the loss hides); App. B (the abnormal values appear in the SwiGLU
// product of gate and up activations, which is h).
//
// For group g (routed expert g < E, or the shared expert g = E) with rows
// R_g, and ||h_r|| the L2 norm of row r of h as stored (bf16):
//   stats[4g + 0] = |R_g|
//   stats[4g + 1] = sum_r ||h_r||
//   stats[4g + 2] = sum_r ||h_r||^2
//   stats[4g + 3] = max_r ||h_r||          (0 for an empty group)
// Over the routed experts with rows, with m_e = stats[4e+1] / stats[4e]
// (the mean activation norm of expert e) and M their median (the mean of
// the two middle values for an even count):
//   ratios[0] = max_e m_e / M,   ratios[1] = min_e m_e / M.
// Every sum runs in a fixed order, so the statistics are deterministic.
#include "smoe_internal.h"

namespace smoe {

// One workgroup per group; wave w takes rows w, w+4, ... of the group; a
// row's squares are summed per lane over its 8-column chunks, then across
// the wave by a fixed butterfly; the four waves' totals are added in order.
__global__ __launch_bounds__(256) void expert_stats_kernel(const int32_t* __restrict__ offsets,
                                                           const uint16_t* __restrict__ h,
                                                           float* __restrict__ stats, int T,
                                                           int E, int KT, int I, int Is) {
  __shared__ float s_red[4][3];
  const int grp = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int r0, n, W;
  const uint16_t* base;
  if (grp < E) {
    r0 = offsets[grp];
    n = offsets[grp + 1] - r0;
    W = I;
    base = h + (size_t)r0 * I;
  } else {
    r0 = KT;
    n = T;
    W = Is;
    base = h + (size_t)KT * I;
  }
  const int chunks = W >> 3;
  float s1 = 0.f, s2 = 0.f, mx = 0.f;
  for (int i = wave; i < n; i += 4) {
    const uint16_t* row = base + (size_t)i * W;
    float ss = 0.f;
    for (int c = lane; c < chunks; c += 64) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(row + 8 * c);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float a = __uint_as_float(v[k] << 16), b = __uint_as_float(v[k] & 0xffff0000u);
        ss += a * a;
        ss += b * b;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    const float nr = sqrtf(ss);
    s1 += nr;
    s2 += ss;
    mx = fmaxf(mx, nr);
  }
  if (lane == 0) {
    s_red[wave][0] = s1;
    s_red[wave][1] = s2;
    s_red[wave][2] = mx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float a = 0.f, b = 0.f, m = 0.f;
    for (int w = 0; w < 4; ++w) {
      a += s_red[w][0];
      b += s_red[w][1];
      m = fmaxf(m, s_red[w][2]);
    }
    float4 out;
    out.x = (float)n;
    out.y = a;
    out.z = b;
    out.w = m;
    *reinterpret_cast<float4*>(stats + 4 * grp) = out;
  }
}

// One workgroup of 1024 threads (E <= 1024): thread e holds m_e; its rank
// among the experts with rows (ties by index) finds the median, the minimum
// and the maximum without a sort.
__global__ __launch_bounds__(1024) void norm_ratio_kernel(const float* __restrict__ stats, int E,
                                                          float* __restrict__ ratios) {
  __shared__ float s_m[1024];
  __shared__ int s_act[1024];
  __shared__ float s_pick[4];  // lower median, upper median, min, max
  const int e = threadIdx.x;
  float m = 0.f;
  int act = 0;
  if (e < E) {
    const float cnt = stats[4 * e];
    if (cnt > 0.f) {
      act = 1;
      m = stats[4 * e + 1] / cnt;
    }
  }
  s_m[e] = m;
  s_act[e] = act;
  const int n_act = __syncthreads_count(act);
  if (act) {
    int rank = 0;
    for (int j = 0; j < E; ++j)
      if (s_act[j] && (s_m[j] < m || (s_m[j] == m && j < e))) ++rank;
    if (rank == (n_act - 1) / 2) s_pick[0] = m;
    if (rank == n_act / 2) s_pick[1] = m;
    if (rank == 0) s_pick[2] = m;
    if (rank == n_act - 1) s_pick[3] = m;
  }
  __syncthreads();
  if (e == 0) {
    if (n_act == 0) {
      ratios[0] = ratios[1] = 0.f;
    } else {
      const float med = 0.5f * (s_pick[0] + s_pick[1]);
      ratios[0] = s_pick[3] / med;
      ratios[1] = s_pick[2] / med;
    }
  }
}

hipError_t launch_expert_stats(int T, int E, int K, int I, int Is, const int32_t* offsets,
                               const uint16_t* h, float* stats, float* ratios, hipStream_t s) {
  const int groups = E + (Is > 0 ? 1 : 0);
  hipLaunchKernelGGL(expert_stats_kernel, dim3(groups), dim3(256), 0, s, offsets, h, stats, T, E,
                     T * K, I, Is);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ratios) hipLaunchKernelGGL(norm_ratio_kernel, dim3(1), dim3(1024), 0, s, stats, E, ratios);
  return hipGetLastError();
}

}  // namespace smoe
