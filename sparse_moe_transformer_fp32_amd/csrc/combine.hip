// Combine (un-permute), the residual + RMSNorm glue between chained layers,
// and the two fused into one pass.
//
// Sources: shd-paper.top summary, 方法详解 / 关键设计 (the selected experts'
// outputs are mixed with the gate weights); hyper.ai summary, 方法 (one
// always-on shared expert per MoE layer); paperlayer.ai summary, App. B
// (RMSNorm over the summed layer outputs); LLM Atlas model card
// "Step-3.5-Flash", raw config field table: zero_centered.
#include "smoe_internal.h"

namespace smoe {

__device__ inline void bf16x8_to_f32(const u32x4& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
  }
}

__device__ inline uint32_t pack2(float a, float b) {
  const __bf16 ha = (__bf16)a, hb = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) |
         ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

// The K slot rows of token t, then their 8 columns at c: all loads issued
// before the first add (K <= 16, uniform), so a thread waits for one memory
// latency instead of K.  Every expert row is read once, here: the loads are
// non-temporal (they stream from HBM faster than ordinary loads).  The same
// holds for the fused kernel's expert rows and residual input.
__device__ inline void load_slots(const uint16_t* __restrict__ o,
                                  const int32_t* __restrict__ slot_pos, int t, int K, int H,
                                  int c, u32x4 (&v)[16]) {
  int rows[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) rows[j] = j < K ? slot_pos[(size_t)t * K + j] : 0;
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (j < K) v[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(o + (size_t)rows[j] * H + c));
}

// y[t] = sum_j o[slot_pos[t,j]] + o[KT + t]: rows already carry their
// weights.  fp32 sum in slot order, shared expert last, one rounding.  No
// atomics: each thread owns 8 columns of one token.
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ o,
                                                      const int32_t* __restrict__ slot_pos,
                                                      uint16_t* __restrict__ y, int T, int H,
                                                      int K, int KT, int has_shared) {
  const int t = blockIdx.x;
  const int c = (blockIdx.y * 256 + threadIdx.x) * 8;
  if (c >= H) return;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  u32x4 v[16];
  load_slots(o, slot_pos, t, K, H, c, v);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j < K) {
      float f[8];
      bf16x8_to_f32(v[j], f);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += f[i];
    }
  }
  if (has_shared) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(o + (size_t)(KT + t) * H + c));
    float f[8];
    bf16x8_to_f32(v, f);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += f[i];
  }
  u32x4 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = pack2(acc[2 * i], acc[2 * i + 1]);
  *reinterpret_cast<u32x4*>(y + (size_t)t * H + c) = out;
}

// One workgroup per row of min(1024, H/8) threads (rounded up to whole
// waves): one chunk of 8 columns per thread up to H = 8192, two above.  (A
// 256-thread workgroup with the row's chunks taken one after another per
// thread left the loads of a thread's second chunk waiting on its first.)
//   FUSED = false:  r = r_in (+ y_add)
//   FUSED = true:   r = r_in + (sum_j o[slot_pos[t,j]] + o[KT + t]), the
//                   combine of the layer folded into the residual add: the
//                   layer output is summed in fp32 in slot order (shared
//                   last) and added to r_in before the one rounding to bf16.
// r is stored to r_out as bf16; then x_out = bf16(r / sqrt(mean(r^2) + eps)
// * (1 + gamma)) from the stored bf16 r, the sum of squares reduced in a
// fixed order (within each wave by shuffles, then the wave partials in wave
// order).  Each element of r_in/r_out is read and written by the same
// thread, so r_out may alias r_in.  r_out and x_out are written with
// non-temporal stores: every byte is written once and the rows stream out
// (faster here; in the combine kernel above the same store was not).
struct ResidualArgs {
  const uint16_t* r_in;
  const uint16_t* y_add;     // FUSED = false; may be null
  const uint16_t* o;         // FUSED = true: weighted expert rows [rows_total, H]
  const int32_t* slot_pos;   // FUSED = true: [T, K]
  const float* gamma;        // [H] or null (gain 1)
  float eps;
  uint16_t* r_out;           // may be null when nothing is added
  uint16_t* x_out;           // may be null (no norm)
  int H, K, KT, has_shared;
};

template <bool FUSED>
__global__ __launch_bounds__(1024) void residual_rmsnorm_kernel(ResidualArgs a) {
  __shared__ float s_part[16];
  const int nt = blockDim.x;
  const int t = blockIdx.x;
  const int H = a.H;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float ss = 0.f;
  float v[2][8];  // H <= 16384, nt = min(1024, H / 8): at most 2 chunks per thread
#pragma unroll
  for (int ch = 0; ch < 2; ++ch) {
    const int c = (ch * nt + threadIdx.x) * 8;
    if (c < H) {
      const u32x4 rin = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.r_in + (size_t)t * H + c));
      float f[8];
      bf16x8_to_f32(rin, f);
      bool add = false;
      float y[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = 0.f;
      if (FUSED) {
        // slot rows 8 at a time (all of them for K = 8): their loads in
        // flight together, then added in slot order.  Batches of 16 raise
        // register use and lower occupancy, and were slower; batches of 4
        // were no faster.
        add = true;
#pragma unroll
        for (int j0 = 0; j0 < 16; j0 += 8) {
          if (j0 < a.K) {
            u32x4 ov[8];
#pragma unroll
            for (int jj = 0; jj < 8; ++jj)
              if (j0 + jj < a.K)
                ov[jj] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                    a.o + (size_t)a.slot_pos[(size_t)t * a.K + j0 + jj] * H + c));
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
              if (j0 + jj < a.K) {
                float fo[8];
                bf16x8_to_f32(ov[jj], fo);
#pragma unroll
                for (int i = 0; i < 8; ++i) y[i] += fo[i];
              }
            }
          }
        }
        if (a.has_shared) {
          float fo[8];
          bf16x8_to_f32(__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.o + (size_t)(a.KT + t) * H + c)), fo);
#pragma unroll
          for (int i = 0; i < 8; ++i) y[i] += fo[i];
        }
      } else if (a.y_add) {
        add = true;
        bf16x8_to_f32(*reinterpret_cast<const u32x4*>(a.y_add + (size_t)t * H + c), y);
      }
      if (add) {
        u32x4 pk;
#pragma unroll
        for (int i = 0; i < 4; ++i) pk[i] = pack2(f[2 * i] + y[2 * i], f[2 * i + 1] + y[2 * i + 1]);
        if (a.r_out) __builtin_nontemporal_store(pk, reinterpret_cast<u32x4*>(a.r_out + (size_t)t * H + c));
        bf16x8_to_f32(pk, f);  // continue from the stored bf16 value
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[ch][i] = f[i];
        ss += f[i] * f[i];
      }
    }
  }
  if (!a.x_out) return;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  if (lane == 0) s_part[wave] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int w = 0; w < nt / 64; ++w) tot += s_part[w];
  const float inv = 1.0f / sqrtf(tot / (float)H + a.eps);
#pragma unroll
  for (int ch = 0; ch < 2; ++ch) {
    const int c = (ch * nt + threadIdx.x) * 8;
    if (c < H) {
      u32x4 pk;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float g0 = 1.f, g1 = 1.f;
        if (a.gamma) {
          g0 += a.gamma[c + 2 * i];
          g1 += a.gamma[c + 2 * i + 1];
        }
        pk[i] = pack2(v[ch][2 * i] * inv * g0, v[ch][2 * i + 1] * inv * g1);
      }
      __builtin_nontemporal_store(pk, reinterpret_cast<u32x4*>(a.x_out + (size_t)t * H + c));
    }
  }
}

hipError_t launch_combine(const Plan& p, const uint16_t* o, const int32_t* slot_pos,
                          uint16_t* y, hipStream_t s) {
  dim3 grid(p.T, (p.H / 8 + 255) / 256);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, s, o, slot_pos, y, p.T, p.H, p.K, p.KT,
                     p.Is > 0 ? 1 : 0);
  return hipGetLastError();
}

// one chunk of 8 columns per thread up to H = 8192, two above
static int residual_threads(int H) {
  const int n = (H / 8 + 63) / 64 * 64;
  return n < 1024 ? n : 1024;
}

hipError_t launch_residual_rmsnorm(int T, int H, const uint16_t* r_in, const uint16_t* y_add,
                                   const float* gamma, float eps, uint16_t* r_out,
                                   uint16_t* x_out, hipStream_t s) {
  ResidualArgs a{};
  a.r_in = r_in; a.y_add = y_add; a.gamma = gamma; a.eps = eps;
  a.r_out = r_out; a.x_out = x_out; a.H = H;
  hipLaunchKernelGGL(residual_rmsnorm_kernel<false>, dim3(T), dim3(residual_threads(H)), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_combine_residual(const Plan& p, const uint16_t* o, const int32_t* slot_pos,
                                   const uint16_t* r_in, const float* gamma, float eps,
                                   uint16_t* r_out, uint16_t* x_out, hipStream_t s) {
  ResidualArgs a{};
  a.r_in = r_in; a.o = o; a.slot_pos = slot_pos; a.gamma = gamma; a.eps = eps;
  a.r_out = r_out; a.x_out = x_out;
  a.H = p.H; a.K = p.K; a.KT = p.KT; a.has_shared = p.Is > 0 ? 1 : 0;
  hipLaunchKernelGGL(residual_rmsnorm_kernel<true>, dim3(p.T), dim3(residual_threads(p.H)), 0, s, a);
  return hipGetLastError();
}

}  // namespace smoe
