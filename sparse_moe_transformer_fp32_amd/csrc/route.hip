// Router of the MoE layer on gfx950: logits, sigmoid + bias, top-K, weights,
// and the expert-contiguous dispatch.
//
// Sources: LLM Atlas model card "Step-3.5-Flash", raw config field table
// (need_fp32_gate, moe_router_activation sigmoid, use_moe_router_bias,
// moe_top_k, norm_expert_weight, moe_router_scaling_factor); shd-paper.top
// summary, 方法详解 / 关键设计 (the gate maps the token representation to one
// weight per expert and the highest-weighted experts are used).
#include "smoe_internal.h"

#include <math.h>

namespace smoe {

// --------------------------------------------------------------------------
// Router logits  l[t,e] = sum_h x[t,h] * W[e,h]  with fp32 semantics.
//
// x is bf16, so it is exact as bf16.  Each fp32 weight w is split on the fly
// into three bf16 parts w = hi + mid + lo (hi = bf16(w), mid = bf16(w - hi),
// lo = bf16(w - hi - mid); each difference is exact in fp32 and the residual
// is below 2^-24 |w|).  Every bf16 x bf16 product is exact in fp32, and the
// MFMA accumulates in fp32, so the result has the accuracy of an fp32 GEMM
// while running on the bf16 matrix cores.
//
// Tile: a workgroup of 4 waves covers 64 experts x (16*NB) tokens; each wave
// owns 16 experts (the MFMA A operand) and all tokens of the tile (B).  H is
// split over gridDim.z so that small-T launches still spread the 4.7 MB of
// router weights over many CUs; each split writes its own partial sums and
// the top-K kernel adds them in a fixed order.
template <int NB>
__global__ __launch_bounds__(256) void route_logits_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ W, float* __restrict__ partial,
    int T, int H, int E, int klen) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int e0 = blockIdx.y * 64 + wave * 16;
  if (e0 >= E) return;
  const int t0 = blockIdx.x * (16 * NB);
  const int split = blockIdx.z;
  const int r = lane & 15, g = lane >> 4;
  const int kbeg = split * klen + 8 * g;

  const float* wrow = W + (size_t)min(e0 + r, E - 1) * H + kbeg;
  const uint16_t* xrow[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    xrow[nb] = x + (size_t)min(t0 + nb * 16 + r, T - 1) * H + kbeg;

  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll 2
  for (int k = 0; k < klen; k += 32) {
    const f32x4 w0 = *reinterpret_cast<const f32x4*>(wrow + k);
    const f32x4 w1 = *reinterpret_cast<const f32x4*>(wrow + k + 4);
    bf16x8 hi, mid, lo;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float w = j < 4 ? w0[j] : w1[j - 4];
      const __bf16 h = (__bf16)w;
      const float r1 = w - (float)h;
      const __bf16 m = (__bf16)r1;
      const float r2 = r1 - (float)m;
      hi[j] = h;
      mid[j] = m;
      lo[j] = (__bf16)r2;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const u32x4 xv = *reinterpret_cast<const u32x4*>(xrow[nb] + k);
      const bf16x8 b = __builtin_bit_cast(bf16x8, xv);
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, b, acc[nb], 0, 0, 0);
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mid, b, acc[nb], 0, 0, 0);
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, b, acc[nb], 0, 0, 0);
    }
  }
  // C layout of the 16x16 MFMA: lane holds rows 4g..4g+3 (experts) of
  // column r (token).
  float* out = partial + (size_t)split * T * E;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int t = t0 + nb * 16 + r;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + 4 * g + j;
      if (e < E) out[(size_t)t * E + e] = acc[nb][j];
    }
  }
}

// --------------------------------------------------------------------------
// Sigmoid, bias, top-K and weights: one wave per token.  Lane l holds the
// experts l, l+64, l+128, ...  K rounds of a wave-wide argmax (larger key
// first, equal keys -> lower expert id) pick the set; ballots then list the
// chosen experts in ascending id.
__global__ __launch_bounds__(256) void route_topk_kernel(
    const float* __restrict__ partial, int S, const float* __restrict__ bias, int T, int E,
    int K, float scale, int norm, int biw, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, float* __restrict__ keys_out, float* __restrict__ scores_out) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int C = (E + 63) >> 6;

  // logits: sum the split-H partial sums in a fixed order; all loads of a
  // group of four splits are issued before any add
  float lg[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) lg[c] = 0.f;
  for (int s0 = 0; s0 < S; s0 += 4) {
    float v[16][4];
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const int e = min(c * 64 + lane, E - 1);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        v[c][q] = (c < C && s0 + q < S) ? partial[((size_t)(s0 + q) * T + t) * E + e] : 0.f;
    }
#pragma unroll
    for (int c = 0; c < 16; ++c)
#pragma unroll
      for (int q = 0; q < 4; ++q) lg[c] += v[c][q];
  }

  float key[16], sc[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    key[c] = -INFINITY;
    sc[c] = 0.f;
    const int e = c * 64 + lane;
    if (c < C && e < E) {
      const float l = lg[c];
      const float sg = 1.0f / (1.0f + expf(-l));
      const float kk = sg + bias[e];
      sc[c] = sg;
      key[c] = kk == kk ? kk : -INFINITY;  // a NaN key never wins (inputs must be finite)
      if (keys_out) keys_out[(size_t)t * E + e] = kk;
      if (scores_out) scores_out[(size_t)t * E + e] = sg;
    }
  }

  uint32_t sel = 0;
  for (int k = 0; k < K; ++k) {
    float bk = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const int e = c * 64 + lane;
      const bool cand = c < C && e < E && !((sel >> c) & 1u);
      if (cand && (key[c] > bk || (key[c] == bk && e < be))) {
        bk = key[c];
        be = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ok = __shfl_xor(bk, off);
      const int oe = __shfl_xor(be, off);
      if (ok > bk || (ok == bk && oe < be)) {
        bk = ok;
        be = oe;
      }
    }
    if ((be & 63) == lane) sel |= 1u << (be >> 6);
  }

  // weight numerator g = s (bias steers selection only) or s + b
  float gsum = 0.f;
#pragma unroll
  for (int c = 0; c < 16; ++c)
    if ((sel >> c) & 1u) gsum += biw ? key[c] : sc[c];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) gsum += __shfl_xor(gsum, off);

  const unsigned long long below = (1ull << lane) - 1ull;
  int base = 0;
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    if (c >= C) break;
    const bool mine = (sel >> c) & 1u;
    const unsigned long long m = __ballot(mine);
    if (mine) {
      const int j = base + __popcll(m & below);
      const float gv = biw ? key[c] : sc[c];
      float w;
      if (norm)
        w = gsum > 0.f ? scale * gv / gsum : scale / (float)K;
      else
        w = scale * gv;
      topk_idx[(size_t)t * K + j] = c * 64 + lane;
      topk_w[(size_t)t * K + j] = w;
    }
    base += __popcll(m);
  }
}

// --------------------------------------------------------------------------
// Dispatch (one workgroup of 1024 threads):
//   counts   LDS histogram of the selected expert ids
//   offsets  exclusive scan of counts
//   rows     stable scatter: inside an expert's block, rows follow ascending
//            token order.  Tokens are taken 256 at a time; a 256-bit LDS mask
//            per expert marks which tokens of the chunk chose it, and a
//            token's rank is the popcount of the mask bits below it.
//   row blocks  work list for the grouped GEMMs: each expert's rows cut into
//            blocks of at most `bn`, then the shared expert's T rows.
__device__ inline int block_exclusive_scan(int v, int* s_wave, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off);
    if (lane >= off) inc += o;
  }
  if (lane == 63) s_wave[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const int nw = blockDim.x >> 6;
    int wv = lane < nw ? s_wave[lane] : 0;
    int winc = wv;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(winc, off);
      if (lane >= off) winc += o;
    }
    if (lane < nw) s_wave[lane] = winc - wv;  // exclusive wave prefix
    if (lane == nw - 1) s_wave[32] = winc;
  }
  __syncthreads();
  const int ex = s_wave[wave] + inc - v;
  *total = s_wave[32];
  __syncthreads();
  return ex;
}

__global__ __launch_bounds__(1024) void dispatch_kernel(
    const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_w, int T, int K,
    int E, int bn, int has_shared, int rb_max, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ slot_pos,
    int32_t* __restrict__ row_token, float* __restrict__ row_w, RowBlock* __restrict__ rb,
    int32_t* __restrict__ n_rb) {
  __shared__ int s_cnt[1024];
  __shared__ int s_fill[1024];
  __shared__ uint32_t s_mask[1024 * 8];
  __shared__ int s_wave[33];
  const int tid = threadIdx.x;
  const int KT = T * K;

  for (int e = tid; e < E; e += 1024) s_cnt[e] = 0;
  __syncthreads();
  // expert ids come from route_topk and are in range; the clamp only keeps
  // LDS indexing in bounds whatever the input
  for (int i = tid; i < KT; i += 1024) atomicAdd(&s_cnt[min(max(topk_idx[i], 0), E - 1)], 1);
  __syncthreads();

  // E <= 1024: one expert per thread
  const int cnt = tid < E ? s_cnt[tid] : 0;
  int total;
  const int off = block_exclusive_scan(cnt, s_wave, &total);
  const int nrb = (cnt + bn - 1) / bn;
  int rb_total;
  const int rbpos = block_exclusive_scan(nrb, s_wave, &rb_total);
  if (tid < E) {
    counts[tid] = cnt;
    offsets[tid] = off;
    s_fill[tid] = off;
    for (int i = 0; i < nrb; ++i) {
      const int p = rbpos + i;
      if (p < rb_max) rb[p] = RowBlock{tid, off + i * bn, min(bn, cnt - i * bn), 0};
    }
  }
  if (tid == 0) offsets[E] = total;
  const int nrb_s = has_shared ? (T + bn - 1) / bn : 0;
  for (int i = tid; i < nrb_s; i += 1024) {
    const int p = rb_total + i;
    if (p < rb_max) rb[p] = RowBlock{E, KT + i * bn, min(bn, T - i * bn), 0};
  }
  if (tid == 0) n_rb[0] = min(rb_total + nrb_s, rb_max);
  __syncthreads();

  for (int c0 = 0; c0 < T; c0 += 256) {
    for (int i = tid; i < E * 8; i += 1024) s_mask[i] = 0u;
    __syncthreads();
    for (int i = tid; i < 256 * K; i += 1024) {
      const int t = c0 + i / K;
      if (t < T) {
        const int e = min(max(topk_idx[(size_t)t * K + (i % K)], 0), E - 1);
        const int lt = t - c0;
        atomicOr(&s_mask[e * 8 + (lt >> 5)], 1u << (lt & 31));
      }
    }
    __syncthreads();
    for (int i = tid; i < 256 * K; i += 1024) {
      const int t = c0 + i / K;
      if (t < T) {
        const int j = i % K;
        const int e = min(max(topk_idx[(size_t)t * K + j], 0), E - 1);
        const int lt = t - c0;
        int rank = 0;
        for (int wd = 0; wd < (lt >> 5); ++wd) rank += __popc(s_mask[e * 8 + wd]);
        rank += __popc(s_mask[e * 8 + (lt >> 5)] & ((1u << (lt & 31)) - 1u));
        const int row = s_fill[e] + rank;
        perm[row] = t;
        row_token[row] = t;
        row_w[row] = topk_w[(size_t)t * K + j];
        slot_pos[(size_t)t * K + j] = row;
      }
    }
    __syncthreads();
    for (int e = tid; e < E; e += 1024) {
      int n = 0;
#pragma unroll
      for (int wd = 0; wd < 8; ++wd) n += __popc(s_mask[e * 8 + wd]);
      s_fill[e] += n;
    }
    __syncthreads();
  }
  if (has_shared) {
    for (int t = tid; t < T; t += 1024) {
      row_token[KT + t] = t;
      row_w[KT + t] = 1.0f;
    }
  }
}

// --------------------------------------------------------------------------
hipError_t launch_route_logits(const Plan& p, const uint16_t* x, const float* W,
                               float* partial, hipStream_t s) {
  const int klen = p.H / p.route_splits;
  dim3 grid((p.T + p.route_tok - 1) / p.route_tok, (p.E + 63) / 64, p.route_splits);
  if (p.route_tok == 16)
    hipLaunchKernelGGL(route_logits_kernel<1>, grid, dim3(256), 0, s, x, W, partial, p.T, p.H,
                       p.E, klen);
  else
    hipLaunchKernelGGL(route_logits_kernel<4>, grid, dim3(256), 0, s, x, W, partial, p.T, p.H,
                       p.E, klen);
  return hipGetLastError();
}

hipError_t launch_route_topk(const Plan& p, const float* partial, const float* bias,
                             float scale, int norm, int biw, int32_t* topk_idx, float* topk_w,
                             float* keys, float* scores, hipStream_t s) {
  dim3 grid((p.T + 3) / 4);
  hipLaunchKernelGGL(route_topk_kernel, grid, dim3(256), 0, s, partial, p.route_splits, bias,
                     p.T, p.E, p.K, scale, norm, biw, topk_idx, topk_w, keys, scores);
  return hipGetLastError();
}

hipError_t launch_dispatch(const Plan& p, const int32_t* topk_idx, const float* topk_w,
                           int32_t* counts, int32_t* offsets, int32_t* perm_token,
                           int32_t* slot_pos, int32_t* row_token, float* row_w, RowBlock* rb,
                           int32_t* n_rb, hipStream_t s) {
  hipLaunchKernelGGL(dispatch_kernel, dim3(1), dim3(1024), 0, s, topk_idx, topk_w, p.T, p.K,
                     p.E, p.bn, p.Is > 0 ? 1 : 0, p.rb_max, counts, offsets, perm_token,
                     slot_pos, row_token, row_w, rb, n_rb);
  return hipGetLastError();
}

}  // namespace smoe
