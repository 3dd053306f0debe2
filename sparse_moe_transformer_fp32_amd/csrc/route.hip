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

#include <type_traits>

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
// router weights over many CUs; each split writes its own partial sum and
// the top-K kernel adds them in a fixed order.
template <int NB, int U>
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

  // two register stages of U k-steps; every load is unconditional (steps
  // past the end re-read the last chunk and skip their MFMAs)
  const int nsteps = klen / 32;
  const int nstages = (nsteps + U - 1) / U;
  f32x4 wa[U][2], wb[U][2];
  u32x4 xa[U][NB], xb[U][NB];
  auto load = [&](f32x4 (&w)[U][2], u32x4 (&xv)[U][NB], int stage) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = min(stage * U + u, nsteps - 1) * 32;
      w[u][0] = *reinterpret_cast<const f32x4*>(wrow + k);
      w[u][1] = *reinterpret_cast<const f32x4*>(wrow + k + 4);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) xv[u][nb] = *reinterpret_cast<const u32x4*>(xrow[nb] + k);
    }
  };
  auto compute = [&](const f32x4 (&w)[U][2], const u32x4 (&xv)[U][NB], int stage) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (stage * U + u < nsteps) {
        bf16x8 hi, mid, lo;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float wv = j < 4 ? w[u][0][j] : w[u][1][j - 4];
          const __bf16 h = (__bf16)wv;
          const float r1 = wv - (float)h;
          const __bf16 m = (__bf16)r1;
          const float r2 = r1 - (float)m;
          hi[j] = h;
          mid[j] = m;
          lo[j] = (__bf16)r2;
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const bf16x8 b = __builtin_bit_cast(bf16x8, xv[u][nb]);
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, b, acc[nb], 0, 0, 0);
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mid, b, acc[nb], 0, 0, 0);
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, b, acc[nb], 0, 0, 0);
        }
      }
    }
  };
  load(wa, xa, 0);
  int st = 0;
  for (; st + 2 < nstages; st += 2) {
    load(wb, xb, st + 1);
    compute(wa, xa, st);
    load(wa, xa, st + 2);
    compute(wb, xb, st + 1);
  }
  if (st + 1 < nstages) {
    load(wb, xb, st + 1);
    compute(wa, xa, st);
    compute(wb, xb, st + 1);
  } else {
    compute(wa, xa, st);
  }

  // C layout of the 16x16 MFMA: lane holds rows 4g..4g+3 (experts) of
  // column r (token).  Partial sums are stored [T][E][S] so that the S
  // splits of one logit are contiguous for the top-K kernel.
  const int S = gridDim.z;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int t = t0 + nb * 16 + r;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + 4 * g + j;
      if (e < E) partial[((size_t)t * E + e) * S + split] = acc[nb][j];
    }
  }
}

// --------------------------------------------------------------------------
// Router logits for many tokens, with the same fp32 semantics.
//
// Workgroup tile: 48 experts x 256 tokens over one split of H.  Wave w owns
// tokens 64w..64w+63 as four 16-token B fragments, loaded from x straight
// into registers (no other wave reads them), and all 48 experts as three
// 16-row A fragments per bf16 part, read from LDS.  Per 64-wide k stage the
// workgroup loads the fp32 weights of its experts once, splits each into its
// three bf16 parts (as above) and stores them to LDS in A-fragment order, so
// a weight is split once per 256 tokens.  Per 32-wide k step the parts are
// applied lo, mid, hi, as in the kernel above.
constexpr int kRouteE = 48;    // experts per workgroup (three 16-row fragments)
constexpr int kRouteT = 256;   // tokens per workgroup (64 per wave)

__global__ __launch_bounds__(256, 2) void route_logits_wide_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ W, float* __restrict__ partial,
    int T, int H, int E, int klen) {
  // A fragments of one stage: [slot][32-k chunk][part lo/mid/hi][fragment][lane] x 16 bytes
  __shared__ __attribute__((aligned(16))) unsigned char s_a[2][2][3][3][1024];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e0 = blockIdx.y * kRouteE;
  const int t0 = blockIdx.x * kRouteT + wave * 64;
  const int split = blockIdx.z;
  const int kb = split * klen;
  const int nst = klen / 64;

  // weights: load m of a thread brings row 16 m + tid / 16 of the tile, k =
  // 4 (tid % 16) .. +3 of the stage (16 threads read a row's 256 bytes).
  // In A-fragment order those 4 values are half (q % 2) of lane
  // 16 ((q % 8) / 2) + tid / 16 of chunk q / 8, q = tid % 16.
  const float* wsrc[3];
#pragma unroll
  for (int m = 0; m < 3; ++m)
    wsrc[m] = W + (size_t)min(e0 + 16 * m + (tid >> 4), E - 1) * H + kb + 4 * (tid & 15);
  const int q = tid & 15;
  const int a_off = (q >> 3) * (3 * 3 * 1024) + (16 * ((q & 7) >> 1) + (tid >> 4)) * 16 + 8 * (q & 1);
  // tokens: B fragment n of chunk c is token t0 + 16 n + lane % 16, k = 32 c
  // + 8 (lane / 16) .. +7 of the stage
  const uint16_t* xsrc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n)
    xsrc[n] = x + (size_t)min(t0 + 16 * n + (lane & 15), T - 1) * H + kb + 8 * (lane >> 4);

  f32x4 acc[3][4];
#pragma unroll
  for (int m = 0; m < 3; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  // past the end of K every load re-reads the last stage (in bounds; unused)
  auto load_w = [&](f32x4 (&w)[3], int st) {
    const int off = min(st, nst - 1) * 64;
#pragma unroll
    for (int m = 0; m < 3; ++m) w[m] = *reinterpret_cast<const f32x4*>(wsrc[m] + off);
  };
  auto load_x = [&](u32x4 (&v)[2][4], int st) {
    const int off = min(st, nst - 1) * 64;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int n = 0; n < 4; ++n) v[c][n] = *reinterpret_cast<const u32x4*>(xsrc[n] + off + 32 * c);
  };
  // split the loaded weights and store the parts to LDS slot `slot`
  auto store_w = [&](const f32x4 (&w)[3], int slot) {
#pragma unroll
    for (int m = 0; m < 3; ++m) {
      uint32_t hi2[2], mid2[2], lo2[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        uint16_t hb[2], mb[2], lb[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float wv = w[m][2 * i + j];
          const __bf16 h = (__bf16)wv;
          const float r1 = wv - (float)h;
          const __bf16 md = (__bf16)r1;
          const float r2 = r1 - (float)md;
          hb[j] = __builtin_bit_cast(uint16_t, h);
          mb[j] = __builtin_bit_cast(uint16_t, md);
          lb[j] = __builtin_bit_cast(uint16_t, (__bf16)r2);
        }
        hi2[i] = (uint32_t)hb[0] | ((uint32_t)hb[1] << 16);
        mid2[i] = (uint32_t)mb[0] | ((uint32_t)mb[1] << 16);
        lo2[i] = (uint32_t)lb[0] | ((uint32_t)lb[1] << 16);
      }
      unsigned char* base = &s_a[slot][0][0][m][0] + a_off;
      *reinterpret_cast<u32x2*>(base + 0 * 3 * 1024) = u32x2{lo2[0], lo2[1]};
      *reinterpret_cast<u32x2*>(base + 1 * 3 * 1024) = u32x2{mid2[0], mid2[1]};
      *reinterpret_cast<u32x2*>(base + 2 * 3 * 1024) = u32x2{hi2[0], hi2[1]};
    }
  };
  auto compute = [&](int slot, const u32x4 (&v)[2][4]) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      u32x4 a[3][3];
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int m = 0; m < 3; ++m)
          a[p][m] = *reinterpret_cast<const u32x4*>(&s_a[slot][c][p][m][lane * 16]);
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int m = 0; m < 3; ++m)
#pragma unroll
          for (int n = 0; n < 4; ++n)
            acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, a[p][m]), __builtin_bit_cast(bf16x8, v[c][n]),
                acc[m][n], 0, 0, 0);
    }
  };

  // stage s: weights of s+2 into register buffer s%2 (its stage-s weights
  // went to LDS at the end of stage s-1), tokens of s+2 into buffer (s+2)%3;
  // at the end of the stage the weights of s+1 (loaded one stage earlier)
  // are split into LDS slot (s+1)%2, last read in stage s-1, before its
  // closing barrier
  f32x4 wreg[2][3];
  u32x4 xb[3][2][4];
  load_w(wreg[0], 0);
  load_w(wreg[1], 1);
  load_x(xb[0], 0);
  load_x(xb[1], 1);
  store_w(wreg[0], 0);
  __syncthreads();
  auto stage = [&](auto jc, int st) {
    constexpr int J = decltype(jc)::value;   // st % 6
    load_w(wreg[J % 2], st + 2);
    load_x(xb[(J + 2) % 3], st + 2);
    compute(J % 2, xb[J % 3]);
    store_w(wreg[(J + 1) % 2], (J + 1) % 2);
    __syncthreads();
  };
  int st = 0;
  for (; st + 6 <= nst; st += 6) {
    stage(std::integral_constant<int, 0>{}, st);
    stage(std::integral_constant<int, 1>{}, st + 1);
    stage(std::integral_constant<int, 2>{}, st + 2);
    stage(std::integral_constant<int, 3>{}, st + 3);
    stage(std::integral_constant<int, 4>{}, st + 4);
    stage(std::integral_constant<int, 5>{}, st + 5);
  }
  if (st < nst) stage(std::integral_constant<int, 0>{}, st);
  if (st + 1 < nst) stage(std::integral_constant<int, 1>{}, st + 1);
  if (st + 2 < nst) stage(std::integral_constant<int, 2>{}, st + 2);
  if (st + 3 < nst) stage(std::integral_constant<int, 3>{}, st + 3);
  if (st + 4 < nst) stage(std::integral_constant<int, 4>{}, st + 4);

  // accumulator register j of fragment (m, n): expert 16 m + 4 (lane / 16) + j,
  // token 16 n + lane % 16.  Partial sums are stored [T][S][E], so a lane's
  // four registers of a fragment are four consecutive floats of one row:
  // one 16-byte store (the row starts 16-byte aligned when E % 4 == 0, and e
  // is a multiple of 4).  ([T][E][S] took one 4-byte store per register,
  // 64 scattered writes per instruction.)
  const int S = gridDim.z;
  const bool vec = (E & 3) == 0;
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int t = t0 + 16 * n + (lane & 15);
    if (t >= T) continue;
    float* row = partial + ((size_t)t * S + split) * E;
#pragma unroll
    for (int m = 0; m < 3; ++m) {
      const int e = e0 + 16 * m + 4 * (lane >> 4);
      if (vec && e < E) {
        *reinterpret_cast<f32x4*>(row + e) = acc[m][n];
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (e + j < E) row[e + j] = acc[m][n][j];
      }
    }
  }
}

// --------------------------------------------------------------------------
// Top-K and weights for one token, by one wave.  Lane l holds experts
// l, l+64, l+128, ... (key[c], sc[c] for expert 64c + l).
//
// Selection is a radix select, with no cross-lane data movement: keys are
// mapped to order-preserving unsigned integers, and the K-th largest is found
// bit by bit from the top (a candidate threshold is kept if at least K keys
// are >= it; counts come from ballots and scalar popcounts).  The chosen set
// is every key above that threshold plus, among keys equal to it, the lowest
// expert ids.  Slots are then listed in ascending expert id, and the weight
// denominator is summed in that slot order with readlane.
__device__ inline uint32_t ordered_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int C>
__device__ inline void wave_select(const float (&key)[C], const float (&sc)[C], int E, int K,
                                   float scale, int norm, int biw, int32_t* idx_out,
                                   float* w_out) {
  const int lane = threadIdx.x & 63;
  const unsigned long long below = (1ull << lane) - 1ull;
  uint32_t ok[C];
  uint32_t valid = 0;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    ok[c] = ordered_key(key[c]);
    if (c * 64 + lane < E) valid |= 1u << c;
  }
  // K-th largest ordered key (K <= E, so it exists)
  uint32_t thr = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = thr | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int c = 0; c < C; ++c) cnt += __popcll(__ballot(((valid >> c) & 1u) && ok[c] >= cand));
    if (cnt >= K) thr = cand;
  }
  int n_gt = 0;
#pragma unroll
  for (int c = 0; c < C; ++c) n_gt += __popcll(__ballot(((valid >> c) & 1u) && ok[c] > thr));
  const int need = K - n_gt;  // >= 1 keys equal to thr, lowest ids first
  uint32_t sel = 0;
  int eq_before = 0;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const bool v = (valid >> c) & 1u;
    const bool eq = v && ok[c] == thr;
    const unsigned long long meq = __ballot(eq);
    const int rank = eq_before + __popcll(meq & below);
    if ((v && ok[c] > thr) || (eq && rank < need)) sel |= 1u << c;
    eq_before += __popcll(meq);
  }

  // denominator in slot order (ascending expert id)
  float gsum = 0.f;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    unsigned long long m = __ballot((sel >> c) & 1u);
    const int gbits = __float_as_int(biw ? key[c] : sc[c]);
    while (m) {
      const int ln = __builtin_ctzll(m);
      m &= m - 1ull;
      gsum += __int_as_float(__builtin_amdgcn_readlane(gbits, ln));
    }
  }

  int base = 0;
#pragma unroll
  for (int c = 0; c < C; ++c) {
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
      idx_out[j] = c * 64 + lane;
      w_out[j] = w;
    }
    base += __popcll(m);
  }
}

// score and key of one expert from its logit; a NaN key never wins (inputs
// must be finite)
__device__ inline void score_key(float l, float b, float* sg, float* kk) {
  *sg = 1.0f / (1.0f + expf(-l));
  const float k = *sg + b;
  *kk = k == k ? k : -INFINITY;
}

// One wave per token (one-wave workgroups, four waves per workgroup from
// 1024 tokens on): add the S split-H partial logits of each expert
// (contiguous, loaded as 16-byte vectors, all loads issued before the adds;
// fixed order), then sigmoid, bias and wave_select.  C = ceil(E/64) expert
// slots per lane, fixed at compile time.  QN = 16-byte vectors per expert: 8
// holds up to 32 splits, the splits of up to five expert slots in flight at
// a time (a 160-VGPR buffer: one round of loads for E <= 320); 1 holds up to
// 4 splits, every expert's in flight at once, in few enough registers for a
// higher occupancy.  Both read the [T][E][S] partial sums of route_logits_kernel.
// QN = 0 reads the [T][S][E] partial sums of route_logits_wide_kernel, SW
// = S splits (1, 2, 4 or 8, fixed at compile time): one float per split and
// expert, each load coalesced over the wave's 64 experts, all in flight at
// once.
template <int C, int QN, int SW>
__global__ __launch_bounds__(256) void route_topk_kernel(
    const float* __restrict__ partial, int S, const float* __restrict__ bias, int T, int E,
    int K, float scale, int norm, int biw, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, float* __restrict__ keys_out, float* __restrict__ scores_out) {
  constexpr int CB = QN == 1 ? C : (C <= 5 ? C : 4);   // expert slots per load batch
  const int lane = threadIdx.x & 63;
  // one token per wave; a workgroup of several waves takes consecutive tokens
  const int t = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (t >= T) return;   // uniform over the wave (no barriers below)

  float key[C], sc[C];
  // expert slot c from its summed logit l: score, key, optional exports
  auto finish = [&](int c, float l) {
    key[c] = -INFINITY;
    sc[c] = 0.f;
    const int e = c * 64 + lane;
    if (e < E) {
      score_key(l, bias[e], &sc[c], &key[c]);
      if (keys_out) keys_out[(size_t)t * E + e] = sc[c] + bias[e];
      if (scores_out) scores_out[(size_t)t * E + e] = sc[c];
    }
  };
  if constexpr (QN == 0) {
    const float* srow = partial + (size_t)t * SW * E;
    float v[C][SW];
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int e = min(c * 64 + lane, E - 1);
#pragma unroll
      for (int s = 0; s < SW; ++s) v[c][s] = srow[(size_t)s * E + e];
    }
#pragma unroll
    for (int c = 0; c < C; ++c) {
      float l = 0.f;
#pragma unroll
      for (int s = 0; s < SW; ++s) l += v[c][s];
      finish(c, l);
    }
  } else {
    const float* prow = partial + (size_t)t * E * S;
#pragma unroll
    for (int c0 = 0; c0 < C; c0 += CB) {
      f32x4 v[CB][QN];
#pragma unroll
      for (int cc = 0; cc < CB; ++cc) {
        const int e = min((c0 + cc) * 64 + lane, E - 1);
#pragma unroll
        for (int q = 0; q < QN; ++q) {
          if (c0 + cc < C && S >= 4 && q < S / 4)
            v[cc][q] = *reinterpret_cast<const f32x4*>(prow + (size_t)e * S + 4 * q);
          else if (c0 + cc < C && S < 4 && q == 0)
            v[cc][q] = f32x4{prow[(size_t)e * S], S > 1 ? prow[(size_t)e * S + 1] : 0.f, 0.f, 0.f};
          else
            v[cc][q] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
#pragma unroll
      for (int cc = 0; cc < CB; ++cc) {
        if (c0 + cc < C) {
          float l = 0.f;
#pragma unroll
          for (int q = 0; q < QN; ++q)
#pragma unroll
            for (int j = 0; j < 4; ++j) l += v[cc][q][j];
          finish(c0 + cc, l);
        }
      }
    }
  }
  wave_select<C>(key, sc, E, K, scale, norm, biw, topk_idx + (size_t)t * K,
                 topk_w + (size_t)t * K);
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
//            ceil(count / bn) blocks of nearly equal height (whole granules
//            of rows), then the shared expert's T rows cut the same way.
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

// counts, offsets (exclusive scan) and the GEMM row-block list from one
// expert count per thread of a 1024-thread workgroup; returns this thread's
// offset.  Every thread must call it.
__device__ inline int finish_counts(int cnt, int E, int T, int K, int bn, int gran,
                                    int has_shared, int rb_max, int* s_wave, int32_t* counts,
                                    int32_t* offsets, RowBlock* rb, int32_t* n_rb) {
  const int tid = threadIdx.x;
  const int KT = T * K;
  int total;
  const int off = block_exclusive_scan(cnt, s_wave, &total);
  const int nrb = (cnt + bn - 1) / bn;
  int rb_total;
  const int rbpos = block_exclusive_scan(nrb, s_wave, &rb_total);
  if (tid < E) {
    counts[tid] = cnt;
    offsets[tid] = off;
    for (int i = 0; i < nrb; ++i) {
      const int p = rbpos + i;
      int st, n;
      split_block(cnt, nrb, gran, i, &st, &n);
      if (p < rb_max) rb[p] = RowBlock{tid, off + st, n, rbpos, nrb, off, cnt, 0};
    }
  }
  if (tid == 0) offsets[E] = total;
  const int nrb_s = has_shared ? (T + bn - 1) / bn : 0;
  for (int i = tid; i < nrb_s; i += blockDim.x) {
    const int p = rb_total + i;
    int st, n;
    split_block(T, nrb_s, gran, i, &st, &n);
    if (p < rb_max) rb[p] = RowBlock{E, KT + st, n, rb_total, nrb_s, KT, T, 0};
  }
  if (tid == 0) n_rb[0] = min(rb_total + nrb_s, rb_max);
  if (tid == 1 || tid == 2) n_rb[tid] = 0;   // the GEMMs' pool claim counters
  return off;
}

struct DispatchArgs {
  const int32_t* topk_idx;
  const float* topk_w;
  int T, K, E, bn, gran, has_shared, rb_max;
  int32_t *counts, *offsets, *perm, *slot_pos, *row_token;
  float* row_w;
  RowBlock* rb;
  int32_t* n_rb;
};

// Dynamic LDS: cnt[E], fill[E], mask[8E], wave scratch[36].
__global__ __launch_bounds__(1024) void dispatch_kernel(DispatchArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int E = a.E, T = a.T, K = a.K;
  int* s_cnt = reinterpret_cast<int*>(smem);
  int* s_fill = s_cnt + E;
  uint32_t* s_mask = reinterpret_cast<uint32_t*>(s_fill + E);
  int* s_wave = reinterpret_cast<int*>(s_mask + 8 * E);
  const int tid = threadIdx.x;
  const int KT = T * K;

  // expert ids come from the top-K and are in range; the clamp only keeps
  // LDS indexing in bounds whatever the input
  auto sel_e = [&](int i) { return min(max(a.topk_idx[i], 0), E - 1); };
  auto sel_w = [&](int i) { return a.topk_w[i]; };

  for (int e = tid; e < E; e += 1024) s_cnt[e] = 0;
  __syncthreads();
  for (int i = tid; i < KT; i += 1024) atomicAdd(&s_cnt[sel_e(i)], 1);
  __syncthreads();

  // E <= 1024: one expert per thread
  const int cnt = tid < E ? s_cnt[tid] : 0;
  const int off = finish_counts(cnt, E, T, K, a.bn, a.gran, a.has_shared, a.rb_max, s_wave,
                                a.counts, a.offsets, a.rb, a.n_rb);
  if (tid < E) s_fill[tid] = off;
  __syncthreads();

  for (int c0 = 0; c0 < T; c0 += 256) {
    for (int i = tid; i < E * 8; i += 1024) s_mask[i] = 0u;
    __syncthreads();
    for (int i = tid; i < 256 * K; i += 1024) {
      const int t = c0 + i / K;
      if (t < T) {
        const int e = sel_e(t * K + (i % K));
        const int lt = t - c0;
        atomicOr(&s_mask[e * 8 + (lt >> 5)], 1u << (lt & 31));
      }
    }
    __syncthreads();
    for (int i = tid; i < 256 * K; i += 1024) {
      const int t = c0 + i / K;
      if (t < T) {
        const int j = i % K;
        const int e = sel_e(t * K + j);
        const int lt = t - c0;
        int rank = 0;
        for (int wd = 0; wd < (lt >> 5); ++wd) rank += __popc(s_mask[e * 8 + wd]);
        rank += __popc(s_mask[e * 8 + (lt >> 5)] & ((1u << (lt & 31)) - 1u));
        const int row = s_fill[e] + rank;
        a.perm[row] = t;
        a.row_token[row] = t;
        a.row_w[row] = sel_w(t * K + j);
        a.slot_pos[(size_t)t * K + j] = row;
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
  if (a.has_shared) {
    for (int t = tid; t < T; t += 1024) {
      a.row_token[KT + t] = t;
      a.row_w[KT + t] = 1.0f;
    }
  }
}

size_t dispatch_lds_bytes(int E) { return (size_t)E * 4 * 2 + (size_t)E * 8 * 4 + 36 * 4; }

// --------------------------------------------------------------------------
// Dispatch for large T in three steps, so that many CUs share the work.
// Block b holds tokens [256b, 256b + 256).
//  1. local: per block, the 256-bit LDS mask of each expert gives every
//     selection its rank among the block's earlier tokens for that expert,
//     and the block's per-expert histogram.
//  2. scan (one workgroup): per expert, the number of rows of all earlier
//     blocks; then counts, offsets and the row-block list.
//  3. scatter: row = offsets[e] + earlier blocks' rows + local rank.
__global__ __launch_bounds__(256) void dispatch_local_kernel(const int32_t* __restrict__ topk_idx,
                                                             int T, int K, int E,
                                                             int32_t* __restrict__ lrank,
                                                             int32_t* __restrict__ hist) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint32_t* s_mask = reinterpret_cast<uint32_t*>(smem);  // 8E words
  const int tid = threadIdx.x, blk = blockIdx.x;
  const int t0 = blk * 256;
  for (int i = tid; i < E * 8; i += 256) s_mask[i] = 0u;
  __syncthreads();
  for (int i = tid; i < 256 * K; i += 256) {
    const int t = t0 + i / K;
    if (t < T) {
      const int e = min(max(topk_idx[(size_t)t * K + (i % K)], 0), E - 1);
      const int lt = t - t0;
      atomicOr(&s_mask[e * 8 + (lt >> 5)], 1u << (lt & 31));
    }
  }
  __syncthreads();
  for (int i = tid; i < 256 * K; i += 256) {
    const int t = t0 + i / K;
    if (t < T) {
      const int j = i % K;
      const int e = min(max(topk_idx[(size_t)t * K + j], 0), E - 1);
      const int lt = t - t0;
      int rank = 0;
      for (int wd = 0; wd < (lt >> 5); ++wd) rank += __popc(s_mask[e * 8 + wd]);
      rank += __popc(s_mask[e * 8 + (lt >> 5)] & ((1u << (lt & 31)) - 1u));
      lrank[(size_t)t * K + j] = rank;
    }
  }
  for (int e = tid; e < E; e += 256) {
    int n = 0;
#pragma unroll
    for (int wd = 0; wd < 8; ++wd) n += __popc(s_mask[e * 8 + wd]);
    hist[(size_t)blk * E + e] = n;
  }
}

__global__ __launch_bounds__(1024) void dispatch_scan_kernel(
    const int32_t* __restrict__ hist, int nblk, int T, int K, int E, int bn, int gran,
    int has_shared, int rb_max, int32_t* __restrict__ block_base, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, RowBlock* __restrict__ rb, int32_t* __restrict__ n_rb) {
  __shared__ int s_wave[36];
  const int tid = threadIdx.x;
  int cnt = 0;
  if (tid < E) {
    for (int b0 = 0; b0 < nblk; b0 += 16) {
      int v[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) v[q] = b0 + q < nblk ? hist[(size_t)(b0 + q) * E + tid] : 0;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        if (b0 + q < nblk) {
          block_base[(size_t)(b0 + q) * E + tid] = cnt;
          cnt += v[q];
        }
      }
    }
  }
  finish_counts(cnt, E, T, K, bn, gran, has_shared, rb_max, s_wave, counts, offsets, rb, n_rb);
}

__global__ __launch_bounds__(256) void dispatch_scatter_kernel(
    const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_w,
    const int32_t* __restrict__ lrank, const int32_t* __restrict__ block_base,
    const int32_t* __restrict__ offsets, int T, int K, int E, int has_shared,
    int32_t* __restrict__ perm, int32_t* __restrict__ slot_pos, int32_t* __restrict__ row_token,
    float* __restrict__ row_w) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int KT = T * K;
  if (i < KT) {
    const int t = i / K;
    const int e = min(max(topk_idx[i], 0), E - 1);
    const int row = offsets[e] + block_base[(size_t)(t >> 8) * E + e] + lrank[i];
    perm[row] = t;
    row_token[row] = t;
    row_w[row] = topk_w[i];
    slot_pos[i] = row;
  }
  if (has_shared && i < T) {
    row_token[KT + i] = i;
    row_w[KT + i] = 1.0f;
  }
}

// --------------------------------------------------------------------------
hipError_t launch_route_logits(const Plan& p, const uint16_t* x, const float* W,
                               float* partial, hipStream_t s) {
  const int klen = p.H / p.route_splits;
  if (p.route_tok == kRouteT) {
    if (klen % 64) return hipErrorInvalidValue;
    dim3 grid((p.T + kRouteT - 1) / kRouteT, (p.E + kRouteE - 1) / kRouteE, p.route_splits);
    hipLaunchKernelGGL(route_logits_wide_kernel, grid, dim3(256), 0, s, x, W, partial, p.T, p.H,
                       p.E, klen);
    return hipGetLastError();
  }
  dim3 grid((p.T + p.route_tok - 1) / p.route_tok, (p.E + 63) / 64, p.route_splits);
  if (p.route_tok == 16)
    hipLaunchKernelGGL((route_logits_kernel<1, 4>), grid, dim3(256), 0, s, x, W, partial, p.T,
                       p.H, p.E, klen);
  else
    hipLaunchKernelGGL((route_logits_kernel<4, 2>), grid, dim3(256), 0, s, x, W, partial, p.T,
                       p.H, p.E, klen);
  return hipGetLastError();
}

template <int C, int QN, int SW>
static void topk_launch(const Plan& p, const float* partial, const float* bias, float scale,
                        int norm, int biw, int32_t* topk_idx, float* topk_w, float* keys,
                        float* scores, hipStream_t s) {
  // one token per wave: one-wave workgroups for small batches, four-wave
  // workgroups (a quarter of the workgroups to launch) from 1024 tokens on
  const int wpg = p.T >= 1024 ? 4 : 1;
  hipLaunchKernelGGL((route_topk_kernel<C, QN, SW>), dim3((p.T + wpg - 1) / wpg), dim3(64 * wpg),
                     0, s, partial, p.route_splits, bias, p.T, p.E, p.K, scale, norm, biw,
                     topk_idx, topk_w, keys, scores);
}

// the instantiation that reads the router's layout: [T][S][E] after the wide
// router (S = 1, 2, 4 or 8), [T][E][S] otherwise
template <int C>
static hipError_t topk_for_layout(const Plan& p, const float* partial, const float* bias,
                                  float scale, int norm, int biw, int32_t* topk_idx,
                                  float* topk_w, float* keys, float* scores, hipStream_t s) {
  if (p.route_tok == kRouteT) {
    switch (p.route_splits) {
      case 1: topk_launch<C, 0, 1>(p, partial, bias, scale, norm, biw, topk_idx, topk_w, keys, scores, s); break;
      case 2: topk_launch<C, 0, 2>(p, partial, bias, scale, norm, biw, topk_idx, topk_w, keys, scores, s); break;
      case 4: topk_launch<C, 0, 4>(p, partial, bias, scale, norm, biw, topk_idx, topk_w, keys, scores, s); break;
      case 8: topk_launch<C, 0, 8>(p, partial, bias, scale, norm, biw, topk_idx, topk_w, keys, scores, s); break;
      default: return hipErrorInvalidValue;
    }
  } else if (p.route_splits <= 4) {
    topk_launch<C, 1, 0>(p, partial, bias, scale, norm, biw, topk_idx, topk_w, keys, scores, s);
  } else {
    topk_launch<C, 8, 0>(p, partial, bias, scale, norm, biw, topk_idx, topk_w, keys, scores, s);
  }
  return hipGetLastError();
}

hipError_t launch_route_topk(const Plan& p, const float* partial, const float* bias,
                             float scale, int norm, int biw, int32_t* topk_idx, float* topk_w,
                             float* keys, float* scores, hipStream_t s) {
  switch ((p.E + 63) / 64) {
#define SMOE_TOPK(CC) \
  case CC:            \
    return topk_for_layout<CC>(p, partial, bias, scale, norm, biw, topk_idx, topk_w, keys, scores, s);
    SMOE_TOPK(1) SMOE_TOPK(2) SMOE_TOPK(3) SMOE_TOPK(4) SMOE_TOPK(5) SMOE_TOPK(6)
    SMOE_TOPK(7) SMOE_TOPK(8) SMOE_TOPK(9) SMOE_TOPK(10) SMOE_TOPK(11) SMOE_TOPK(12)
    SMOE_TOPK(13) SMOE_TOPK(14) SMOE_TOPK(15) SMOE_TOPK(16)
#undef SMOE_TOPK
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_dispatch(const Plan& p, const RouteLaunch& r, hipStream_t s) {
  const int has_shared = p.Is > 0 ? 1 : 0;
  if (p.dispatch_blocks > 0) {
    const int nblk = p.dispatch_blocks;
    hipLaunchKernelGGL(dispatch_local_kernel, dim3(nblk), dim3(256), (size_t)p.E * 8 * 4, s,
                       r.topk_idx, p.T, p.K, p.E, r.lrank, r.hist);
    hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(1024), 0, s, r.hist, nblk, p.T, p.K,
                       p.E, p.bn, p.rb_gran, has_shared, p.rb_max, r.block_base, r.counts,
                       r.offsets, r.rb,
                       r.n_rb);
    hipLaunchKernelGGL(dispatch_scatter_kernel, dim3((p.KT + 255) / 256), dim3(256), 0, s,
                       r.topk_idx, r.topk_w, r.lrank, r.block_base, r.offsets, p.T, p.K, p.E,
                       has_shared, r.perm, r.slot, r.row_token, r.row_w);
    return hipGetLastError();
  }
  DispatchArgs a{};
  a.topk_idx = r.topk_idx;
  a.topk_w = r.topk_w;
  a.T = p.T; a.K = p.K; a.E = p.E; a.bn = p.bn; a.gran = p.rb_gran; a.has_shared = has_shared;
  a.rb_max = p.rb_max;
  a.counts = r.counts; a.offsets = r.offsets; a.perm = r.perm; a.slot_pos = r.slot;
  a.row_token = r.row_token; a.row_w = r.row_w; a.rb = r.rb; a.n_rb = r.n_rb;
  hipLaunchKernelGGL(dispatch_kernel, dim3(1), dim3(1024), dispatch_lds_bytes(p.E), s, a);
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// The routing of an empty batch: every count and offset is 0.
__global__ __launch_bounds__(256) void zero_counts_kernel(int32_t* counts, int32_t* offsets,
                                                          int E) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < E) counts[i] = 0;
  if (i <= E) offsets[i] = 0;
}

hipError_t launch_zero_counts(int32_t* counts, int32_t* offsets, int E, hipStream_t s) {
  hipLaunchKernelGGL(zero_counts_kernel, dim3(E / 256 + 1), dim3(256), 0, s, counts, offsets, E);
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// Row list of a dense gated FFN run through the grouped GEMMs (the dense
// layers of the model; hyper.ai summary, 方法, and paperlayer.ai summary,
// §2.2: the first layers use a dense FFN; model card: intermediate_size).
// The intermediate dimension is cut into S slices, slice s acting as group
// s: every token t is row s*T + t of group s with weight 1, and slot s of
// token t points at that row, so the combine adds the S partial outputs of
// a token in slice order.  Blocks of one slice are consecutive.
__global__ __launch_bounds__(256) void dense_rows_kernel(int T, int S, int bn, int gran,
                                                         int32_t* row_token, float* row_w,
                                                         int32_t* slot_pos, RowBlock* rb,
                                                         int32_t* n_rb) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int per = (T + bn - 1) / bn;   // blocks per slice
  if (i < S * T) {
    const int sl = i / T, t = i - sl * T;
    row_token[i] = t;
    row_w[i] = 1.0f;
    slot_pos[(size_t)t * S + sl] = i;
  }
  if (i < S * per) {
    const int sl = i / per, b = i - sl * per;
    RowBlock blk{};
    blk.group = sl;
    int st, n;
    split_block(T, per, gran, b, &st, &n);
    blk.row_start = sl * T + st;
    blk.n_rows = n;
    blk.first = sl * per;
    blk.n_group = per;
    blk.group_row0 = sl * T;
    blk.group_rows = T;
    rb[i] = blk;
  }
  if (i == 0) *n_rb = S * per;
  if (i == 1 || i == 2) n_rb[i] = 0;   // the GEMMs' pool claim counters
}

hipError_t launch_dense_rows(const Plan& p, int32_t* row_token, float* row_w, int32_t* slot_pos,
                             RowBlock* rb, int32_t* n_rb, hipStream_t s) {
  // p.E = p.K = S slices, p.KT = S * T rows
  const int n = p.KT;
  hipLaunchKernelGGL(dense_rows_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p.T, p.E, p.bn,
                     p.rb_gran, row_token, row_w, slot_pos, rb, n_rb);
  return hipGetLastError();
}

}  // namespace smoe
