// Grouped expert GEMMs of the MoE layer on gfx950 (bf16 MFMA, fp32 accumulate).
//
//   gate/up:  h[r, i] = silu(x_t . Wg_e[i]) * (x_t . Wu_e[i])   (t = row_token[r])
//   down:     o[r, n] = w_r * (h[r] . Wd_e[n])
//
// Sources: paperlayer.ai summary, App. B (Detail Analysis of Localized
// Activation Blow-up): SwiGLU experts whose gate and up activations are
// multiplied element-wise; LLM Atlas model card "Step-3.5-Flash", raw config
// field table: moe_intermediate_size 1280, share_expert_dim 1280,
// hidden_size 4096, torch_dtype bfloat16, swiglu_limits.
//
// Design (weight-streaming): every weight element is read from HBM exactly
// once per row block and goes straight from global memory into the MFMA A
// operand registers of the one wave that uses it -- no LDS round trip.
// Weights arrive fragment-packed (see pack.hip): each wave-wide A load is one
// contiguous kilobyte.  The
// token rows (B operand) are small and hot in L2.  A wave owns FR fragments
// of 16 weight rows and all 16*NB rows of its row block; KSPLIT waves of a
// workgroup split K (interleaved k steps) and add their partial sums in a
// fixed order through LDS
// (so small-T launches have enough, small enough workgroups to balance the
// weight stream over the CUs).
//
// 16x16x32 bf16 MFMA operand layout (lane l, r = l & 15, g = l >> 4):
//   A: row r, k = 8g..8g+7    B: column r, k = 8g..8g+7
//   C: rows 4g..4g+3 of column r
// Each lane reads its 16 contiguous bytes of a packed weight tile and of a
// token row at the same k range.
#include "smoe_internal.h"

namespace smoe {

struct GemmParams {
  const uint16_t* wa0;     // gate/up: gate [E,I,H];  down: down [E,H,I]
  const uint16_t* wa1;     // gate/up: up [E,I,H]
  const uint16_t* sa0;     // shared gate [Is,H] / shared down [H,Is]
  const uint16_t* sa1;     // shared up [Is,H]
  const uint16_t* bsrc;    // gate/up: x [T,H];  down: h
  const int32_t* row_token;
  const float* row_w;
  const RowBlock* rb;
  const int32_t* n_rb;
  uint16_t* out;           // gate/up: h;  down: o [rows, H]
  int E, H, I, Is, KT, tiles;
  float limit, limit_shared;
};

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  const __bf16 ha = (__bf16)a, hb = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) |
         ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

__device__ inline f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <int KSPLIT, int FR, int NB>
constexpr int red_slots() { return ((KSPLIT > 1) ? (4 - 4 / KSPLIT) : 1) * FR * NB * 64; }

// One workgroup's tile of one row block.  MODE 0: gate/up + SwiGLU.  MODE 1:
// down + combine weight.  NT: the weight loads are non-temporal.
template <int MODE, int NB, int FR, int KSPLIT, int U, bool NT>
__device__ __forceinline__ void gemm_tile(const GemmParams& P, const RowBlock& blk, int tile,
                                          f32x4* s_red) {
  constexpr int RG = 4 / KSPLIT;                       // row groups per workgroup
  constexpr int WROWS = (MODE == 0) ? 8 * FR : 16 * FR;  // output columns per wave

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rg = wave / KSPLIT, kp = wave % KSPLIT;
  const int r = lane & 15, g = lane >> 4;
  const bool shared = blk.group == P.E;
  const int inter = shared ? P.Is : P.I;
  const int nout = (MODE == 0) ? inter : P.H;          // output columns of this group
  const int col0 = tile * (RG * WROWS);
  if (col0 >= nout) return;                            // whole workgroup: uniform
  const int cbase = col0 + rg * WROWS;                 // this wave's first column
  const int Kdim = (MODE == 0) ? P.H : inter;
  const int klen = Kdim / KSPLIT;
  const int kbeg = kp * 32 + 8 * g;

  // A operand: fragment-packed weights (16x32 tiles of 1 KB in lane order,
  // row-tile-major).  The KSPLIT waves of a row group take every KSPLIT-th
  // 32-wide k step, so together they read each row tile's kilobytes front to
  // back: one sequential stream per row tile and workgroup.  (With
  // non-temporal loads, a plain read kernel reaches ~6.0 TB/s when each of
  // four waves reads its own contiguous quarter of a region, ~7.0 TB/s when
  // the four interleave like this.)
  const int ksteps = Kdim / 32;
  const int kstep0 = kp;
  const uint16_t* aptr[FR];
  if (MODE == 0) {
    const uint16_t* Wg = shared ? P.sa0 : P.wa0 + (size_t)blk.group * P.I * P.H;
    const uint16_t* Wu = shared ? P.sa1 : P.wa1 + (size_t)blk.group * P.I * P.H;
#pragma unroll
    for (int f = 0; f < FR; ++f) {
      const int rt = (cbase >> 4) + (f >> 1);
      aptr[f] = ((f & 1) ? Wu : Wg) + ((size_t)rt * ksteps + kstep0) * 512 + lane * 8;
    }
  } else {
    const uint16_t* Wd = shared ? P.sa0 : P.wa0 + (size_t)blk.group * P.H * P.I;
#pragma unroll
    for (int f = 0; f < FR; ++f) {
      const int rt = (cbase >> 4) + f;
      aptr[f] = Wd + ((size_t)rt * ksteps + kstep0) * 512 + lane * 8;
    }
  }
  // B operand rows (tokens); rows past the block repeat its last row
  const uint16_t* bptr[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int row = blk.row_start + min(nb * 16 + r, blk.n_rows - 1);
    if (MODE == 0) {
      bptr[nb] = P.bsrc + (size_t)P.row_token[row] * P.H + kbeg;
    } else {
      const uint16_t* hrow = shared ? P.bsrc + (size_t)P.KT * P.I + (size_t)(row - P.KT) * P.Is
                                    : P.bsrc + (size_t)row * P.I;
      bptr[nb] = hrow + kbeg;
    }
  }

  f32x4 acc[FR][NB];
#pragma unroll
  for (int f = 0; f < FR; ++f)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[f][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Software pipeline over stages of U k-steps with two register buffers.
  // Every load is unconditional so the compiler's wait counts let one stage
  // stream in while the other is multiplied; slots past the end of K re-read
  // the last valid chunk (in bounds) and skip their MFMAs.  Token rows,
  // re-read by every workgroup of their row block, are ordinary loads.
  const int nsteps = klen / 32;
  const int nstages = (nsteps + U - 1) / U;
  u32x4 a0[U][FR], b0[U][NB], a1[U][FR], b1[U][NB];
  auto load = [&](u32x4 (&a)[U][FR], u32x4 (&b)[U][NB], int stage) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ks = min(stage * U + u, nsteps - 1);
#pragma unroll
      for (int f = 0; f < FR; ++f) {
        const u32x4* src = reinterpret_cast<const u32x4*>(aptr[f] + (size_t)ks * (KSPLIT * 512));
        a[u][f] = NT ? __builtin_nontemporal_load(src) : *src;
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        b[u][nb] = *reinterpret_cast<const u32x4*>(bptr[nb] + ks * (KSPLIT * 32));
    }
  };
  auto compute = [&](const u32x4 (&a)[U][FR], const u32x4 (&b)[U][NB], int stage) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (stage * U + u < nsteps) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int f = 0; f < FR; ++f) acc[f][nb] = mfma16(a[u][f], b[u][nb], acc[f][nb]);
      }
    }
  };

  load(a0, b0, 0);
  int st = 0;
  for (; st + 2 < nstages; st += 2) {
    load(a1, b1, st + 1);
    compute(a0, b0, st);
    load(a0, b0, st + 2);
    compute(a1, b1, st + 1);
  }
  if (st + 1 < nstages) {
    load(a1, b1, st + 1);
    compute(a0, b0, st);
    compute(a1, b1, st + 1);
  } else {
    compute(a0, b0, st);
  }

  if (KSPLIT > 1) {
    // waves kp > 0 park their partial sums; kp == 0 adds them in order
    if (kp > 0) {
      const int slot = rg * (KSPLIT - 1) + (kp - 1);
#pragma unroll
      for (int f = 0; f < FR; ++f)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) s_red[((slot * FR + f) * NB + nb) * 64 + lane] = acc[f][nb];
    }
    __syncthreads();
    if (kp > 0) return;
#pragma unroll
    for (int q = 1; q < KSPLIT; ++q) {
      const int slot = rg * (KSPLIT - 1) + (q - 1);
#pragma unroll
      for (int f = 0; f < FR; ++f)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[f][nb] += s_red[((slot * FR + f) * NB + nb) * 64 + lane];
    }
  }

  // epilogue: lane holds output columns cbase + 16*frag + 4g .. +3 of row r
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int lr = nb * 16 + r;
    if (lr >= blk.n_rows) continue;
    const int row = blk.row_start + lr;
    if (MODE == 0) {
      const float lim = shared ? P.limit_shared : P.limit;
      uint16_t* hrow = shared ? P.out + (size_t)P.KT * P.I + (size_t)(row - P.KT) * P.Is
                              : P.out + (size_t)row * P.I;
#pragma unroll
      for (int pf = 0; pf < FR / 2; ++pf) {
        float hv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float gv = acc[2 * pf][nb][j];
          float uv = acc[2 * pf + 1][nb][j];
          if (lim > 0.f) {
            gv = fminf(gv, lim);
            uv = fminf(fmaxf(uv, -lim), lim);
          }
          hv[j] = gv / (1.0f + __expf(-gv)) * uv;
        }
        u32x2 pk;
        pk[0] = pack_bf16x2(hv[0], hv[1]);
        pk[1] = pack_bf16x2(hv[2], hv[3]);
        *reinterpret_cast<u32x2*>(hrow + cbase + pf * 16 + 4 * g) = pk;
      }
    } else {
      const float w = P.row_w[row];
      uint16_t* orow = P.out + (size_t)row * P.H;
#pragma unroll
      for (int f = 0; f < FR; ++f) {
        u32x2 pk;
        pk[0] = pack_bf16x2(acc[f][nb][0] * w, acc[f][nb][1] * w);
        pk[1] = pack_bf16x2(acc[f][nb][2] * w, acc[f][nb][3] * w);
        *reinterpret_cast<u32x2*>(orow + cbase + f * 16 + 4 * g) = pk;
      }
    }
  }
}

// The grid covers rb_max row blocks x tiles; workgroups past the list's end
// exit.  A row block that is its group's only one is the single reader of
// its weight tile, which then streams with non-temporal loads: they lift the
// HBM read rate (a plain read kernel moves ~6.2 TB/s with ordinary loads and
// ~7.0 TB/s with non-temporal ones).  Tiles that several row blocks read use
// ordinary loads, so the blocks after the first find them in L2.
template <int MODE, int NB, int FR, int KSPLIT, int U>
__global__ __launch_bounds__(256) void expert_gemm_kernel(GemmParams P) {
  __shared__ f32x4 s_red[red_slots<KSPLIT, FR, NB>()];
  const int tile = blockIdx.x % P.tiles;
  const int rbi = blockIdx.x / P.tiles;
  // both loads at once: rbi < rb_max, so the entry is in bounds even past
  // the list's end (where it is not used)
  const RowBlock blk = P.rb[rbi];
  if (rbi >= *P.n_rb) return;
  if (blk.n_group == 1)
    gemm_tile<MODE, NB, FR, KSPLIT, U, true>(P, blk, tile, s_red);
  else
    gemm_tile<MODE, NB, FR, KSPLIT, U, false>(P, blk, tile, s_red);
}

// --------------------------------------------------------------------------
// Launch configurations.  Row blocks of 16 tokens (decode): one 16-row
// fragment pair per wave, four waves split K, so a workgroup streams
// 16 x 2 x H weights and there are many small workgroups to balance.  Row
// blocks of 32 or 64 tokens: waves own different weight rows.  Larger row
// blocks use the LDS-pipelined kernels (expert_gemm_lds.hip).
template <int MODE>
static hipError_t launch_mode(const Plan& p, const GemmParams& gp, int ksplit, hipStream_t s) {
  const int grid = p.rb_max * gp.tiles;
  if (grid == 0) return hipSuccess;
  switch (p.nb) {
    case 1:
      if (ksplit == 4)
        hipLaunchKernelGGL((expert_gemm_kernel<MODE, 1, 2, 4, 4>), dim3(grid), dim3(256), 0, s, gp);
      else if (ksplit == 2)
        hipLaunchKernelGGL((expert_gemm_kernel<MODE, 1, 2, 2, 4>), dim3(grid), dim3(256), 0, s, gp);
      else
        hipLaunchKernelGGL((expert_gemm_kernel<MODE, 1, 2, 1, 4>), dim3(grid), dim3(256), 0, s, gp);
      break;
    case 2:
      hipLaunchKernelGGL((expert_gemm_kernel<MODE, 2, 2, 1, 2>), dim3(grid), dim3(256), 0, s, gp);
      break;
    case 4:
      hipLaunchKernelGGL((expert_gemm_kernel<MODE, 4, 2, 1, 2>), dim3(grid), dim3(256), 0, s, gp);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gate_up(const Plan& p, const GateUpArgs& a, hipStream_t s) {
  GemmParams gp{};
  gp.wa0 = a.wg;
  gp.wa1 = a.wu;
  gp.sa0 = a.sg;
  gp.sa1 = a.su;
  gp.bsrc = a.x;
  gp.row_token = a.row_token;
  gp.rb = a.rb;
  gp.n_rb = a.n_rb;
  gp.out = a.h;
  gp.E = p.E; gp.H = p.H; gp.I = p.I; gp.Is = p.Is; gp.KT = p.KT;
  gp.tiles = p.gu_tiles;
  gp.limit = a.limit;
  gp.limit_shared = a.limit_shared;
  return launch_mode<0>(p, gp, p.ksplit_gu, s);
}

hipError_t launch_down(const Plan& p, const DownArgs& a, hipStream_t s) {
  GemmParams gp{};
  gp.wa0 = a.wd;
  gp.sa0 = a.sd;
  gp.bsrc = a.h;
  gp.row_w = a.row_w;
  gp.rb = a.rb;
  gp.n_rb = a.n_rb;
  gp.out = a.o;
  gp.E = p.E; gp.H = p.H; gp.I = p.I; gp.Is = p.Is; gp.KT = p.KT;
  gp.tiles = p.dn_tiles;
  return launch_mode<1>(p, gp, p.ksplit_dn, s);
}

}  // namespace smoe
