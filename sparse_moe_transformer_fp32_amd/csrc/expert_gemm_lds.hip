// Grouped expert GEMMs for large row blocks (prefill), gfx950.
//
//   gate/up:  h[r, i] = silu(x_t . Wg_e[i]) * (x_t . Wu_e[i])   (t = row_token[r])
//   down:     o[r, n] = w_r * (h[r] . Wd_e[n])
//
// Sources: paperlayer.ai summary, App. B (Detail Analysis of Localized
// Activation Blow-up): SwiGLU experts; LLM Atlas model card "Step-3.5-Flash",
// raw config field table: moe_intermediate_size 1280, hidden_size 4096,
// torch_dtype bfloat16.
//
// Workgroup tile: 16 packed weight fragments (256 weight rows; for gate/up
// 128 intermediate columns as gate/up pairs) x one row block of up to 16*NB
// tokens.  Each of the 4 waves owns 4 fragments and multiplies them with
// every token fragment of the block, so each weight element is read from
// HBM once per row block.
//
// Pipeline, one 32-wide k-step per stage.  The token tile of a stage is
// shared by all waves: it is gathered row by row straight into B-operand lane
// order in an NS-slot LDS ring by global_load_lds_dwordx4 (lane l's 16 bytes
// land at tile base + 16 l), so LDS reads are conflict-free ds_read_b128.
// Each weight fragment is used by one wave only, so weights skip LDS: a
// packed weight tile is one contiguous kilobyte already in A-operand lane
// order and goes straight into a 4-slot register ring, NS-1 steps ahead.
// Token operands are double-buffered in registers (the LDS reads of step k+1
// overlap the MFMAs of step k).  Token fragments past the block's rows are
// skipped.
//
// XCD-aware order: block b runs on XCD b % 8; work items are dealt so that
// each XCD walks a contiguous range of items ordered (group, weight tile,
// row block).  Workgroups that run side by side on one XCD then share weight
// tiles (across an expert's row blocks) and token rows (across weight tiles),
// and since they advance through K at about the same pace, each k-step's
// tiles are fetched from HBM once and served to the others from L2.
#include "smoe_internal.h"

#include <type_traits>

#ifndef SMOE_LDS_STAGES
#define SMOE_LDS_STAGES 4
#endif

namespace smoe {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void glob_void_t;

struct LdsGemmParams {
  const uint16_t* wa0;   // gate/up: gate (packed) [E,I,H];  down: down (packed) [E,H,I]
  const uint16_t* wa1;   // gate/up: up (packed)
  const uint16_t* sa0;   // shared gate / shared down (packed)
  const uint16_t* sa1;   // shared up (packed)
  const uint16_t* bsrc;  // gate/up: x [T,H];  down: h
  const int32_t* row_token;
  const float* row_w;
  const RowBlock* rb;
  const int32_t* n_rb;
  uint16_t* out;
  int E, H, I, Is, KT, tiles;
  float limit, limit_shared;
};

__device__ inline uint32_t pack_bf16x2_l(float a, float b) {
  const __bf16 ha = (__bf16)a, hb = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) |
         ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

// s_waitcnt vmcnt(n) with the other counters left unconstrained (gfx9
// encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] at [15:14]).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | (((N >> 4) & 3) << 14));
}

// s_waitcnt vmcnt(n) lgkmcnt(0): also every LDS read of this wave is done.
template <int N>
__device__ inline void wait_vmcnt_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0x0 << 8) | (((N >> 4) & 3) << 14));
}

template <int MODE, int NB, int NS>
__global__ __launch_bounds__(256) void expert_gemm_lds_kernel(LdsGemmParams P) {
  constexpr int FRW = 4;                  // weight fragments per wave
  constexpr int NBW = NB / 4;             // token fragments each wave loads
  static_assert(NB % 4 == 0, "token fragments are loaded 4 ways");
  constexpr int STAGE = NB * 1024;         // bytes of token tiles per stage
  constexpr int LOADS = FRW + NBW;        // vector-memory ops per wave per stage
  static_assert(NS % 2 == 0 && NS >= 4 && NS <= 8, "ring of 4, 6 or 8 slots");
  static_assert(LOADS * (NS - 1) < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) unsigned char ring[NS][STAGE];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;

  // XCD-aware deal of work items; items run in (group, weight tile, row
  // block) order, so the row blocks that share a weight tile and the tiles
  // that share a row block run side by side on one XCD and meet in its L2
  const int n_items = *P.n_rb * P.tiles;
  const int per = (n_items + 7) >> 3;
  const int slot_b = blockIdx.x >> 3;
  if (slot_b >= per) return;
  const int item = (blockIdx.x & 7) * per + slot_b;
  if (item >= n_items) return;
  // a group's items fill [first * tiles, (first + n_group) * tiles)
  const RowBlock any = P.rb[item / P.tiles];
  const int local = item - any.first * P.tiles;
  const int tile = local / any.n_group;
  const int rbi = any.first + (local - tile * any.n_group);
  if (rbi >= *P.n_rb) return;
  const RowBlock blk = P.rb[rbi];
  const bool shared = blk.group == P.E;
  const int inter = shared ? P.Is : P.I;
  const int nout = (MODE == 0) ? inter : P.H;
  const int col0 = tile * (MODE == 0 ? 128 : 256);  // first output column of the workgroup
  if (col0 >= nout) return;                          // uniform over the workgroup
  const int Kdim = (MODE == 0) ? P.H : inter;
  const int nsteps = Kdim >> 5;
  const int nb_act = (blk.n_rows + 15) >> 4;         // token fragments with real rows

  // this wave's weight fragments (packed, row-tile-major)
  const uint16_t* wsrc[FRW];
  if (MODE == 0) {
    const uint16_t* Wg = shared ? P.sa0 : P.wa0 + (size_t)blk.group * P.I * P.H;
    const uint16_t* Wu = shared ? P.sa1 : P.wa1 + (size_t)blk.group * P.I * P.H;
#pragma unroll
    for (int f = 0; f < FRW; ++f) {
      const int rt = (col0 >> 4) + wave * 2 + (f >> 1);
      wsrc[f] = ((f & 1) ? Wu : Wg) + (size_t)rt * nsteps * 512 + lane * 8;
    }
  } else {
    const uint16_t* Wd = shared ? P.sa0 : P.wa0 + (size_t)blk.group * P.H * P.I;
#pragma unroll
    for (int f = 0; f < FRW; ++f) {
      const int rt = (col0 >> 4) + wave * FRW + f;
      wsrc[f] = Wd + (size_t)rt * nsteps * 512 + lane * 8;
    }
  }
  // token fragments this wave loads: nb = wave*NBW + i; rows past the block
  // repeat its last row
  const uint16_t* tsrc[NBW];
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    const int nb = wave * NBW + i;
    const int row = blk.row_start + min(nb * 16 + r, blk.n_rows - 1);
    const uint16_t* base;
    if (MODE == 0)
      base = P.bsrc + (size_t)P.row_token[row] * P.H;
    else
      base = shared ? P.bsrc + (size_t)P.KT * P.I + (size_t)(row - P.KT) * P.Is
                    : P.bsrc + (size_t)row * P.I;
    tsrc[i] = base + 8 * g;
  }

  f32x4 acc[FRW][NB];
#pragma unroll
  for (int f = 0; f < FRW; ++f)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[f][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // past the end of K every load re-reads the last step (harmless, in bounds)
  auto load_w = [&](u32x4 (&a)[FRW], int step) {
    const int ks = min(step, nsteps - 1);
#pragma unroll
    for (int f = 0; f < FRW; ++f)
      a[f] = *reinterpret_cast<const u32x4*>(wsrc[f] + (size_t)ks * 512);
  };
  auto load_t = [&](unsigned char* st, int step) {
    const int ks = min(step, nsteps - 1);
#pragma unroll
    for (int i = 0; i < NBW; ++i)
      __builtin_amdgcn_global_load_lds((glob_void_t*)(tsrc[i] + ks * 32),
                                       (lds_void_t*)(st + (wave * NBW + i) * 1024), 16, 0, 0);
  };
  auto read_t = [&](const unsigned char* st, u32x4 (&b)[NB]) {
    // fragments past the block hold valid repeated rows; their MFMAs are skipped
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      b[nb] = *reinterpret_cast<const u32x4*>(st + nb * 1024 + lane * 16);
  };
  auto mma = [&](const u32x4 (&a)[FRW], const u32x4 (&b)[NB]) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if (nb < nb_act) {
#pragma unroll
        for (int f = 0; f < FRW; ++f)
          acc[f][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, a[f]), __builtin_bit_cast(bf16x8, b[nb]), acc[f][nb],
              0, 0, 0);
      }
    }
  };
  // One k-step (j = k mod NS, a compile-time slot index).  Step k issues the
  // weights of step k+NS-1 and the tokens of step k+NS.  The tokens of step
  // k+1 were issued NS-1 steps ago, so exactly NS-2 steps' ops are younger:
  // the wait below completes the weights of step k and the tokens of step
  // k+1 (and, lgkmcnt(0), this wave's LDS reads of step k).  The barrier then
  // makes everyone's token tile k+1 visible and frees slot j for step k+NS.
  u32x4 w[NS][FRW];
  u32x4 t[2][NB];
  auto step = [&](auto jc, int k) {
    constexpr int j = decltype(jc)::value;
    wait_vmcnt_lds<LOADS * (NS - 2)>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);  // this step's loads stay after the wait
    load_w(w[(j + NS - 1) % NS], k + NS - 1);
    load_t(ring[j], k + NS);
    read_t(ring[(j + 1) % NS], t[(j + 1) % 2]);
    __builtin_amdgcn_sched_barrier(0);  // the loads go out before the MFMAs
    mma(w[j], t[j % 2]);
  };

  // prologue, issued in this exact order (scheduling barriers keep the
  // compiler from interleaving the groups): T0 W0 T1 W1 ... T(NS-2) W(NS-2) T(NS-1)
#pragma unroll
  for (int s2 = 0; s2 < NS - 1; ++s2) {
    load_t(ring[s2], s2);
    load_w(w[s2], s2);
    __builtin_amdgcn_sched_barrier(0);
  }
  load_t(ring[NS - 1], NS - 1);
  __builtin_amdgcn_sched_barrier(0);
  // T0 and W0 are the LOADS oldest ops: wait until the rest remain
  wait_vmcnt_lds<LOADS * (NS - 2) + NBW>();
  __builtin_amdgcn_s_barrier();
  read_t(ring[0], t[0]);
  int k = 0;
  for (; k + NS <= nsteps; k += NS) {
    step(std::integral_constant<int, 0>{}, k);
    step(std::integral_constant<int, 1>{}, k + 1);
    step(std::integral_constant<int, 2>{}, k + 2);
    step(std::integral_constant<int, 3>{}, k + 3);
    if constexpr (NS > 4) {
      step(std::integral_constant<int, 4 % NS>{}, k + 4);
      step(std::integral_constant<int, 5 % NS>{}, k + 5);
    }
    if constexpr (NS > 6) {
      step(std::integral_constant<int, 6 % NS>{}, k + 6);
      step(std::integral_constant<int, 7 % NS>{}, k + 7);
    }
  }
  // tail: the remaining steps continue the same slot sequence
  if (k < nsteps) step(std::integral_constant<int, 0>{}, k);
  if (k + 1 < nsteps) step(std::integral_constant<int, 1>{}, k + 1);
  if (k + 2 < nsteps) step(std::integral_constant<int, 2>{}, k + 2);
  if constexpr (NS > 4) {
    if (k + 3 < nsteps) step(std::integral_constant<int, 3>{}, k + 3);
    if (k + 4 < nsteps) step(std::integral_constant<int, 4 % NS>{}, k + 4);
  }
  if constexpr (NS > 6) {
    if (k + 5 < nsteps) step(std::integral_constant<int, 5 % NS>{}, k + 5);
    if (k + 6 < nsteps) step(std::integral_constant<int, 6 % NS>{}, k + 6);
  }
  wait_vmcnt<0>();  // no LDS write may be in flight when the workgroup ends

  // epilogue: lane holds output columns (frag base) + 4g..4g+3 of token row r
  const int cw = col0 + wave * (MODE == 0 ? 32 : 64);   // this wave's first column
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int lr = nb * 16 + r;
    if (nb >= nb_act || lr >= blk.n_rows) continue;
    const int row = blk.row_start + lr;
    if (MODE == 0) {
      const float lim = shared ? P.limit_shared : P.limit;
      uint16_t* hrow = shared ? P.out + (size_t)P.KT * P.I + (size_t)(row - P.KT) * P.Is
                              : P.out + (size_t)row * P.I;
#pragma unroll
      for (int pf = 0; pf < FRW / 2; ++pf) {
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
        pk[0] = pack_bf16x2_l(hv[0], hv[1]);
        pk[1] = pack_bf16x2_l(hv[2], hv[3]);
        *reinterpret_cast<u32x2*>(hrow + cw + pf * 16 + 4 * g) = pk;
      }
    } else {
      const float w = P.row_w[row];
      uint16_t* orow = P.out + (size_t)row * P.H;
#pragma unroll
      for (int f = 0; f < FRW; ++f) {
        u32x2 pk;
        pk[0] = pack_bf16x2_l(acc[f][nb][0] * w, acc[f][nb][1] * w);
        pk[1] = pack_bf16x2_l(acc[f][nb][2] * w, acc[f][nb][3] * w);
        *reinterpret_cast<u32x2*>(orow + cw + f * 16 + 4 * g) = pk;
      }
    }
  }
}

// grid: enough blocks for every (row block, weight tile) item, rounded up to
// a multiple of the 8 XCDs
static unsigned lds_grid(const Plan& p, int tiles) {
  const long long items = (long long)p.rb_max * tiles;
  return (unsigned)((items + 7) / 8 * 8);
}

hipError_t launch_gate_up_lds(const Plan& p, const GateUpArgs& a, hipStream_t s) {
  LdsGemmParams gp{};
  gp.wa0 = a.wg; gp.wa1 = a.wu; gp.sa0 = a.sg; gp.sa1 = a.su; gp.bsrc = a.x;
  gp.row_token = a.row_token; gp.rb = a.rb; gp.n_rb = a.n_rb; gp.out = a.h;
  gp.E = p.E; gp.H = p.H; gp.I = p.I; gp.Is = p.Is; gp.KT = p.KT; gp.tiles = p.gu_tiles;
  gp.limit = a.limit; gp.limit_shared = a.limit_shared;
  hipLaunchKernelGGL((expert_gemm_lds_kernel<0, 12, SMOE_LDS_STAGES>), dim3(lds_grid(p, p.gu_tiles)), dim3(256),
                     0, s, gp);
  return hipGetLastError();
}

hipError_t launch_down_lds(const Plan& p, const DownArgs& a, hipStream_t s) {
  LdsGemmParams gp{};
  gp.wa0 = a.wd; gp.sa0 = a.sd; gp.bsrc = a.h; gp.row_w = a.row_w;
  gp.rb = a.rb; gp.n_rb = a.n_rb; gp.out = a.o;
  gp.E = p.E; gp.H = p.H; gp.I = p.I; gp.Is = p.Is; gp.KT = p.KT; gp.tiles = p.dn_tiles;
  hipLaunchKernelGGL((expert_gemm_lds_kernel<1, 12, SMOE_LDS_STAGES>), dim3(lds_grid(p, p.dn_tiles)), dim3(256),
                     0, s, gp);
  return hipGetLastError();
}

}  // namespace smoe
