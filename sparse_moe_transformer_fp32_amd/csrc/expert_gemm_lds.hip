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
// Pipeline: a ring of NS stages in LDS, one 32-wide k-step per stage.  Every
// operand tile is moved global -> LDS by global_load_lds_dwordx4 (lane l's
// 16 bytes land at tile base + 16 l): a packed weight tile is one contiguous
// kilobyte already in MFMA A-operand lane order, and a token tile is gathered
// row by row straight into B-operand lane order, so all LDS reads are
// conflict-free ds_read_b128.  Per k-step: wait for this wave's loads of the
// stage, barrier (all waves' token loads landed, and the slot of the previous
// stage is free), issue the loads of the stage NS-1 ahead into that slot,
// multiply.  Token fragments past the block's rows are skipped.
//
// XCD-aware order: block b runs on XCD b % 8; work items are dealt so that
// each XCD walks a contiguous range of (row block, weight tile) items, which
// keeps a row block's token rows (and repeated weight tiles of one expert's
// consecutive row blocks) in that XCD's L2.
#include "smoe_internal.h"

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

template <int MODE, int NB, int NS>
__global__ __launch_bounds__(256) void expert_gemm_lds_kernel(LdsGemmParams P) {
  constexpr int FRW = 4;                  // weight fragments per wave
  constexpr int NBW = NB / 4;             // token fragments each wave loads
  static_assert(NB % 4 == 0, "token fragments are loaded 4 ways");
  constexpr int STAGE_A = 4 * FRW * 1024; // bytes of weight tiles per stage
  constexpr int STAGE = STAGE_A + NB * 1024;
  constexpr int LOADS = FRW + NBW;        // loads per wave per stage
  static_assert(NS == 4 || NS == 5, "the k-loop below is unrolled for 4- or 5-slot rings");
  // one array per ring slot: the compiler can tell the slot being filled
  // from the slot being read, so it adds no waits of its own between them
  __shared__ __attribute__((aligned(1024))) unsigned char ring0[STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char ring1[STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char ring2[STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char ring3[STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char ring4[NS == 5 ? STAGE : 16];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;

  // XCD-aware deal of (row block, weight tile) work items
  const int n_items = *P.n_rb * P.tiles;
  const int per = (n_items + 7) >> 3;
  const int slot_b = blockIdx.x >> 3;
  if (slot_b >= per) return;
  const int item = (blockIdx.x & 7) * per + slot_b;
  if (item >= n_items) return;
  const int rbi = item / P.tiles;
  const int tile = item - rbi * P.tiles;
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

  auto issue = [&](unsigned char* st, int step) {
    const int ks = min(step, nsteps - 1);   // past the end: harmless re-load
#pragma unroll
    for (int f = 0; f < FRW; ++f)
      __builtin_amdgcn_global_load_lds((glob_void_t*)(wsrc[f] + (size_t)ks * 512),
                                       (lds_void_t*)(st + (wave * FRW + f) * 1024), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < NBW; ++i)
      __builtin_amdgcn_global_load_lds((glob_void_t*)(tsrc[i] + ks * 32),
                                       (lds_void_t*)(st + STAGE_A + (wave * NBW + i) * 1024), 16,
                                       0, 0);
  };

  f32x4 acc[FRW][NB];
#pragma unroll
  for (int f = 0; f < FRW; ++f)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[f][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const unsigned char* st) {
    // all fragment reads first (fragments past the block hold valid repeated
    // rows), then the MFMAs of the fragments with real rows
    u32x4 a[FRW], b[NB];
#pragma unroll
    for (int f = 0; f < FRW; ++f)
      a[f] = *reinterpret_cast<const u32x4*>(st + (wave * FRW + f) * 1024 + lane * 16);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      b[nb] = *reinterpret_cast<const u32x4*>(st + STAGE_A + nb * 1024 + lane * 16);
    __builtin_amdgcn_sched_barrier(0);  // keep every read ahead of the MFMAs
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if (nb < nb_act) {
#pragma unroll
        for (int f = 0; f < FRW; ++f)
          acc[f][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, a[f]), __builtin_bit_cast(bf16x8, b[nb]), acc[f][nb], 0,
              0, 0);
      }
    }
  };
  // one k-step: this wave's loads of the step have landed (the NS-2 later
  // stages may still be in flight); the barrier makes everyone's visible and
  // frees the slot read one step earlier, which then takes the step NS-1 ahead
  auto step = [&](unsigned char* cur, unsigned char* next_free, int k) {
    wait_vmcnt<LOADS * (NS - 2)>();
    __builtin_amdgcn_s_barrier();
    issue(next_free, k + NS - 1);
    compute(cur);
  };

  int k = 0;
  if constexpr (NS == 4) {
    issue(ring0, 0);
    issue(ring1, 1);
    issue(ring2, 2);
    for (; k + 4 <= nsteps; k += 4) {
      step(ring0, ring3, k);
      step(ring1, ring0, k + 1);
      step(ring2, ring1, k + 2);
      step(ring3, ring2, k + 3);
    }
    if (k < nsteps) step(ring0, ring3, k);
    if (k + 1 < nsteps) step(ring1, ring0, k + 1);
    if (k + 2 < nsteps) step(ring2, ring1, k + 2);
  } else {
    issue(ring0, 0);
    issue(ring1, 1);
    issue(ring2, 2);
    issue(ring3, 3);
    for (; k + 5 <= nsteps; k += 5) {
      step(ring0, ring4, k);
      step(ring1, ring0, k + 1);
      step(ring2, ring1, k + 2);
      step(ring3, ring2, k + 3);
      step(ring4, ring3, k + 4);
    }
    if (k < nsteps) step(ring0, ring4, k);
    if (k + 1 < nsteps) step(ring1, ring0, k + 1);
    if (k + 2 < nsteps) step(ring2, ring1, k + 2);
    if (k + 3 < nsteps) step(ring3, ring2, k + 3);
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
  hipLaunchKernelGGL((expert_gemm_lds_kernel<0, 12, 4>), dim3(lds_grid(p, p.gu_tiles)), dim3(256),
                     0, s, gp);
  return hipGetLastError();
}

hipError_t launch_down_lds(const Plan& p, const DownArgs& a, hipStream_t s) {
  LdsGemmParams gp{};
  gp.wa0 = a.wd; gp.sa0 = a.sd; gp.bsrc = a.h; gp.row_w = a.row_w;
  gp.rb = a.rb; gp.n_rb = a.n_rb; gp.out = a.o;
  gp.E = p.E; gp.H = p.H; gp.I = p.I; gp.Is = p.Is; gp.KT = p.KT; gp.tiles = p.dn_tiles;
  hipLaunchKernelGGL((expert_gemm_lds_kernel<1, 12, 4>), dim3(lds_grid(p, p.dn_tiles)), dim3(256),
                     0, s, gp);
  return hipGetLastError();
}

}  // namespace smoe
