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

struct NoFill {
  __device__ void operator()() const {}
};

// One workgroup's tile of one row block.  MODE 0: gate/up + SwiGLU.  MODE 1:
// down + combine weight.  NT: the weight loads are non-temporal.  DENSE: the
// row block is a whole slice of the dense FFN, whose row i is token i.
// BL: the B operands (16 token rows) are read from LDS (`xl`, rows `xpitch`
// bytes apart, row r holding token min(r, T-1)), which `fill` writes and
// publishes right after the first weight loads are issued; the tile is then
// run by waves 4 j .. 4 j + 3 of the workgroup, whichever j.
template <int MODE, int NB, int FR, int KSPLIT, int U, bool NT, bool DENSE = false,
          bool BL = false, typename Fill = NoFill>
__device__ __forceinline__ void gemm_tile(const GemmParams& P, const RowBlock& blk, int tile,
                                          f32x4* s_red, const unsigned char* xl = nullptr,
                                          int xpitch = 0, Fill fill = Fill{}) {
  static_assert(!BL || (KSPLIT == 4 && NB == 1 && MODE == 0), "LDS B operands: gate/up, 4-way K split");
  constexpr int RG = 4 / KSPLIT;                       // row groups per workgroup
  constexpr int WROWS = (MODE == 0) ? 8 * FR : 16 * FR;  // output columns per wave

  const int lane = threadIdx.x & 63;
  const int wave = BL ? ((threadIdx.x >> 6) & 3) : (threadIdx.x >> 6);
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
      const int tok = DENSE ? row - blk.row_start : P.row_token[row];
      bptr[nb] = P.bsrc + (size_t)tok * P.H + kbeg;
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
      if constexpr (!BL) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          b[u][nb] = *reinterpret_cast<const u32x4*>(bptr[nb] + ks * (KSPLIT * 32));
      }
    }
  };
  auto compute = [&](const u32x4 (&a)[U][FR], const u32x4 (&b)[U][NB], int stage) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (stage * U + u < nsteps) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          u32x4 bv;
          if constexpr (BL) {
            // token r, k = 32 (kp + KSPLIT ks) + 8 g .. +7: 16-byte chunk 4 (kp + KSPLIT ks) + g
            const int chunk = 4 * (kp + KSPLIT * (stage * U + u)) + g;
            bv = *reinterpret_cast<const u32x4*>(xl + r * xpitch + chunk * 16);
          } else {
            bv = b[u][nb];
          }
#pragma unroll
          for (int f = 0; f < FR; ++f) acc[f][nb] = mfma16(a[u][f], bv, acc[f][nb]);
        }
      }
    }
  };

  load(a0, b0, 0);
  if constexpr (BL) fill();
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
          hv[j] = swiglu(gv, uv);
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

// Share (%) of each XCD's work items that go to a common pool, per GEMM, and
// the claimer workgroups per pooled item.  Per-workgroup timestamps at
// decode (T = 16) showed the 8 XCDs streaming the same item count at rates
// up to ~5% apart, so the kernel ended when the slowest XCD did; with the
// pool the faster XCDs take more of the last items.  Measured against a
// plain one-item-per-block grid on one box: gate/up -1.2% with 4%, down
// -0.9% with 2% (4% for down gained nothing: its items are a third as
// long, so each claim's latency weighs more).
template <int MODE>
constexpr int reg_pool_pct() { return MODE == 0 ? 4 : 2; }
constexpr int kRegPoolRoom = 2;

// Work items are (row block, weight tile) pairs, row-block-major; only the
// first n_rb * tiles exist.  XCD-aware deal: block b runs on XCD b % 8; the
// items are cut into 8 contiguous ranges, one per XCD, and the last
// reg_pool_pct() percent of every range form a common pool.  Block j of
// XCD x runs item j of its range while j is below the range's own part;
// the next kRegPoolRoom * (its pool share) blocks of the XCD each claim one
// pooled item with an atomic on the GEMM's pool counter (n_rb[1] for
// gate/up, n_rb[2] for down, zeroed by the dispatch), whichever range it
// comes from; the rest of the grid exits.  Which CU runs an item does not
// change its result.
//
// A row block that is its group's only one is the single reader of its
// weight tile, which then streams with non-temporal loads: they lift the
// HBM read rate (a plain read kernel moves ~6.2 TB/s with ordinary loads and
// ~7.0 TB/s with non-temporal ones).  Tiles that several row blocks read use
// ordinary loads, so the blocks after the first find them in L2.
template <int MODE, int NB, int FR, int KSPLIT, int U>
__global__ __launch_bounds__(256) void expert_gemm_kernel(GemmParams P) {
  __shared__ f32x4 s_red[red_slots<KSPLIT, FR, NB>()];
  __shared__ int s_claim;
  constexpr int kPct = reg_pool_pct<MODE>();
  const long long n_items = (long long)*P.n_rb * P.tiles;
  auto lo = [&](int y) { return (int)((y * n_items) >> 3); };   // first item of XCD y's range
  auto pooled = [&](int y) { return ((lo(y + 1) - lo(y)) * kPct) / 100; };
  auto own = [&](int y) { return lo(y + 1) - lo(y) - pooled(y); };
  const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
  int item;
  if (j < own(x)) {
    item = lo(x) + j;
  } else if (j - own(x) < kRegPoolRoom * pooled(x)) {   // uniform over the workgroup
    int n_pool = 0;
    for (int y = 0; y < 8; ++y) n_pool += pooled(y);
    if (threadIdx.x == 0) s_claim = atomicAdd(const_cast<int32_t*>(P.n_rb) + 1 + MODE, 1);
    __syncthreads();
    int idx = s_claim;
    if (idx >= n_pool) return;   // uniform over the workgroup
    int y = 0;
    while (idx >= pooled(y)) idx -= pooled(y++);
    item = lo(y) + own(y) + idx;
  } else {
    return;
  }
  const int tile = item % P.tiles;
  const int rbi = item / P.tiles;
  const RowBlock blk = P.rb[rbi];
  if (blk.n_group == 1)
    gemm_tile<MODE, NB, FR, KSPLIT, U, true>(P, blk, tile, s_red);
  else
    gemm_tile<MODE, NB, FR, KSPLIT, U, false>(P, blk, tile, s_red);
}

// Gate/up of the dense FFN for a batch of at most 16 tokens.  Slice g of
// the intermediate dimension is group g, and its one row block holds every
// token (row g*T + t is token t), so the row list follows from the block
// index and no dispatch runs before it.  The weight tiles have one reader
// each: non-temporal loads.
__global__ __launch_bounds__(256) void dense_gate_up_kernel(GemmParams P, int T) {
  __shared__ f32x4 s_red[red_slots<4, 2, 1>()];
  const int tile = blockIdx.x % P.tiles;
  const int g = blockIdx.x / P.tiles;
  const RowBlock blk{g, g * T, T, g, 1, g * T, T, 0};
  gemm_tile<0, 1, 2, 4, 4, true, true>(P, blk, tile, s_red);
}

// The same gate/up with x held in LDS, for H <= 4096: three 16-column output
// pairs per workgroup (12 waves, four per pair as above) and one workgroup
// per CU (x takes 128 KB of LDS).  Per-workgroup timestamps of the kernel
// above (704 one-pair workgroups at the Flash shape, all resident at once)
// showed that a CU streams weights at a fixed rate shared by the workgroups
// it holds, which left the CUs with three pairs running long after those
// with two, and that the B operand loads (each instruction 16 token rows x
// 64 bytes, from L2) took part of that rate: a copy without them ran 13%
// faster.  Here each workgroup brings x into LDS once with whole-line loads
// (row r holds token min(r, T-1); rows 2H + 16 bytes apart, so the 16 rows
// of one B read fall on distinct banks) and every CU streams at most three
// pairs.  The last workgroup's spare groups repeat the last pair: the same
// values to the same addresses.
constexpr int kDenseXMaxH = 4096;
constexpr int kDensePairs = 3;

__global__ __launch_bounds__(64 * 4 * kDensePairs) void dense_gate_up_x_kernel(GemmParams P, int T,
                                                                               int n_pairs) {
  __shared__ f32x4 s_red[kDensePairs * red_slots<4, 2, 1>()];
  __shared__ __attribute__((aligned(16))) unsigned char s_x[16 * (2 * kDenseXMaxH + 16)];
  const int grp = threadIdx.x >> 8;   // four waves per pair
  const int q = min((int)blockIdx.x * kDensePairs + grp, n_pairs - 1);
  const int g = q / P.tiles, tile = q % P.tiles;
  const RowBlock blk{g, g * T, T, g, 1, g * T, T, 0};
  const int pitch = 2 * P.H + 16;
  auto fill = [&]() {
    constexpr int kMaxIt = (16 * kDenseXMaxH / 8 + 64 * 4 * kDensePairs - 1) / (64 * 4 * kDensePairs);
    const int cpr = P.H / 8;              // 16-byte chunks per row
    const int total = 16 * cpr;
    u32x4 v[kMaxIt];
#pragma unroll
    for (int i = 0; i < kMaxIt; ++i) {
      const int c = min((int)threadIdx.x + i * 64 * 4 * kDensePairs, total - 1);
      const int r = c / cpr, col = c - r * cpr;
      v[i] = *reinterpret_cast<const u32x4*>(P.bsrc + (size_t)min(r, T - 1) * P.H + col * 8);
    }
#pragma unroll
    for (int i = 0; i < kMaxIt; ++i) {
      const int c = (int)threadIdx.x + i * 64 * 4 * kDensePairs;
      if (c < total) {
        const int r = c / cpr, col = c - r * cpr;
        *reinterpret_cast<u32x4*>(s_x + r * pitch + col * 16) = v[i];
      }
    }
    __syncthreads();
  };
  gemm_tile<0, 1, 2, 4, 4, true, true, true>(P, blk, tile, s_red + grp * red_slots<4, 2, 1>(),
                                             s_x, pitch, fill);
}

// Down projection of the dense FFN for a batch of at most 16 tokens, with
// the sum over the S slices inside the workgroup:
//   y[t, n] = sum_s h_s[t] . Wd_s[n]
// where h_s is slice s of the intermediate activations (rows s*T .. s*T+T-1
// of h, I/S columns) and Wd_s the matching column slice of the down weights
// (packed as S matrices [H, I/S]).  Wave s streams slice s's 16 weight rows
// of the workgroup's output tile front to back (one contiguous kilobyte per
// 32-wide k step, non-temporal: each is read once), with the same two-buffer
// pipeline as the grouped kernel; the S partial sums meet in LDS and wave 0
// adds them in slice order and writes y rounded once to bf16.  No o rows
// and no combine pass.
//
// The B operands (16 tokens of h per 32-wide k step) go through LDS: read
// straight into the MFMA's lane layout, each load instruction would touch
// 16 rows of h for 64 bytes each; instead each wave brings its slice's U
// k steps (16 rows x 32U columns) with loads that cover 4 rows x 256 bytes
// (whole lines) into a private double buffer, and reads its B operands from
// there.  A wave reads only what it wrote, and a wave's LDS accesses run in
// order, so no barrier is needed.  16-byte chunk c of row r sits at chunk
// c ^ r: the B reads of one k step (16 rows, one chunk column each) hit
// distinct banks.
template <int U>
__global__ __launch_bounds__(512) void dense_down_kernel(const uint16_t* __restrict__ wd,
                                                         const uint16_t* __restrict__ h,
                                                         uint16_t* __restrict__ y, int T, int H,
                                                         int Isl) {
  static_assert(U == 4, "one stage of B operands is 16 rows x 256 bytes");
  __shared__ f32x4 s_red[7 * 64];
  __shared__ __attribute__((aligned(16))) u32x4 s_h[8][2][16 * 16];   // [wave][buffer][row x chunk]
  const int lane = threadIdx.x & 63;
  const int sl = threadIdx.x >> 6;                  // slice of this wave
  const int S = blockDim.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int rt = blockIdx.x;                        // 16-row tile of the output
  const int ksteps = Isl / 32;
  const uint16_t* aptr = wd + (size_t)sl * H * Isl + (size_t)rt * ksteps * 512 + lane * 8;
  // h rows of this slice: load i of a stage brings rows 4i .. 4i+3 (lane / 16
  // picks the row, lane % 16 the 16-byte chunk); rows past the batch repeat
  // its last one
  const uint16_t* hrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    hrow[i] = h + ((size_t)sl * T + min(4 * i + (lane >> 4), T - 1)) * Isl;
  u32x4(*hb)[16 * 16] = s_h[sl];
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int nstages = (ksteps + U - 1) / U;
  // past the end of K the loads re-read the last stage (in bounds; unused)
  auto load_a = [&](u32x4 (&a)[U], int stage) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ks = min(stage * U + u, ksteps - 1);
      a[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(aptr + (size_t)ks * 512));
    }
  };
  // the stage's 16 x 256-byte block of h (its columns 128 stage .. +127);
  // in a ragged last stage the chunks past the row's end re-read its last
  // chunk (in bounds; their k steps are skipped)
  auto load_h = [&](u32x4 (&v)[4], int stage) {
    const int col = min(stage * U * 32 + 8 * (lane & 15), Isl - 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = *reinterpret_cast<const u32x4*>(hrow[i] + col);
  };
  auto store_h = [&](int buf, const u32x4 (&v)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * i + (lane >> 4), c = lane & 15;
      hb[buf][row * 16 + (c ^ row)] = v[i];
    }
  };
  auto compute = [&](const u32x4 (&a)[U], int buf, int stage) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (stage * U + u < ksteps) {
        // B operand: token r, k = 32 u + 8 g .. +7 of the stage
        const u32x4 b = hb[buf][r * 16 + ((4 * u + g) ^ r)];
        acc = mfma16(a[u], b, acc);
      }
    }
  };
  u32x4 a0[U], a1[U], v[4];
  load_h(v, 0);
  load_a(a0, 0);
  store_h(0, v);
  int st = 0;
  for (; st + 1 < nstages; ++st) {
    u32x4 (&ac)[U] = (st & 1) ? a1 : a0;
    u32x4 (&an)[U] = (st & 1) ? a0 : a1;
    load_h(v, st + 1);
    load_a(an, st + 1);
    compute(ac, st & 1, st);
    store_h((st + 1) & 1, v);
  }
  compute((st & 1) ? a1 : a0, st & 1, st);
  // slices 1 .. S-1 park their sums; slice 0 adds them in order
  if (sl > 0) s_red[(sl - 1) * 64 + lane] = acc;
  __syncthreads();
  if (sl > 0) return;
  for (int q = 1; q < S; ++q) acc += s_red[(q - 1) * 64 + lane];
  // lane holds output columns 16 rt + 4 g .. +3 of token r
  if (r < T) {
    u32x2 pk;
    pk[0] = pack_bf16x2(acc[0], acc[1]);
    pk[1] = pack_bf16x2(acc[2], acc[3]);
    *reinterpret_cast<u32x2*>(y + (size_t)r * H + 16 * rt + 4 * g) = pk;
  }
}

hipError_t launch_gate_up_dense(const Plan& p, const GateUpArgs& a, hipStream_t s) {
  // p.E = p.K = S slices of I = p.I columns, one 16-row block per slice
  if (p.T < 1 || p.T > 16 || p.nb != 1 || p.ksplit_gu != 4 || p.Is != 0)
    return hipErrorInvalidValue;
  GemmParams gp{};
  gp.wa0 = a.wg;
  gp.wa1 = a.wu;
  gp.bsrc = a.x;
  gp.out = a.h;
  gp.E = p.E; gp.H = p.H; gp.I = p.I; gp.Is = 0; gp.KT = p.KT;
  gp.tiles = p.gu_tiles;
  gp.limit = a.limit;
  const int n_pairs = p.E * p.gu_tiles;
  if (p.H <= kDenseXMaxH)
    hipLaunchKernelGGL(dense_gate_up_x_kernel, dim3((n_pairs + kDensePairs - 1) / kDensePairs),
                       dim3(64 * 4 * kDensePairs), 0, s, gp, p.T, n_pairs);
  else
    hipLaunchKernelGGL(dense_gate_up_kernel, dim3(n_pairs), dim3(256), 0, s, gp, p.T);
  return hipGetLastError();
}

hipError_t launch_dense_down(const Plan& p, const uint16_t* wd, const uint16_t* h, uint16_t* y,
                             hipStream_t s) {
  if (p.T < 1 || p.T > 16 || p.E < 1 || p.E > 8 || p.H % 16 || p.I < 32 || p.I % 32)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(dense_down_kernel<4>, dim3(p.H / 16), dim3(64 * p.E), 0, s, wd, h, y, p.T,
                     p.H, p.I);
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// Launch configurations.  Row blocks of 16 tokens (decode): one 16-row
// fragment pair per wave, four waves split K, so a workgroup streams
// 16 x 2 x H weights and there are many small workgroups to balance.  Row
// blocks of 32 or 64 tokens: waves own different weight rows.  Larger row
// blocks use the LDS-pipelined kernels (expert_gemm_lds.hip).
// grid: 8 XCDs x (the most items one XCD's range can hold, an eighth of the
// row-block bound times the tiles, rounded up, plus its claimers)
template <int MODE>
static unsigned reg_grid(const Plan& p, int tiles) {
  const long long per_xcd = ((long long)p.rb_max * tiles + 7) / 8;
  return (unsigned)(8 * (per_xcd + kRegPoolRoom * (per_xcd * reg_pool_pct<MODE>() / 100 + 1)));
}

// Dynamic LDS requested by the 16-row, 4-way K-split gate/up launch (decode)
// so that at most two of its workgroups share a CU (2 x 56 KB of the 160 KB;
// the kernel itself uses 6 KB): a CU streams at the same rate with two
// resident workgroups as with three, and fewer in flight per CU shorten the
// kernel's tail.  Measured on one box, two runs each: gate/up 330 -> 326.5 us
// at T = 16 (the down kernel, with shorter items, lost 4% the same way and
// keeps its occupancy).
constexpr unsigned kDecodeGateUpLds = 50 * 1024;

template <int MODE>
static hipError_t launch_mode(const Plan& p, const GemmParams& gp, int ksplit, hipStream_t s) {
  if (p.rb_max == 0 || gp.tiles == 0) return hipSuccess;
  const unsigned grid = reg_grid<MODE>(p, gp.tiles);
  switch (p.nb) {
    case 1:
      if (ksplit == 4)
        hipLaunchKernelGGL((expert_gemm_kernel<MODE, 1, 2, 4, 4>), dim3(grid), dim3(256),
                           MODE == 0 ? kDecodeGateUpLds : 0u, s, gp);
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
