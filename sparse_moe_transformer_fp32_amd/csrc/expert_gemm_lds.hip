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
// Matrix cores: v_mfma_f32_32x32x16_bf16.  Lane l holds A row l%32 and B
// column l%32, k = 8(l/32)..+7 of a 16-wide k chunk; accumulator register j
// holds row 8(j/4) + 4(l/32) + j%4 of column l%32.
//
// Workgroup tile: 256 weight rows x one row block of up to 192 tokens.  Each
// of the 8 waves (two per SIMD) owns one 32-row weight fragment and
// multiplies it with every 32-token fragment of the block (6 accumulator
// tiles, 96 registers), so each weight element is read from memory once per
// row block, and while one wave of a SIMD waits for memory the other can
// issue MFMAs.  For gate/up a
// weight fragment is 16 gate rows over 16 up rows of the same intermediate
// columns, so accumulator registers j and j+8 of a lane are the gate and up
// values of one output and SwiGLU happens in registers.
//
// Pipeline, one 64-wide k stage per step:
//  - Tokens (shared by the 8 waves) are gathered with full-line loads: one
//    load instruction moves 8 rows x 128 bytes (8 lanes per row) into
//    registers, and one stage later the wave writes them to a 2-slot LDS
//    ring, lane l's 16 bytes at row-group base + 16 l.  The global side
//    fetches chunk (l%8) ^ s(row) of its row, s(row) = (row/2) % 8: the
//    swizzle spreads the rows of every 8-lane read group over distinct LDS
//    banks, and ds_read_b128 of a B operand is conflict-free.  (Loads that
//    write LDS directly are not used: their completion is not ordered with
//    the register loads of the same wave, so a vmcnt count cannot tell
//    when their data has landed.)
//  - Weights are used by one wave only and skip LDS: packed tiles go straight
//    into a 3-slot register ring.  One 64-wide stage of a packed 16-row tile
//    is 1024 contiguous elements.  When the row block is its group's only
//    one, the workgroup is its weight tile's single reader and the loads are
//    non-temporal (a higher HBM read rate); otherwise they are ordinary, so
//    the sibling blocks find the tile in L2.
//  - Stage s issues the weights and the tokens of stage s+2, multiplies its
//    four k chunks
//    (the LDS reads of chunk q+1 in flight under the MFMAs of chunk q), and
//    before its last chunk stores stage s+1's tokens to LDS and meets the
//    other waves at a barrier, so the first chunk of stage s+1 is read under
//    that last chunk's MFMAs.
//  - The number of 32-token fragments with real rows (NA) is a template
//    argument, so the MFMA stream has no branches, and the waves gather only
//    those fragments' rows (ceil(NA/2) loads per wave per stage).
//  - The epilogue (SwiGLU for gate/up, the routing weight for down) stages
//    the output tile in LDS, in the token ring's memory, and writes whole
//    rows with 16-byte non-temporal stores.
//
// XCD-aware order: block b runs on XCD b % 8.  Work items, ordered (group,
// weight tile, row block), are dealt to the XCDs in chunks of 32 in turn.
// Workgroups that run side by side on one XCD then share weight tiles
// (across an expert's row blocks, which the dispatch cuts to nearly equal
// heights so that they keep pace) and token rows (across weight tiles)
// through that XCD's L2, and no XCD is left with all of a heavy group.
#include <type_traits>

#include "smoe_internal.h"

namespace smoe {

typedef float f32x16 __attribute__((ext_vector_type(16)));

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

namespace {

constexpr int kRows = 192;            // token rows per row block at most (the plan's bn)
constexpr int kFR = 1;                // 32-row weight fragments per wave
constexpr int kWaves = 8;             // waves per workgroup: 8 x 32 = 256 weight rows
constexpr int kKC = 4;                // 16-wide k chunks per 64-wide stage
constexpr int kStage = kRows * 128;   // token bytes per stage
constexpr int kWSlots = 3;            // weight register ring slots
constexpr int kTSlots = 2;            // LDS ring slots
constexpr int kChunk = 32;            // consecutive work items per XCD turn

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

// s_waitcnt lgkmcnt(0): every LDS access of this wave is done.
__device__ inline void wait_lds() {
  __builtin_amdgcn_s_waitcnt((0xF) | (0x7 << 4) | (0x0 << 8) | (3 << 14));
}

// LDS bank swizzle of a token row's 16-byte chunks
__device__ inline int row_swizzle(int R) { return (R >> 1) & 7; }

template <int I>
using ic = std::integral_constant<int, I>;

}  // namespace

// The pipelined K loop and the epilogue for one work item whose row block
// has NA 32-token fragments with real rows.
template <int MODE, int NA, bool NT>
__device__ __forceinline__ void lds_gemm_item(const LdsGemmParams& P, const RowBlock& blk,
                                              bool shared, int col0, int nst,
                                              unsigned char (*ring)[kStage]) {
  // token loads per wave per stage (8 rows each): the 8 waves bring the
  // 32 NA rows of the fragments in use (for odd NA the last loads repeat the
  // block's last row into LDS rows no fragment reads)
  constexpr int kTL = (NA * 4 + kWaves - 1) / kWaves;
  constexpr int kLoads = kFR * kKC + kTL;   // vector-memory ops per wave per stage
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l31 = lane & 31, hi = lane >> 5;
  const int ktiles = 2 * nst;   // packed 32-wide tiles along K

  // weights: this lane's row of each 32-row fragment, in the packed 16x32
  // tiles (element (r, 8g..8g+7) of a tile at 8 (16 g + r)); chunk q of
  // stage s sits at +1024 s + 256 q from the base below
  const uint16_t* wsrc[kFR];
  if (MODE == 0) {
    const uint16_t* Wg = shared ? P.sa0 : P.wa0 + (size_t)blk.group * P.I * P.H;
    const uint16_t* Wu = shared ? P.sa1 : P.wa1 + (size_t)blk.group * P.I * P.H;
    const uint16_t* M = (l31 < 16) ? Wg : Wu;   // fragment rows 0-15 gate, 16-31 up
#pragma unroll
    for (int f = 0; f < kFR; ++f) {
      const int rt = (col0 >> 4) + wave * kFR + f;
      wsrc[f] = M + (size_t)rt * ktiles * 512 + 8 * (lane & 15) + 128 * hi;
    }
  } else {
    const uint16_t* Wd = shared ? P.sa0 : P.wa0 + (size_t)blk.group * P.H * P.I;
#pragma unroll
    for (int f = 0; f < kFR; ++f) {
      const int rt = (col0 >> 4) + wave * 2 * kFR + 2 * f + (l31 >> 4);
      wsrc[f] = Wd + (size_t)rt * ktiles * 512 + 8 * (lane & 15) + 128 * hi;
    }
  }
  // tokens: load i of this wave brings rows 8 g .. 8 g + 7 (g = wave*kTL + i),
  // 8 lanes per row; rows past the block (inside its last fragment) repeat
  // its last row
  const uint16_t* tsrc[kTL];
#pragma unroll
  for (int i = 0; i < kTL; ++i) {
    const int R = 8 * (wave * kTL + i) + (lane >> 3);
    const int row = blk.row_start + min(R, blk.n_rows - 1);
    const uint16_t* base;
    if (MODE == 0)
      base = P.bsrc + (size_t)P.row_token[row] * P.H;
    else
      base = shared ? P.bsrc + (size_t)P.KT * P.I + (size_t)(row - P.KT) * P.Is
                    : P.bsrc + (size_t)row * P.I;
    tsrc[i] = base + 8 * ((lane & 7) ^ row_swizzle(R));
  }
  // B operand of fragment n, chunk q: row R = 32 n + l31, 16-byte chunk
  // 2 q + hi of that row, at (R/8)*1024 + (R%8)*128 + (chunk ^ s(R))*16
  int roff[kKC];
#pragma unroll
  for (int q = 0; q < kKC; ++q)
    roff[q] = (l31 >> 3) * 1024 + (lane & 7) * 128 + (((2 * q + hi) ^ ((l31 >> 1) & 7)) << 4);

  f32x16 acc[kFR][NA];
#pragma unroll
  for (int f = 0; f < kFR; ++f)
#pragma unroll
    for (int n = 0; n < NA; ++n)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[f][n][j] = 0.f;

  // past the end of K every load re-reads the last stage (in bounds; unused)
  auto load_w = [&](u32x4 (&w)[kFR][kKC], int s) {
    const size_t off = (size_t)min(s, nst - 1) * 1024;
#pragma unroll
    for (int f = 0; f < kFR; ++f)
#pragma unroll
      for (int q = 0; q < kKC; ++q)
        w[f][q] = NT ? __builtin_nontemporal_load(
                           reinterpret_cast<const u32x4*>(wsrc[f] + off + 256 * q))
                     : *reinterpret_cast<const u32x4*>(wsrc[f] + off + 256 * q);
  };
  auto load_t = [&](u32x4 (&v)[kTL], int s) {
    const int off = min(s, nst - 1) * 64;
#pragma unroll
    for (int i = 0; i < kTL; ++i) v[i] = *reinterpret_cast<const u32x4*>(tsrc[i] + off);
  };
  auto write_t = [&](unsigned char* slot, const u32x4 (&v)[kTL]) {
#pragma unroll
    for (int i = 0; i < kTL; ++i)
      *reinterpret_cast<u32x4*>(slot + (wave * kTL + i) * 1024 + lane * 16) = v[i];
  };
  auto read_t = [&](const unsigned char* slot, int q, u32x4 (&t)[NA]) {
#pragma unroll
    for (int n = 0; n < NA; ++n)
      t[n] = *reinterpret_cast<const u32x4*>(slot + n * 4096 + roff[q]);
  };
  auto mma = [&](const u32x4 (&w)[kFR][kKC], int q, const u32x4 (&t)[NA]) {
#pragma unroll
    for (int n = 0; n < NA; ++n)
#pragma unroll
      for (int f = 0; f < kFR; ++f)
        acc[f][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, w[f][q]), __builtin_bit_cast(bf16x8, t[n]), acc[f][n], 0,
            0, 0);
  };

  u32x4 w[kWSlots][kFR][kKC];   // weights of stages s, s+1, s+2
  u32x4 ts[2][kTL];              // tokens of stages s+1, s+2 on their way to LDS
  u32x4 t[2][NA];                // B operands of the current and the next k chunk
  // Stage s (weight slot s%3, token staging buffer and LDS slot s%2) first
  // issues the weights and the tokens of stage s+2.  Stage s+1's tokens were
  // loaded one stage ago; all loads go to registers and complete in order,
  // so vmcnt(kLoads) leaves only this stage's loads in flight and they have
  // arrived.  They go to LDS slot (s+1)%2, last read in stage s-1 (every
  // wave finished those reads before the barrier of stage s-1, which all
  // waves have passed).  The barrier after lgkmcnt(0) publishes them for the
  // first chunk of s+1.
  auto stage = [&](auto wc, auto tc, int s) {
    constexpr int jw = decltype(wc)::value;   // s % 3
    constexpr int jt = decltype(tc)::value;   // s % 2
    constexpr int jw2 = (jw + 2) % kWSlots, jt1 = (jt + 1) % kTSlots;
    load_w(w[jw2], s + 2);
    load_t(ts[jt], s + 2);
    __builtin_amdgcn_sched_barrier(0);
    read_t(ring[jt], 1, t[1]);
    __builtin_amdgcn_sched_barrier(0);
    mma(w[jw], 0, t[0]);
    __builtin_amdgcn_sched_barrier(0);
    read_t(ring[jt], 2, t[0]);
    __builtin_amdgcn_sched_barrier(0);
    mma(w[jw], 1, t[1]);
    __builtin_amdgcn_sched_barrier(0);
    read_t(ring[jt], 3, t[1]);
    __builtin_amdgcn_sched_barrier(0);
    mma(w[jw], 2, t[0]);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<kLoads>();
    write_t(ring[jt1], ts[jt1]);
    wait_lds();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read_t(ring[jt1], 0, t[0]);
    __builtin_amdgcn_sched_barrier(0);
    mma(w[jw], 3, t[1]);
    __builtin_amdgcn_sched_barrier(0);
  };

  // prologue in the same issue pattern: (W0, T0) and (W1, T1) as stages -2
  // and -1 would issue them
  load_w(w[0], 0);
  load_t(ts[0], 0);
  load_w(w[1], 1);
  load_t(ts[1], 1);
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt<kLoads>();   // stage 0's tokens have arrived
  write_t(ring[0], ts[0]);
  wait_lds();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  read_t(ring[0], 0, t[0]);
  int s = 0;
  for (; s + 6 <= nst; s += 6) {
    stage(ic<0>{}, ic<0>{}, s);
    stage(ic<1>{}, ic<1>{}, s + 1);
    stage(ic<2>{}, ic<0>{}, s + 2);
    stage(ic<0>{}, ic<1>{}, s + 3);
    stage(ic<1>{}, ic<0>{}, s + 4);
    stage(ic<2>{}, ic<1>{}, s + 5);
  }
  // tail: the remaining stages continue the same slot sequence
  if (s < nst) stage(ic<0>{}, ic<0>{}, s);
  if (s + 1 < nst) stage(ic<1>{}, ic<1>{}, s + 1);
  if (s + 2 < nst) stage(ic<2>{}, ic<0>{}, s + 2);
  if (s + 3 < nst) stage(ic<0>{}, ic<1>{}, s + 3);
  if (s + 4 < nst) stage(ic<1>{}, ic<0>{}, s + 4);
  wait_vmcnt<0>();

  // epilogue: accumulator register j of a lane is weight row
  // 8(j/4) + 4 hi + j%4 of the fragment, token row 32 n + l31.  The tile's
  // bf16 outputs go to LDS as [token][output column] rows (pitch padded by
  // 16 bytes against bank conflicts); then every thread stores 16-byte
  // chunks of whole rows, so a wave writes full cache lines instead of
  // 16-byte pieces of 32 rows.  The stores are non-temporal: h and o are
  // read once, by the next kernel, and need not displace weights and token
  // rows from L2.
  constexpr int kOut = ((MODE == 0) ? 16 : 32) * kFR * kWaves;   // output columns of the tile
  constexpr int kPitch = kOut * 2 + 16;                     // bytes per staged row
  constexpr int kCPR = kOut / 8;                            // 16-byte chunks per row
  unsigned char* stg = &ring[0][0];
  __syncthreads();   // every wave is done with the ring
#pragma unroll
  for (int n = 0; n < NA; ++n) {
    const int R = 32 * n + l31;
    unsigned char* srow = stg + R * kPitch;
    if (MODE == 0) {
      const float lim = shared ? P.limit_shared : P.limit;
#pragma unroll
      for (int f = 0; f < kFR; ++f) {
        const int lc = wave * 16 * kFR + 16 * f;   // tile column of fragment f
        float hv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float gv = acc[f][n][j];
          float uv = acc[f][n][j + 8];
          if (lim > 0.f) {
            gv = fminf(gv, lim);
            uv = fminf(fmaxf(uv, -lim), lim);
          }
          hv[j] = gv / (1.0f + __expf(-gv)) * uv;
        }
        u32x2 p0, p1;
        p0[0] = pack_bf16x2_l(hv[0], hv[1]);
        p0[1] = pack_bf16x2_l(hv[2], hv[3]);
        p1[0] = pack_bf16x2_l(hv[4], hv[5]);
        p1[1] = pack_bf16x2_l(hv[6], hv[7]);
        *reinterpret_cast<u32x2*>(srow + 2 * (lc + 4 * hi)) = p0;
        *reinterpret_cast<u32x2*>(srow + 2 * (lc + 8 + 4 * hi)) = p1;
      }
    } else {
      const float wr = R < blk.n_rows ? P.row_w[blk.row_start + R] : 0.f;
#pragma unroll
      for (int f = 0; f < kFR; ++f) {
        const int lr = wave * 32 * kFR + 32 * f;   // tile column (output row) of fragment f
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          u32x2 pk;
          pk[0] = pack_bf16x2_l(acc[f][n][4 * jj] * wr, acc[f][n][4 * jj + 1] * wr);
          pk[1] = pack_bf16x2_l(acc[f][n][4 * jj + 2] * wr, acc[f][n][4 * jj + 3] * wr);
          *reinterpret_cast<u32x2*>(srow + 2 * (lr + 8 * jj + 4 * hi)) = pk;
        }
      }
    }
  }
  __syncthreads();
  // rows past the block's end stay in LDS
  const int n_chunks = blk.n_rows * kCPR;
  for (int q = threadIdx.x; q < n_chunks; q += 64 * kWaves) {
    const int R = q / kCPR, c = q % kCPR;
    const u32x4 v = *reinterpret_cast<const u32x4*>(stg + R * kPitch + 16 * c);
    const int row = blk.row_start + R;
    uint16_t* dst;
    if (MODE == 0)
      dst = (shared ? P.out + (size_t)P.KT * P.I + (size_t)(row - P.KT) * P.Is
                    : P.out + (size_t)row * P.I) + col0 + 8 * c;
    else
      dst = P.out + (size_t)row * P.H + col0 + 8 * c;
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst));
  }
}

// the item's body for its number of 32-token fragments with rows
template <int MODE, bool NT>
__device__ __forceinline__ void lds_gemm_fragments(const LdsGemmParams& P, const RowBlock& blk,
                                                   bool shared, int col0, int nst,
                                                   unsigned char (*ring)[kStage]) {
  switch ((blk.n_rows + 31) >> 5) {
    case 1: lds_gemm_item<MODE, 1, NT>(P, blk, shared, col0, nst, ring); break;
    case 2: lds_gemm_item<MODE, 2, NT>(P, blk, shared, col0, nst, ring); break;
    case 3: lds_gemm_item<MODE, 3, NT>(P, blk, shared, col0, nst, ring); break;
    case 4: lds_gemm_item<MODE, 4, NT>(P, blk, shared, col0, nst, ring); break;
    case 5: lds_gemm_item<MODE, 5, NT>(P, blk, shared, col0, nst, ring); break;
    default: lds_gemm_item<MODE, 6, NT>(P, blk, shared, col0, nst, ring); break;
  }
}

template <int MODE>
__global__ __launch_bounds__(64 * kWaves) void expert_gemm_lds_kernel(LdsGemmParams P) {
  // the token ring during the K loop, then the output tile of the epilogue
  constexpr int kStg = kRows * (((MODE == 0) ? 16 : 32) * kFR * kWaves * 2 + 16);
  constexpr int kLds = kStg > kTSlots * kStage ? kStg : kTSlots * kStage;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[kLds];
  auto ring = reinterpret_cast<unsigned char (*)[kStage]>(lds);

  // XCD-aware deal of work items, ordered (group, weight tile, row block):
  // the items are cut in chunks of kChunk, dealt to the 8 XCDs in turn, so
  // the row blocks that share a weight tile and the tiles that share a row
  // block run side by side on one XCD and meet in its L2, while the work of
  // heavy groups (the shared expert, hot experts) spreads over all XCDs
  const int n_items = *P.n_rb * P.tiles;
  const int slot_b = blockIdx.x >> 3;   // this XCD's slot_b-th workgroup
  const int item = ((slot_b / kChunk) * 8 + (blockIdx.x & 7)) * kChunk + slot_b % kChunk;
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
  const int nst = ((MODE == 0) ? P.H : inter) >> 6;  // 64-wide k stages
  // A row block that is its group's only one is the single reader of its
  // weight tile, which then streams with non-temporal loads (a higher HBM
  // read rate); tiles that several row blocks read use ordinary loads, so
  // the blocks after the first find them in L2.
  if (blk.n_group == 1)
    lds_gemm_fragments<MODE, true>(P, blk, shared, col0, nst, ring);
  else
    lds_gemm_fragments<MODE, false>(P, blk, shared, col0, nst, ring);
}

// grid: every chunk of kChunk (row block, weight tile) items up to the
// row-block bound gets kChunk workgroups on its XCD; 8 XCDs per turn
static unsigned lds_grid(const Plan& p, int tiles) {
  const long long items = (long long)p.rb_max * tiles;
  const long long turns = ((items + kChunk - 1) / kChunk + 7) / 8;
  return (unsigned)(turns * 8 * kChunk);
}

hipError_t launch_gate_up_lds(const Plan& p, const GateUpArgs& a, hipStream_t s) {
  if (p.bn != kRows || p.H % 64 || p.I % 128 || p.Is % 128) return hipErrorInvalidValue;
  LdsGemmParams gp{};
  gp.wa0 = a.wg; gp.wa1 = a.wu; gp.sa0 = a.sg; gp.sa1 = a.su; gp.bsrc = a.x;
  gp.row_token = a.row_token; gp.rb = a.rb; gp.n_rb = a.n_rb; gp.out = a.h;
  gp.E = p.E; gp.H = p.H; gp.I = p.I; gp.Is = p.Is; gp.KT = p.KT; gp.tiles = p.gu_tiles;
  gp.limit = a.limit; gp.limit_shared = a.limit_shared;
  hipLaunchKernelGGL(expert_gemm_lds_kernel<0>, dim3(lds_grid(p, p.gu_tiles)), dim3(64 * kWaves), 0, s,
                     gp);
  return hipGetLastError();
}

hipError_t launch_down_lds(const Plan& p, const DownArgs& a, hipStream_t s) {
  if (p.bn != kRows || p.H % 256 || p.I % 128 || p.Is % 128) return hipErrorInvalidValue;
  LdsGemmParams gp{};
  gp.wa0 = a.wd; gp.sa0 = a.sd; gp.bsrc = a.h; gp.row_w = a.row_w;
  gp.rb = a.rb; gp.n_rb = a.n_rb; gp.out = a.o;
  gp.E = p.E; gp.H = p.H; gp.I = p.I; gp.Is = p.Is; gp.KT = p.KT; gp.tiles = p.dn_tiles;
  hipLaunchKernelGGL(expert_gemm_lds_kernel<1>, dim3(lds_grid(p, p.dn_tiles)), dim3(64 * kWaves), 0, s,
                     gp);
  return hipGetLastError();
}

}  // namespace smoe
