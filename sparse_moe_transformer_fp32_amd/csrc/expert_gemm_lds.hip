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
// Down work items cover 512 output rows (when H allows): a row block of at
// most 128 tokens runs them as one tile of two weight fragments per wave
// (512 x 128: twice the weight bytes per item for the same fixed prologue
// and epilogue, which are a quarter of a 256-row down item at that height),
// a taller block as two 256-row passes one after the other.
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
//  - Stage s first writes stage s+1's tokens (loaded in stage s-1) to LDS,
//    then multiplies its four k chunks.  The MFMAs of each chunk carry the
//    instructions the pipeline needs next, one after each MFMA: the LDS
//    reads of the next chunk's B operands, and this stage's global loads
//    for stage s+2 (tokens during chunk 0, two weight loads during chunks 1
//    and 2).  Issued in bursts instead, the loads and reads stalled both
//    waves of a SIMD at the same point of every stage and left the matrix
//    core idle.  Before the last chunk the waves meet at a barrier that
//    publishes stage s+1's tokens, so the first chunk of stage s+1 is read
//    under the last chunk's MFMAs.
//  - The number of 32-token fragments with real rows (NA) is a template
//    argument, so the MFMA stream has no branches, and the waves gather only
//    those fragments' rows (ceil(NA/2) loads per wave per stage).
//  - The epilogue (SwiGLU for gate/up, the routing weight for down) stages
//    the output tile in LDS, in the token ring's memory, and writes whole
//    rows with 16-byte non-temporal stores.
//
// XCD-aware order: block b runs on XCD b % 8.  The routed experts' row
// blocks and the shared expert's are each cut into 8 contiguous ranges, one
// per XCD, whose work items run group by group, weight tile by weight tile,
// row block by row block: the workgroups that run side by side on one XCD
// share weight tiles (across an expert's row blocks, which the dispatch cuts
// to nearly equal heights so that they keep pace) and token rows (across
// weight tiles) through that XCD's L2.
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
  int nrb_shared;        // row blocks of the shared expert (the list's last ones)
  float limit, limit_shared;
  int* pool;             // claim counter of the pooled items (zeroed by the dispatch)
  int wide;              // down: 512-row items (else 256)
};

namespace {

constexpr int kRows = 192;            // token rows per row block at most (the plan's bn)
constexpr int kGran = 32;             // row blocks are cut in 32-row fragments (rb_gran)
constexpr int kWaves = 8;             // waves per workgroup
constexpr int kKC = 4;                // 16-wide k chunks per 64-wide stage
constexpr int kTSlots = 2;            // LDS ring slots

// The shape of one work item: FR 32-row weight fragments per wave (8 x 32 FR
// weight rows per workgroup), at most ROWS tokens, a WS-slot weight register
// ring.  kStage is the bytes of one LDS ring slot: what the waves' token
// loads bring, 8 rows a load and ceil(NA/2) loads a wave.
template <int FR, int ROWS, int WS>
struct TileShape {
  static constexpr int kFR = FR;
  static constexpr int kRows = ROWS;
  static constexpr int kWSlots = WS;
  static constexpr int kMaxNA = ROWS / 32;
  static constexpr int kStage = kWaves * ((kMaxNA * 4 + kWaves - 1) / kWaves) * 8 * 128;
};
// 256 weight rows x up to 192 tokens, one fragment per wave, a 3-slot ring
typedef TileShape<1, 192, 3> TileA;
// 512 weight rows x up to 128 tokens, two fragments per wave: twice the
// weight bytes per item for the same fixed prologue and epilogue; a stage
// is twice as long, so a 2-slot ring keeps as much time in flight (and the
// registers within 256).  Used for the down items of at most 128 rows.
typedef TileShape<2, 128, 2> TileW;
// Share (%) of each XCD's items that go to a common pool, per GEMM.  The
// XCDs get equal shares of the work but do not run at equal speed, so the
// kernel ends when the slowest XCD does; workgroups past their XCD's own
// items claim the pooled ones with one atomic each, and the XCDs that got
// through their own items first take the most.  For gate/up 5% took 1.4-1.8%
// off at T = 4096 to 32768.  Down items of 256 rows were short enough that
// the claim's latency and the lost L2 locality cost more than the balance
// gained; the 512-row items gain a little at T = 8192 and 32768.
template <int MODE>
constexpr int pool_pct() { return 5; }
// claimer slots per XCD, in multiples of its own pool share (each claimer
// that finds the pool empty costs a workgroup launch)
constexpr int kPoolRoom = 3;

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

// Publishes this wave's LDS writes to the workgroup: wait until they are
// done (lgkmcnt(0)), then meet the other waves at the barrier.  The barrier
// builtin is not modelled as touching memory, so the empty asm statements
// with a memory clobber on both sides keep the compiler from moving any
// memory access across it.
__device__ inline void lds_publish() {
  asm volatile("" ::: "memory");
  wait_lds();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS bank swizzle of a token row's 16-byte chunks
__device__ inline int row_swizzle(int R) { return (R >> 1) & 7; }

template <int I>
using ic = std::integral_constant<int, I>;

// f(ic<B>{}), f(ic<B + 1>{}), ..., f(ic<E - 1>{}), unrolled at compile time
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(ic<B>{});
    static_for<B + 1, E>(f);
  }
}

}  // namespace

// The pipelined K loop and the epilogue for one work item whose row block
// has NA 32-token fragments with real rows.
template <int MODE, int NA, bool NT, typename TS>
__device__ __forceinline__ void lds_gemm_item(const LdsGemmParams& P, const RowBlock& blk,
                                              bool shared, int col0, int nst,
                                              unsigned char (*ring)[TS::kStage]) {
  constexpr int kFR = TS::kFR;
  constexpr int kWSlots = TS::kWSlots;
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
  // its last row.  For gate/up the rows' tokens are looked up here, before
  // the first weight loads are issued, so that the lookups and the weights
  // travel together; the token pointers are formed after those loads.
  int trow[kTL], tok[kTL];
#pragma unroll
  for (int i = 0; i < kTL; ++i) {
    const int R = 8 * (wave * kTL + i) + (lane >> 3);
    trow[i] = blk.row_start + min(R, blk.n_rows - 1);
    if (MODE == 0) tok[i] = P.row_token[trow[i]];
  }
  const uint16_t* tsrc[kTL];
  auto token_pointers = [&]() {
#pragma unroll
    for (int i = 0; i < kTL; ++i) {
      const int R = 8 * (wave * kTL + i) + (lane >> 3);
      const int row = trow[i];
      const uint16_t* base;
      if (MODE == 0)
        base = P.bsrc + (size_t)tok[i] * P.H;
      else
        base = shared ? P.bsrc + (size_t)P.KT * P.I + (size_t)(row - P.KT) * P.Is
                      : P.bsrc + (size_t)row * P.I;
      tsrc[i] = base + 8 * ((lane & 7) ^ row_swizzle(R));
    }
  };
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
  // In the K loop, non-temporal weight loads past the end of K read a line
  // of this lane's token row instead (in bounds, in L2 since the last
  // stage's token loads; unused): a re-read of the last weight stage, which
  // streamed past L2, would add an HBM round trip to the end of every item.
  // Ordinary weight loads re-read the last stage, an L2 hit.
  auto load_w1 = [&](u32x4 (&w)[kFR][kKC], int s, int q) {
#pragma unroll
    for (int f = 0; f < kFR; ++f) {
      if constexpr (NT) {
        const u32x4* src = s < nst
            ? reinterpret_cast<const u32x4*>(wsrc[f] + (size_t)s * 1024 + 256 * q)
            : reinterpret_cast<const u32x4*>(tsrc[0] + (nst - 1) * 64);
        w[f][q] = __builtin_nontemporal_load(src);
      } else {
        w[f][q] = *reinterpret_cast<const u32x4*>(wsrc[f] + (size_t)min(s, nst - 1) * 1024 + 256 * q);
      }
    }
  };
  auto load_t1 = [&](u32x4 (&v)[kTL], int s, int i) {
    const int off = min(s, nst - 1) * 64;
    v[i] = *reinterpret_cast<const u32x4*>(tsrc[i] + off);
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
  auto read_t1 = [&](const unsigned char* slot, int q, u32x4 (&t)[NA], int n) {
    t[n] = *reinterpret_cast<const u32x4*>(slot + n * 4096 + roff[q]);
  };
  auto read_t = [&](const unsigned char* slot, int q, u32x4 (&t)[NA]) {
#pragma unroll
    for (int n = 0; n < NA; ++n)
      t[n] = *reinterpret_cast<const u32x4*>(slot + n * 4096 + roff[q]);
  };
  // one k chunk's MFMAs with hook(n) issued right after MFMA n (the
  // scheduler keeps the order), so memory instructions interleave with them
  auto mma_h = [&](const u32x4 (&w)[kFR][kKC], int q, const u32x4 (&t)[NA], auto hook) {
#pragma unroll
    for (int n = 0; n < NA; ++n) {
#pragma unroll
      for (int f = 0; f < kFR; ++f)
        acc[f][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, w[f][q]), __builtin_bit_cast(bf16x8, t[n]), acc[f][n], 0,
            0, 0);
      __builtin_amdgcn_sched_barrier(0);
      hook(n);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  u32x4 w[kWSlots][kFR][kKC];   // weights of stages s .. s + kWSlots - 1
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
    constexpr int jw = decltype(wc)::value;   // s % kWSlots
    constexpr int jt = decltype(tc)::value;   // s % 2
    constexpr int jw2 = (jw + kWSlots - 1) % kWSlots, jt1 = (jt + 1) % kTSlots;
    // stage s+1's tokens were loaded in stage s-1 before its weights: once at
    // most those 4 kFR weight loads are outstanding, they have arrived
    wait_vmcnt<4 * kFR>();
    write_t(ring[jt1], ts[jt1]);
    // each chunk's MFMAs carry the next chunk's LDS reads and this stage's
    // global loads: tokens in chunk 0, two weight loads in chunks 1 and 2
    mma_h(w[jw], 0, t[0], [&](int n) {
      read_t1(ring[jt], 1, t[1], n);
#pragma unroll
      for (int i = 0; i < kTL; ++i)
        if (min(i, NA - 1) == n) load_t1(ts[jt], s + 2, i);
    });
    mma_h(w[jw], 1, t[1], [&](int n) {
      read_t1(ring[jt], 2, t[0], n);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        if (min(i, NA - 1) == n) load_w1(w[jw2], s + kWSlots - 1, i);
    });
    mma_h(w[jw], 2, t[0], [&](int n) {
      read_t1(ring[jt], 3, t[1], n);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        if (min(i, NA - 1) == n) load_w1(w[jw2], s + kWSlots - 1, 2 + i);
    });
    lds_publish();
    __builtin_amdgcn_sched_barrier(0);
    mma_h(w[jw], 3, t[1], [&](int n) { read_t1(ring[jt1], 0, t[0], n); });
    __builtin_amdgcn_sched_barrier(0);
  };

  // prologue: the weights of stages 0 and 1 first (they need no token
  // lookup), then the tokens of stages 0 and 1
#pragma unroll
  for (int k = 0; k + 1 < kWSlots; ++k) load_w(w[k], k);
  __builtin_amdgcn_sched_barrier(0);
  token_pointers();
  load_t(ts[0], 0);
  load_t(ts[1], 1);
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt<kTL>();   // stage 0's tokens have arrived (stage 1's may not)
  write_t(ring[0], ts[0]);
  lds_publish();
  __builtin_amdgcn_sched_barrier(0);
  read_t(ring[0], 0, t[0]);
  wait_vmcnt<0>();     // stage 1's tokens, which stage 0 writes to LDS first
  // the slot pair (s % kWSlots, s % 2) repeats every kPer stages
  constexpr int kPer = (kWSlots % 2) ? 2 * kWSlots : kWSlots;
  int s = 0;
  for (; s + kPer <= nst; s += kPer)
    static_for<0, kPer>([&](auto k) {
      constexpr int K = decltype(k)::value;
      stage(ic<K % kWSlots>{}, ic<K % 2>{}, s + K);
    });
  // tail: the remaining stages continue the same slot sequence
  static_for<0, kPer - 1>([&](auto k) {
    constexpr int K = decltype(k)::value;
    if (s + K < nst) stage(ic<K % kWSlots>{}, ic<K % 2>{}, s + K);
  });
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
          hv[j] = swiglu(gv, uv);
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

// The item's body for its number of 32-token fragments with rows.  Gate/up
// items are 256 weight rows (128 outputs).  Down items are 512 output rows
// when H allows (P.wide): one 512-row pass when the block has at most 128
// rows, else two 256-row passes one after the other; otherwise 256 rows.
template <int MODE, bool NT, typename TS>
__device__ __forceinline__ void lds_gemm_na(const LdsGemmParams& P, const RowBlock& blk, bool shared,
                                            int col0, int nst, unsigned char* lds) {
  auto ring = reinterpret_cast<unsigned char (*)[TS::kStage]>(lds);
  switch ((blk.n_rows + 31) >> 5) {
    case 1: lds_gemm_item<MODE, 1, NT, TS>(P, blk, shared, col0, nst, ring); break;
    case 2: lds_gemm_item<MODE, 2, NT, TS>(P, blk, shared, col0, nst, ring); break;
    case 3: lds_gemm_item<MODE, 3, NT, TS>(P, blk, shared, col0, nst, ring); break;
    case 4: lds_gemm_item<MODE, 4, NT, TS>(P, blk, shared, col0, nst, ring); break;
    case 5:
      if constexpr (TS::kMaxNA >= 5) lds_gemm_item<MODE, 5, NT, TS>(P, blk, shared, col0, nst, ring);
      break;
    default:
      if constexpr (TS::kMaxNA >= 6) lds_gemm_item<MODE, 6, NT, TS>(P, blk, shared, col0, nst, ring);
      break;
  }
}

template <int MODE, bool NT>
__device__ __forceinline__ void lds_gemm_fragments(const LdsGemmParams& P, const RowBlock& blk,
                                                   bool shared, int col0, int nst,
                                                   unsigned char* lds) {
  if constexpr (MODE == 0) {
    lds_gemm_na<MODE, NT, TileA>(P, blk, shared, col0, nst, lds);
  } else if (!P.wide) {
    lds_gemm_na<MODE, NT, TileA>(P, blk, shared, col0, nst, lds);
  } else if (blk.n_rows <= TileW::kRows) {
    lds_gemm_na<MODE, NT, TileW>(P, blk, shared, col0, nst, lds);
  } else {
    lds_gemm_na<MODE, NT, TileA>(P, blk, shared, col0, nst, lds);
    __syncthreads();   // every wave is done with the first pass's staging area
    lds_gemm_na<MODE, NT, TileA>(P, blk, shared, col0 + 256, nst, lds);
  }
}

template <int MODE>
__global__ __launch_bounds__(64 * kWaves) void expert_gemm_lds_kernel(LdsGemmParams P) {
  // the token ring during the K loop, then the output tile of the epilogue
  // (down: the larger of the two item shapes)
  constexpr int kStgA = TileA::kRows * (((MODE == 0) ? 16 : 32) * kWaves * 2 + 16);
  constexpr int kStgW = MODE == 1 ? TileW::kRows * (2 * 32 * kWaves * 2 + 16) : 0;
  constexpr int kStg = kStgA > kStgW ? kStgA : kStgW;
  constexpr int kLds = kStg > kTSlots * TileA::kStage ? kStg : kTSlots * TileA::kStage;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[kLds];

  // XCD-aware deal of work items.  Block b runs on XCD b % 8.  The routed
  // experts' row blocks (a prefix of the list, ordered by group) are cut into
  // 8 contiguous ranges of equal length, and so are the shared expert's; XCD
  // x takes routed range x, then shared range x.  Inside a range the items
  // run group by group, weight tile by weight tile, row block by row block,
  // so the workgroups that run side by side on one XCD share an expert's
  // weight tile (across its row blocks) and its token rows (across weight
  // tiles) through that XCD's L2, and every XCD gets an eighth of the work.
  // The last pool_pct() percent of each XCD's items are claimed from a
  // common pool by the workgroups past their XCD's own items (the grid has
  // room for an XCD to claim three times its share; the claim counter is zeroed
  // by the dispatch).  Which CU runs an item does not change its result.
  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  const int nrb = *P.n_rb;
  const int n_routed = nrb - P.nrb_shared;
  // items of XCD x, and how many of its last ones go to the shared pool
  auto count = [&](int x) {
    return ((((x + 1) * n_routed) >> 3) - ((x * n_routed) >> 3) +
            (((x + 1) * P.nrb_shared) >> 3) - ((x * P.nrb_shared) >> 3)) * P.tiles;
  };
  constexpr int kPoolPct = pool_pct<MODE>();
  auto pooled = [&](int x) { return (count(x) * kPoolPct) / 100; };
  int x = xcd, j = slot;
  if (slot >= count(xcd) - pooled(xcd)) {
    // past this XCD's own items: claim the next pooled item, whichever
    // XCD's range it comes from (workgroups of the XCDs that got through
    // their own items first take the most)
    if (kPoolPct == 0) return;
    int n_pool = 0;
    for (int y = 0; y < 8; ++y) n_pool += pooled(y);
    __shared__ int s_claim;
    if (threadIdx.x == 0) s_claim = atomicAdd(P.pool, 1);
    __syncthreads();
    int idx = s_claim;
    if (idx >= n_pool) return;   // uniform over the workgroup
    x = 0;
    while (idx >= pooled(x)) idx -= pooled(x++);
    j = count(x) - pooled(x) + idx;
  }
  {
    int lo = (x * n_routed) >> 3, hi = ((x + 1) * n_routed) >> 3;
    int jj = j;
    bool valid = true;
    if (jj >= (hi - lo) * P.tiles) {   // past the routed range: the shared range
      jj -= (hi - lo) * P.tiles;
      lo = n_routed + ((x * P.nrb_shared) >> 3);
      hi = n_routed + (((x + 1) * P.nrb_shared) >> 3);
      valid = jj < (hi - lo) * P.tiles;
    }
    if (valid) {
      // the group segment (the part of one group inside [lo, hi)) that holds
      // item jj: its items fill [(seg0 - lo) * tiles, (seg1 - lo) * tiles)
      const RowBlock any = P.rb[lo + jj / P.tiles];
      const int seg0 = max(lo, any.first);
      const int seg1 = min(hi, any.first + any.n_group);
      const int local = jj - (seg0 - lo) * P.tiles;
      const int tile = local / (seg1 - seg0);
      const int rbi = seg0 + local % (seg1 - seg0);
      // the block itself follows from its group's rows (no second list load)
      RowBlock blk = any;
      {
        int st, n;
        split_block(any.group_rows, any.n_group, kGran, rbi - any.first, &st, &n);
        blk.row_start = any.group_row0 + st;
        blk.n_rows = n;
      }
      const bool shared = blk.group == P.E;
      const int inter = shared ? P.Is : P.I;
      const int nout = (MODE == 0) ? inter : P.H;
      const int col0 = tile * (MODE == 0 ? 128 : P.wide ? 512 : 256);  // first output column
      const int nst = ((MODE == 0) ? P.H : inter) >> 6;  // 64-wide k stages
      // A row block that is its group's only one is the single reader of its
      // weight tile, which then streams with non-temporal loads (a higher
      // HBM read rate); tiles that several row blocks read use ordinary
      // loads, so the blocks after the first find them in L2.
      if (col0 < nout) {                                 // uniform over the workgroup
        if (blk.n_group == 1)
          lds_gemm_fragments<MODE, true>(P, blk, shared, col0, nst, lds);
        else
          lds_gemm_fragments<MODE, false>(P, blk, shared, col0, nst, lds);
      }
    }
  }
}

// grid: 8 XCDs x the most items one XCD can receive (an eighth of the
// row-block bound, rounded up, for the routed and for the shared experts)
static unsigned lds_grid(const Plan& p, int tiles, int pct) {
  const long long nrb_s = p.Is > 0 ? (p.T + p.bn - 1) / p.bn : 0;
  const long long routed = p.rb_max - nrb_s;
  const long long per_xcd = ((routed + 7) / 8 + (nrb_s + 7) / 8) * tiles;
  // room for every XCD to claim kPoolRoom times its own share of the pool
  return (unsigned)(8 * (per_xcd + kPoolRoom * (per_xcd * pct / 100)));
}

hipError_t launch_gate_up_lds(const Plan& p, const GateUpArgs& a, hipStream_t s) {
  if (p.bn != kRows || p.rb_gran != kGran || p.H % 64 || p.I % 128 || p.Is % 128)
    return hipErrorInvalidValue;
  LdsGemmParams gp{};
  gp.wa0 = a.wg; gp.wa1 = a.wu; gp.sa0 = a.sg; gp.sa1 = a.su; gp.bsrc = a.x;
  gp.row_token = a.row_token; gp.rb = a.rb; gp.n_rb = a.n_rb; gp.out = a.h;
  gp.E = p.E; gp.H = p.H; gp.I = p.I; gp.Is = p.Is; gp.KT = p.KT; gp.tiles = p.gu_tiles;
  gp.nrb_shared = p.Is > 0 ? (p.T + p.bn - 1) / p.bn : 0;
  gp.limit = a.limit; gp.limit_shared = a.limit_shared;
  gp.pool = const_cast<int32_t*>(a.n_rb) + 1;
  hipLaunchKernelGGL(expert_gemm_lds_kernel<0>, dim3(lds_grid(p, p.gu_tiles, pool_pct<0>())), dim3(64 * kWaves), 0, s,
                     gp);
  return hipGetLastError();
}

hipError_t launch_down_lds(const Plan& p, const DownArgs& a, hipStream_t s) {
  if (p.bn != kRows || p.rb_gran != kGran || p.I % 128 || p.Is % 128 ||
      (p.dn_rows_wg != 256 && p.dn_rows_wg != 512) || p.H % p.dn_rows_wg)
    return hipErrorInvalidValue;
  LdsGemmParams gp{};
  gp.wa0 = a.wd; gp.sa0 = a.sd; gp.bsrc = a.h; gp.row_w = a.row_w;
  gp.rb = a.rb; gp.n_rb = a.n_rb; gp.out = a.o;
  gp.E = p.E; gp.H = p.H; gp.I = p.I; gp.Is = p.Is; gp.KT = p.KT; gp.tiles = p.dn_tiles;
  gp.nrb_shared = p.Is > 0 ? (p.T + p.bn - 1) / p.bn : 0;
  gp.pool = const_cast<int32_t*>(a.n_rb) + 2;
  gp.wide = p.dn_rows_wg == 512;
  hipLaunchKernelGGL(expert_gemm_lds_kernel<1>, dim3(lds_grid(p, p.dn_tiles, pool_pct<1>())), dim3(64 * kWaves), 0, s,
                     gp);
  return hipGetLastError();
}

}  // namespace smoe
