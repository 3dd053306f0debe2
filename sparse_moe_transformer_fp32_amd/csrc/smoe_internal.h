// Internal declarations shared by the gfx950 kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace smoe {

// ---------------------------------------------------------------- device types
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// One row block of the grouped GEMMs: `n_rows` consecutive rows (in the
// expert-contiguous row order) that belong to `group` (an expert id, or E for
// the shared expert), starting at global row `row_start`.  The blocks of one
// group are consecutive in the list: `first` is the index of the group's
// first block and `n_group` the number of its blocks; the group's rows are
// `group_rows` rows from global row `group_row0`, cut by split_block, so any
// block of a group gives every other block of it.
struct RowBlock {
  int32_t group;
  int32_t row_start;
  int32_t n_rows;
  int32_t first;
  int32_t n_group;
  int32_t group_row0;
  int32_t group_rows;
  int32_t pad;
};

// Block i of the n_blk = ceil(cnt / bn) row blocks of a group with cnt rows.
// The rows are cut in whole granules of g rows (g divides bn), and the
// blocks' granule counts differ by at most one, so every block holds at most
// bn rows, at least one, and the last one takes the ragged end.  Blocks of
// one group then have (nearly) the same height: the workgroups that stream
// the same weight tile for them run at the same pace.
__device__ inline void split_block(int cnt, int n_blk, int g, int i, int* start, int* n) {
  const int F = (cnt + g - 1) / g;
  const int q = F / n_blk, r = F % n_blk;
  const int st = g * (i * q + min(i, r));
  *start = st;
  *n = min(g * (q + (i < r ? 1 : 0)), cnt - st);
}

// SwiGLU of one output, silu(g) * u with silu(g) = g / (1 + e^-g) (SiLU on
// the gate, times the up projection).  The reciprocal is the hardware's one
// instruction v_rcp_f32 (about 1 ulp), not a correctly rounded division (a
// sequence of about ten): h is rounded to bf16 right after, which is 2^16
// times coarser.  For g below about -88, e^-g overflows to infinity and the
// result is a signed zero, as with the division.
__device__ inline float swiglu(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// ---------------------------------------------------------------- tiling plan
// Every size the launches use is a pure function of the layer sizes, so the
// workspace size, the dispatch kernel and the GEMM launches agree.
struct Plan {
  int32_t T, H, E, K, I, Is;
  int32_t KT;            // T*K routed rows
  int32_t rows_total;    // KT + (Is > 0 ? T : 0)
  int32_t route_tok;     // tokens per router tile (16 or 64; 256: the wide kernel)
  int32_t route_splits;  // split of H across router workgroups
  int32_t dispatch_blocks;  // > 0: three-kernel dispatch over this many 256-token blocks
  int32_t nb;            // 16-token column blocks per GEMM tile (1, 2, 4; 12 = LDS kernels)
  int32_t bn;            // rows per row block at most = 16 * nb
  int32_t rb_gran;       // row blocks are cut in whole granules of this many rows
  int32_t rb_max;        // upper bound on row blocks
  int32_t ksplit_gu;     // waves splitting K in the gate/up GEMM
  int32_t ksplit_dn;     // waves splitting K in the down GEMM
  int32_t gu_rows_wg;    // intermediate rows per gate/up workgroup
  int32_t dn_rows_wg;    // hidden rows per down workgroup
  int32_t gu_tiles;      // workgroups per row block (gate/up)
  int32_t dn_tiles;      // workgroups per row block (down)
  // workspace byte offsets
  size_t ws_partial, ws_topk_idx, ws_topk_w, ws_counts, ws_offsets, ws_perm,
      ws_slot, ws_row_token, ws_row_w, ws_rb, ws_nrb, ws_lrank, ws_hist, ws_bbase, ws_h, ws_o,
      ws_total;
};

void make_plan(int T, int H, int E, int K, int I, int Is, Plan* p);

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.
hipError_t launch_route_logits(const Plan& p, const uint16_t* x, const float* W,
                               float* partial, hipStream_t s);
hipError_t launch_route_topk(const Plan& p, const float* partial, const float* bias,
                             float scale, int norm, int bias_in_weights, int32_t* topk_idx,
                             float* topk_w, float* keys, float* scores, hipStream_t s);
// Everything the dispatch launch touches: it reads topk_idx/topk_w.
struct RouteLaunch {
  const int32_t* topk_idx;
  const float* topk_w;
  int32_t *counts, *offsets, *perm, *slot, *row_token;
  float* row_w;
  RowBlock* rb;
  int32_t* n_rb;
  int32_t *lrank, *hist, *block_base;   // three-kernel dispatch scratch
};
size_t dispatch_lds_bytes(int E);
hipError_t launch_dispatch(const Plan& p, const RouteLaunch& r, hipStream_t s);
// dense FFN cut into p.E = p.K slices: identity row list, weight 1
hipError_t launch_dense_rows(const Plan& p, int32_t* row_token, float* row_w, int32_t* slot_pos,
                             RowBlock* rb, int32_t* n_rb, hipStream_t s);

struct GateUpArgs {
  const uint16_t* wg;   // [E, I, H]
  const uint16_t* wu;   // [E, I, H]
  const uint16_t* sg;   // [Is, H]  (shared)
  const uint16_t* su;   // [Is, H]
  const uint16_t* x;    // [T, H]
  const int32_t* row_token;
  const RowBlock* rb;
  const int32_t* n_rb;
  uint16_t* h;          // routed [KT, I] then shared [T, Is]
  float limit, limit_shared;
};
struct DownArgs {
  const uint16_t* wd;   // [E, H, I]
  const uint16_t* sd;   // [H, Is]
  const uint16_t* h;
  const float* row_w;
  const RowBlock* rb;
  const int32_t* n_rb;
  uint16_t* o;          // [rows_total, H]
};
hipError_t launch_gate_up(const Plan& p, const GateUpArgs& a, hipStream_t s);
hipError_t launch_down(const Plan& p, const DownArgs& a, hipStream_t s);
// dense FFN at T <= 16 (plan nb == 1, p.E = p.K = S slices): gate/up with
// the row list implied by the block index, and the down projection summed
// over the S <= 8 slices in the workgroup, written straight to y
hipError_t launch_gate_up_dense(const Plan& p, const GateUpArgs& a, hipStream_t s);
hipError_t launch_dense_down(const Plan& p, const uint16_t* wd, const uint16_t* h, uint16_t* y,
                             hipStream_t s);
// large row blocks (plan nb == 12): LDS-pipelined variants
hipError_t launch_gate_up_lds(const Plan& p, const GateUpArgs& a, hipStream_t s);
hipError_t launch_down_lds(const Plan& p, const DownArgs& a, hipStream_t s);

// counts[0..E) = 0 and offsets[0..E] = 0 (the routing of an empty batch)
hipError_t launch_read_probe(const void* buf, size_t bytes, bool nontemporal, void* sink,
                             hipStream_t s);
// one workgroup of 8 waves on each of `grid` CUs, `iters` rounds of 4 MFMAs
hipError_t launch_mfma_probe(int iters, int grid, unsigned long long* clocks, void* sink,
                             hipStream_t s);
hipError_t launch_zero_counts(int32_t* counts, int32_t* offsets, int E, hipStream_t s);

hipError_t launch_pack(const uint16_t* src, uint16_t* dst, int n_mats, int rows, int cols,
                       long long ld, long long mat_stride, hipStream_t s);

hipError_t launch_combine(const Plan& p, const uint16_t* o, const int32_t* slot_pos,
                          uint16_t* y, hipStream_t s);
hipError_t launch_residual_rmsnorm(int T, int H, const uint16_t* r_in, const uint16_t* y_add,
                                   const float* gamma, float eps, uint16_t* r_out,
                                   uint16_t* x_out, hipStream_t s);
// per-group activation statistics of h, and their max/min-to-median ratios
hipError_t launch_expert_stats(int T, int E, int K, int I, int Is, const int32_t* offsets,
                               const uint16_t* h, float* stats, float* ratios, hipStream_t s);
// combine + residual add (+ the next layer's RMSNorm when x_out != null)
hipError_t launch_combine_residual(const Plan& p, const uint16_t* o, const int32_t* slot_pos,
                                   const uint16_t* r_in, const float* gamma, float eps,
                                   uint16_t* r_out, uint16_t* x_out, hipStream_t s);

}  // namespace smoe
