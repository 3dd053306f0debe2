// C-ABI entry points: argument checks (host only, before any HIP call), the
// tiling plan, workspace carving and the kernel launch sequence.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "moe_mi355x.h"
#include "smoe_internal.h"

namespace {

thread_local std::string g_err;
thread_local hipEvent_t* g_stage_events = nullptr;

// Records the stage's begin/end event when the timing hook is set.
struct StageMark {
  int stage;
  hipStream_t s;
  StageMark(int st, hipStream_t stream) : stage(st), s(stream) {
    if (g_stage_events) (void)hipEventRecord(g_stage_events[2 * stage], s);
  }
  ~StageMark() {
    if (g_stage_events) (void)hipEventRecord(g_stage_events[2 * stage + 1], s);
  }
};

moe_status fail(moe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

moe_status ok() {
  g_err.clear();
  return MOE_OK;
}

size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

moe_status check_shape(const moe_dims* d) {
  if (d->T < 0 || d->T > (1 << 20))
    return fail(MOE_ERR_SHAPE, "T=%d out of range [0, 1048576]", d->T);
  if (d->H < 128 || d->H > 16384 || d->H % 128)
    return fail(MOE_ERR_SHAPE, "H=%d must be a multiple of 128 in [128, 16384]", d->H);
  if (d->E < 1 || d->E > 1024) return fail(MOE_ERR_SHAPE, "E=%d out of range [1, 1024]", d->E);
  if (d->K < 1 || d->K > 16 || d->K > d->E)
    return fail(MOE_ERR_SHAPE, "K=%d must be in [1, min(E=%d, 16)]", d->K, d->E);
  if (d->I < 64 || d->I > 16384 || d->I % 64)
    return fail(MOE_ERR_SHAPE, "I=%d must be a multiple of 64 in [64, 16384]", d->I);
  if (d->Is < 0 || d->Is > 16384 || d->Is % 64)
    return fail(MOE_ERR_SHAPE, "Is=%d must be 0 or a multiple of 64 up to 16384", d->Is);
  return MOE_OK;
}

moe_status check_dense(int T, int H, int I, int S) {
  if (T < 0 || T > (1 << 20)) return fail(MOE_ERR_SHAPE, "T=%d out of range [0, 1048576]", T);
  if (H < 128 || H > 16384 || H % 128)
    return fail(MOE_ERR_SHAPE, "H=%d must be a multiple of 128 in [128, 16384]", H);
  if (S < 1 || S > 16) return fail(MOE_ERR_SHAPE, "S=%d out of range [1, 16]", S);
  if (I < 64 || I % S || (I / S) % 64 || I / S > 16384)
    return fail(MOE_ERR_SHAPE, "I=%d must split into S=%d slices that are multiples of 64", I, S);
  if ((long long)T * S > (1 << 24))
    return fail(MOE_ERR_SHAPE, "T*S=%lld rows exceed 16777216", (long long)T * S);
  return MOE_OK;
}

moe_status check_opts(const moe_opts* o) {
  if (!o) return MOE_OK;
  if (!isfinite(o->route_scale) || o->route_scale <= 0.f)
    return fail(MOE_ERR_OPTION, "route_scale must be finite and > 0");
  if (o->norm_topk != 0 && o->norm_topk != 1) return fail(MOE_ERR_OPTION, "norm_topk must be 0 or 1");
  if (o->bias_in_weights != 0 && o->bias_in_weights != 1)
    return fail(MOE_ERR_OPTION, "bias_in_weights must be 0 or 1");
  if (!isfinite(o->swiglu_limit) || o->swiglu_limit < 0.f ||
      !isfinite(o->swiglu_limit_shared) || o->swiglu_limit_shared < 0.f)
    return fail(MOE_ERR_OPTION, "swiglu limits must be finite and >= 0");
  return MOE_OK;
}

moe_opts default_opts() {
  moe_opts o;
  o.route_scale = 3.0f;
  o.norm_topk = 1;
  o.bias_in_weights = 0;
  o.swiglu_limit = 0.f;
  o.swiglu_limit_shared = 0.f;
  return o;
}

moe_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "%s launch failed: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

struct RouteBufs {
  int32_t *topk_idx, *counts, *offsets, *perm, *slot;
  float *topk_w, *keys, *scores;
};

moe_status run_route(const smoe::Plan& p, const moe_opts& o, const uint16_t* x,
                     const moe_router* router, const RouteBufs& rbuf, char* ws, hipStream_t s) {
  float* partial = reinterpret_cast<float*>(ws + p.ws_partial);
  moe_status st;
  {
    StageMark m(MOE_STAGE_ROUTE_LOGITS, s);
    if ((st = launched(smoe::launch_route_logits(p, x, router->W, partial, s), "route_logits")))
      return st;
  }
  {
    StageMark m(MOE_STAGE_ROUTE_TOPK, s);
    if ((st = launched(smoe::launch_route_topk(p, partial, router->b, o.route_scale, o.norm_topk,
                                               o.bias_in_weights, rbuf.topk_idx, rbuf.topk_w,
                                               rbuf.keys, rbuf.scores, s),
                       "route_topk")))
      return st;
  }
  smoe::RouteLaunch rl{};
  rl.topk_idx = rbuf.topk_idx;
  rl.topk_w = rbuf.topk_w;
  rl.counts = rbuf.counts;
  rl.offsets = rbuf.offsets;
  rl.perm = rbuf.perm;
  rl.slot = rbuf.slot;
  rl.row_token = reinterpret_cast<int32_t*>(ws + p.ws_row_token);
  rl.row_w = reinterpret_cast<float*>(ws + p.ws_row_w);
  rl.rb = reinterpret_cast<smoe::RowBlock*>(ws + p.ws_rb);
  rl.n_rb = reinterpret_cast<int32_t*>(ws + p.ws_nrb);
  rl.lrank = reinterpret_cast<int32_t*>(ws + p.ws_lrank);
  rl.hist = reinterpret_cast<int32_t*>(ws + p.ws_hist);
  rl.block_base = reinterpret_cast<int32_t*>(ws + p.ws_bbase);
  StageMark m(MOE_STAGE_DISPATCH, s);
  return launched(smoe::launch_dispatch(p, rl, s), "dispatch");
}

RouteBufs bufs_from(const moe_routing* r) {
  return RouteBufs{r->topk_idx, r->counts, r->offsets, r->perm_token, r->slot_pos,
                   r->topk_w,   r->keys,   r->scores};
}

RouteBufs bufs_from_ws(const smoe::Plan& p, char* ws) {
  return RouteBufs{reinterpret_cast<int32_t*>(ws + p.ws_topk_idx),
                   reinterpret_cast<int32_t*>(ws + p.ws_counts),
                   reinterpret_cast<int32_t*>(ws + p.ws_offsets),
                   reinterpret_cast<int32_t*>(ws + p.ws_perm),
                   reinterpret_cast<int32_t*>(ws + p.ws_slot),
                   reinterpret_cast<float*>(ws + p.ws_topk_w),
                   nullptr,
                   nullptr};
}

// An empty batch (T = 0) writes only counts and offsets.
moe_status check_routing_out(const moe_routing* r, bool for_route, bool empty) {
  if (!r->counts || !r->offsets ||
      (!empty && (!r->topk_idx || !r->topk_w || !r->perm_token || !r->slot_pos)))
    return fail(MOE_ERR_NULL, "%s: routing output members must be non-NULL (keys/scores optional)",
                for_route ? "moe_route" : "moe_forward");
  return MOE_OK;
}

// counts = 0 and offsets = 0: the routing of an empty batch
moe_status route_empty(int E, const moe_routing* r, hipStream_t s) {
  return launched(smoe::launch_zero_counts(r->counts, r->offsets, E, s), "zero_counts");
}

moe_status check_routing_align(const moe_routing* r) {
  const void* ptrs[] = {r->topk_idx, r->topk_w, r->counts, r->offsets,
                        r->perm_token, r->slot_pos, r->keys, r->scores};
  for (const void* q : ptrs)
    if (q && misaligned(q)) return fail(MOE_ERR_ALIGN, "routing output pointer %p not 16-byte aligned", q);
  return MOE_OK;
}

}  // namespace

namespace smoe {

// Router tiling: tokens per tile and the number of H splits for T tokens.
static int route_tiling(int T, int H, int E, int* route_tok) {
  // router: 16-token tiles for decode, 64 otherwise; split H until the
  // launch has ~1024 workgroups (each split keeps >= 256 columns) so that
  // loads of many waves overlap
  int S = 1;
  if (T >= 1024 && H % 64 == 0) {
    // many tokens: 256-token x 48-expert tiles (from 1024 tokens on they beat
    // the 64-token tiles on MI355X); split H while the launch stays within
    // two workgroups per CU
    *route_tok = 256;
    const int tiles = ((T + 255) / 256) * ((E + 47) / 48);
    while (S < 8 && tiles * 2 * S <= 512 && H % (2 * S * 64) == 0) S *= 2;
  } else {
    *route_tok = T <= 16 ? 16 : 64;
    const int tiles = ((T + *route_tok - 1) / *route_tok) * ((E + 63) / 64);
    const int min_cols = T <= 64 ? 128 : 256;
    while (S < 32 && tiles * S < 1024 && H % (2 * S * min_cols) == 0) S *= 2;
  }
  return S;
}

// The largest S(t) * t over 1 <= t <= T.  The router's partial sums take
// S * T * E floats; the split count falls as T grows, so S * T alone can
// shrink from one T to the next.  Sizing the buffer by this maximum keeps
// the workspace non-decreasing in T: one workspace sized for the largest
// batch serves every smaller one.
static size_t route_partial_rows(int T, int H, int E) {
  size_t best = 0;
  int rt;
  for (int t = 1; t <= std::min(T, 1023); ++t)
    best = std::max(best, (size_t)route_tiling(t, H, E, &rt) * t);
  // from 1024 tokens on S depends on ceil(t / 256) only, so within each
  // 256-token step the largest t is the step's last
  for (int k = 4; 256 * (k - 1) < T; ++k) {
    const int tt = std::min(256 * k, T);
    best = std::max(best, (size_t)route_tiling(tt, H, E, &rt) * tt);
  }
  return best;
}

void make_plan(int T, int H, int E, int K, int I, int Is, Plan* p) {
  *p = Plan{};
  p->T = T; p->H = H; p->E = E; p->K = K; p->I = I; p->Is = Is;
  p->KT = T * K;
  p->rows_total = p->KT + (Is > 0 ? T : 0);

  const int S = route_tiling(T, H, E, &p->route_tok);
  p->route_splits = S;

  // dispatch: one workgroup for small T, three kernels over 256-token blocks
  // for large T
  p->dispatch_blocks = T > 1024 ? (T + 255) / 256 : 0;

  // grouped GEMMs: row-block height follows the mean rows per expert
  const double avg = (double)K * T / E;
  int nb = avg <= 16 ? 1 : avg <= 32 ? 2 : avg <= 64 ? 4 : 12;
  if (nb == 12 && !(I % 128 == 0 && Is % 128 == 0 && H % 256 == 0)) nb = 4;
  p->nb = nb;
  p->bn = 16 * nb;
  // the LDS kernels multiply 32-token fragments, the register kernels 16
  p->rb_gran = nb == 12 ? 32 : 16;
  p->rb_max = std::min(E, p->KT) + p->KT / p->bn + (Is > 0 ? (T + p->bn - 1) / p->bn : 0);
  if (nb == 1) {
    p->ksplit_gu = 4;
    p->ksplit_dn = (I % 128 == 0 && Is % 128 == 0) ? 4 : 2;
    p->gu_rows_wg = 64 / p->ksplit_gu;
    p->dn_rows_wg = 128 / p->ksplit_dn;
  } else if (nb < 8) {
    p->ksplit_gu = p->ksplit_dn = 1;
    p->gu_rows_wg = 64;
    p->dn_rows_wg = 128;
  } else {  // LDS-pipelined kernels: 128 gate/up columns; 512 down rows
            // (256 when H is not a multiple of 512)
    p->ksplit_gu = p->ksplit_dn = 1;
    p->gu_rows_wg = 128;
    p->dn_rows_wg = H % 512 == 0 ? 512 : 256;
  }
  p->gu_tiles = std::max(I, Is) / p->gu_rows_wg;
  p->dn_tiles = H / p->dn_rows_wg;

  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  const size_t KT = (size_t)p->KT;
  p->ws_partial = take(route_partial_rows(T, H, E) * E * 4);
  p->ws_topk_idx = take(KT * 4);
  p->ws_topk_w = take(KT * 4);
  p->ws_counts = take((size_t)E * 4);
  p->ws_offsets = take((size_t)(E + 1) * 4);
  p->ws_perm = take(KT * 4);
  p->ws_slot = take(KT * 4);
  p->ws_row_token = take((size_t)p->rows_total * 4);
  p->ws_row_w = take((size_t)p->rows_total * 4);
  // the row-block list is sized for the finest cut (16-row blocks), a bound
  // on rb_max for every batch up to T, so that the workspace never shrinks
  // as T grows
  const size_t rb_cap = (size_t)std::min(E, p->KT) + p->KT / 16 + (Is > 0 ? (T + 15) / 16 : 0);
  p->ws_rb = take(std::max(rb_cap, (size_t)p->rb_max) * sizeof(RowBlock));
  p->ws_nrb = take(16);
  const size_t nblk = (size_t)p->dispatch_blocks;
  p->ws_lrank = take(nblk ? KT * 4 : 0);
  p->ws_hist = take(nblk * E * 4);
  p->ws_bbase = take(nblk * E * 4);
  p->ws_h = take((KT * I + (size_t)T * Is) * 2);
  p->ws_o = take((size_t)p->rows_total * H * 2);
  p->ws_total = off;
}

}  // namespace smoe

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_last_error(void) { return g_err.c_str(); }

size_t moe_workspace_bytes(const moe_dims* d) {
  if (!d) {
    fail(MOE_ERR_NULL, "moe_workspace_bytes: dims is NULL");
    return 0;
  }
  if (check_shape(d) != MOE_OK) return 0;
  smoe::Plan p;
  smoe::make_plan(d->T, d->H, d->E, d->K, d->I, d->Is, &p);
  ok();
  return p.ws_total;
}

moe_status moe_workspace_layout(const moe_dims* d, moe_ws_layout* out) {
  if (!d || !out) return fail(MOE_ERR_NULL, "moe_workspace_layout: NULL argument");
  moe_status st = check_shape(d);
  if (st) return st;
  smoe::Plan p;
  smoe::make_plan(d->T, d->H, d->E, d->K, d->I, d->Is, &p);
  out->h = p.ws_h;
  out->o = p.ws_o;
  out->total = p.ws_total;
  return ok();
}

moe_status moe_route(const moe_dims* d, const moe_opts* opts, const uint16_t* x,
                     const moe_router* router, const moe_routing* out, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  if (!d || !router || !router->W || !router->b || !out || !ws || (!x && d->T != 0))
    return fail(MOE_ERR_NULL, "moe_route: NULL argument (dims, x, router, router->W/b, out, ws)");
  moe_status st = check_routing_out(out, true, d->T == 0);
  if (st) return st;
  if ((st = check_shape(d))) return st;
  if ((st = check_opts(opts))) return st;
  if (misaligned(x) || misaligned(router->W) || misaligned(router->b) || misaligned(ws))
    return fail(MOE_ERR_ALIGN, "moe_route: x, router W/b and ws must be 16-byte aligned");
  if ((st = check_routing_align(out))) return st;
  smoe::Plan p;
  smoe::make_plan(d->T, d->H, d->E, d->K, d->I, d->Is, &p);
  if (ws_bytes < p.ws_total)
    return fail(MOE_ERR_WORKSPACE, "moe_route: workspace %zu bytes < required %zu", ws_bytes,
                p.ws_total);
  if (d->T == 0) {
    if ((st = route_empty(d->E, out, stream))) return st;
    return ok();
  }
  const moe_opts o = opts ? *opts : default_opts();
  if ((st = run_route(p, o, x, router, bufs_from(out), static_cast<char*>(ws), stream))) return st;
  return ok();
}

}  // extern "C"

namespace {

// The weight structs must declare the packed layout the GEMMs read: a
// row-major matrix has the same size, so it would otherwise pass every other
// check and give wrong output.
moe_status check_layout(const char* fn, const char* what, int32_t layout) {
  if (layout == MOE_LAYOUT_PACKED) return MOE_OK;
  if (layout == MOE_LAYOUT_ROW_MAJOR)
    return fail(MOE_ERR_DTYPE,
                "%s: %s weights declare MOE_LAYOUT_ROW_MAJOR; pack them with moe_pack_weights "
                "and declare MOE_LAYOUT_PACKED",
                fn, what);
  return fail(MOE_ERR_DTYPE, "%s: %s weights declare unknown layout %d", fn, what, layout);
}

// Checks shared by moe_forward and moe_forward_residual (null -> layout ->
// shape -> option -> alignment; the workspace is checked by the caller).
moe_status check_forward(const char* fn, const moe_dims* d, const moe_opts* opts,
                         const uint16_t* x, const moe_router* router,
                         const moe_experts* experts, const moe_shared* shared,
                         const moe_routing* routing_out) {
  moe_status st;
  if (d->Is > 0 && (!shared || !shared->w_gate || !shared->w_up || !shared->w_down))
    return fail(MOE_ERR_NULL, "%s: Is=%d but the shared expert weights are NULL", fn, d->Is);
  if (routing_out && (st = check_routing_out(routing_out, false, d->T == 0))) return st;
  if ((st = check_layout(fn, "routed expert", experts->layout))) return st;
  if (d->Is > 0 && (st = check_layout(fn, "shared expert", shared->layout))) return st;
  if ((st = check_shape(d))) return st;
  if ((st = check_opts(opts))) return st;
  if (misaligned(x) || misaligned(router->W) || misaligned(router->b) ||
      misaligned(experts->w_gate) || misaligned(experts->w_up) || misaligned(experts->w_down))
    return fail(MOE_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
  if (d->Is > 0 && (misaligned(shared->w_gate) || misaligned(shared->w_up) ||
                    misaligned(shared->w_down)))
    return fail(MOE_ERR_ALIGN, "%s: shared expert pointers must be 16-byte aligned", fn);
  if (routing_out && (st = check_routing_align(routing_out))) return st;
  return MOE_OK;
}

// The two grouped GEMMs over the row list already in the workspace.
moe_status run_experts(const smoe::Plan& p, const moe_opts& o, const uint16_t* x,
                       const uint16_t* wg, const uint16_t* wu, const uint16_t* wd,
                       const moe_shared* shared, char* w, uint16_t* out_rows,
                       hipStream_t stream) {
  const smoe::RowBlock* rbl = reinterpret_cast<const smoe::RowBlock*>(w + p.ws_rb);
  const int32_t* nrb = reinterpret_cast<const int32_t*>(w + p.ws_nrb);
  uint16_t* h = reinterpret_cast<uint16_t*>(w + p.ws_h);
  const bool has_sh = p.Is > 0;
  moe_status st;

  smoe::GateUpArgs ga{};
  ga.wg = wg;
  ga.wu = wu;
  ga.sg = has_sh ? shared->w_gate : nullptr;
  ga.su = has_sh ? shared->w_up : nullptr;
  ga.x = x;
  ga.row_token = reinterpret_cast<const int32_t*>(w + p.ws_row_token);
  ga.rb = rbl;
  ga.n_rb = nrb;
  ga.h = h;
  ga.limit = o.swiglu_limit;
  ga.limit_shared = o.swiglu_limit_shared;
  {
    StageMark m(MOE_STAGE_GATE_UP, stream);
    const hipError_t e =
        p.nb == 12 ? smoe::launch_gate_up_lds(p, ga, stream) : smoe::launch_gate_up(p, ga, stream);
    if ((st = launched(e, "gate_up"))) return st;
  }

  smoe::DownArgs da{};
  da.wd = wd;
  da.sd = has_sh ? shared->w_down : nullptr;
  da.h = h;
  da.row_w = reinterpret_cast<const float*>(w + p.ws_row_w);
  da.rb = rbl;
  da.n_rb = nrb;
  da.o = out_rows;
  {
    StageMark m(MOE_STAGE_DOWN, stream);
    const hipError_t e =
        p.nb == 12 ? smoe::launch_down_lds(p, da, stream) : smoe::launch_down(p, da, stream);
    if ((st = launched(e, "down"))) return st;
  }
  return MOE_OK;
}

// moe_forward (res == nullptr: y = layer output) and moe_forward_residual
// (r_out = r_in + layer output, optionally followed by the next norm).
moe_status forward_impl(const char* fn, const moe_dims* d, const moe_opts* opts,
                        const uint16_t* x, const moe_router* router, const moe_experts* experts,
                        const moe_shared* shared, uint16_t* y, const moe_residual* res,
                        const moe_routing* routing_out, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  smoe::Plan p;
  smoe::make_plan(d->T, d->H, d->E, d->K, d->I, d->Is, &p);
  if (ws_bytes < p.ws_total)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, ws_bytes,
                p.ws_total);
  if (d->T == 0) {   // empty batch: nothing to compute, routing output is empty
    moe_status st;
    if (routing_out && (st = route_empty(d->E, routing_out, stream))) return st;
    return ok();
  }
  const moe_opts o = opts ? *opts : default_opts();
  char* w = static_cast<char*>(ws);
  const RouteBufs rb = routing_out ? bufs_from(routing_out) : bufs_from_ws(p, w);
  moe_status st;
  if ((st = run_route(p, o, x, router, rb, w, stream))) return st;
  uint16_t* ob = reinterpret_cast<uint16_t*>(w + p.ws_o);
  if ((st = run_experts(p, o, x, experts->w_gate, experts->w_up, experts->w_down, shared, w, ob,
                        stream)))
    return st;
  StageMark m(MOE_STAGE_COMBINE, stream);
  const hipError_t e =
      res ? smoe::launch_combine_residual(p, ob, rb.slot, res->r_in, res->gamma, res->eps,
                                          res->r_out, res->x_next, stream)
          : smoe::launch_combine(p, ob, rb.slot, y, stream);
  if ((st = launched(e, "combine"))) return st;
  return ok();
}

}  // namespace

extern "C" {

moe_status moe_forward(const moe_dims* d, const moe_opts* opts, const uint16_t* x,
                       const moe_router* router, const moe_experts* experts,
                       const moe_shared* shared, uint16_t* y, const moe_routing* routing_out,
                       void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!d || !router || !router->W || !router->b || !experts || !experts->w_gate ||
      !experts->w_up || !experts->w_down || !ws || ((!x || !y) && d->T != 0))
    return fail(MOE_ERR_NULL,
                "moe_forward: NULL argument (dims, x, router, router->W/b, experts->w_*, y, ws)");
  moe_status st;
  if ((st = check_forward("moe_forward", d, opts, x, router, experts, shared, routing_out)))
    return st;
  if (misaligned(y) || misaligned(ws))
    return fail(MOE_ERR_ALIGN, "moe_forward: device pointers must be 16-byte aligned");
  if (x == y && d->T != 0) return fail(MOE_ERR_OPTION, "moe_forward: x and y must not alias");
  return forward_impl("moe_forward", d, opts, x, router, experts, shared, y, nullptr, routing_out,
                      ws, ws_bytes, stream);
}

moe_status moe_forward_residual(const moe_dims* d, const moe_opts* opts, const uint16_t* x,
                                const moe_router* router, const moe_experts* experts,
                                const moe_shared* shared, const moe_residual* res,
                                const moe_routing* routing_out, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  if (!d || !router || !router->W || !router->b || !experts || !experts->w_gate ||
      !experts->w_up || !experts->w_down || !res || !ws ||
      ((!x || !res->r_in || !res->r_out) && d->T != 0))
    return fail(MOE_ERR_NULL,
                "moe_forward_residual: NULL argument (dims, x, router, router->W/b, "
                "experts->w_*, res, res->r_in/r_out, ws)");
  moe_status st;
  if ((st = check_forward("moe_forward_residual", d, opts, x, router, experts, shared,
                          routing_out)))
    return st;
  if (!isfinite(res->eps) || res->eps < 0.f)
    return fail(MOE_ERR_OPTION, "moe_forward_residual: eps must be finite and >= 0");
  if (misaligned(res->r_in) || misaligned(res->r_out) || misaligned(res->x_next) ||
      misaligned(res->gamma) || misaligned(ws))
    return fail(MOE_ERR_ALIGN, "moe_forward_residual: device pointers must be 16-byte aligned");
  if (d->T != 0 && res->x_next && (res->x_next == res->r_out || res->x_next == res->r_in))
    return fail(MOE_ERR_OPTION, "moe_forward_residual: x_next must not alias r_in or r_out");
  if (d->T != 0 && (res->r_out == x || (const uint16_t*)res->r_in == x))
    return fail(MOE_ERR_OPTION, "moe_forward_residual: x must not alias r_in or r_out");
  return forward_impl("moe_forward_residual", d, opts, x, router, experts, shared, nullptr, res,
                      routing_out, ws, ws_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// moe_forward_noalloc: the scratch memory is this fixed device array.  In
// host code its name is a host-side stand-in, not a device address: host
// code only ever uses the address hipGetSymbolAddress returns for the current
// device, kept per device below.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device (looked up once per
// device, with that device current).
moe_status device_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_DEVICE, "device %d out of the supported range [0, %d)", dev, kMaxDevices);
  if (stream) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess)
      return fail(MOE_ERR_DEVICE, "hipStreamGetDevice failed: %s", hipGetErrorString(e));
    if (sdev != dev)
      return fail(MOE_ERR_DEVICE,
                  "moe_forward_noalloc: the stream belongs to device %d but device %d is current",
                  (int)sdev, dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(MOE_ERR_DEVICE, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_forward_noalloc(const moe_dims* d, const moe_opts* opts, const uint16_t* x,
                               const moe_router* router, const moe_experts* experts,
                               const moe_shared* shared, uint16_t* y,
                               const moe_routing* routing_out, hipStream_t stream) {
  if (!d || !router || !router->W || !router->b || !experts || !experts->w_gate ||
      !experts->w_up || !experts->w_down || ((!x || !y) && d->T != 0))
    return fail(MOE_ERR_NULL,
                "moe_forward_noalloc: NULL argument (dims, x, router, router->W/b, "
                "experts->w_*, y)");
  moe_status st;
  if ((st = check_forward("moe_forward_noalloc", d, opts, x, router, experts, shared,
                          routing_out)))
    return st;
  if (misaligned(y)) return fail(MOE_ERR_ALIGN, "moe_forward_noalloc: y must be 16-byte aligned");
  if (x == y && d->T != 0)
    return fail(MOE_ERR_OPTION, "moe_forward_noalloc: x and y must not alias");
  smoe::Plan p;
  smoe::make_plan(d->T, d->H, d->E, d->K, d->I, d->Is, &p);
  if (p.ws_total > MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_WORKSPACE,
                "moe_forward_noalloc: this layer needs %zu bytes of scratch, more than the "
                "fixed %u; call moe_forward with a workspace",
                p.ws_total, (unsigned)MOE_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((st = device_scratch(stream, &ws))) return st;
  return forward_impl("moe_forward_noalloc", d, opts, x, router, experts, shared, y, nullptr,
                      routing_out, ws, MOE_NOALLOC_SCRATCH_BYTES, stream);
}

size_t moe_dense_workspace_bytes(int32_t T, int32_t H, int32_t I, int32_t S) {
  if (check_dense(T, H, I, S) != MOE_OK) return 0;
  smoe::Plan p;
  smoe::make_plan(T, H, S, S, I / S, 0, &p);
  return p.ws_total;
}

moe_status moe_dense_ffn(int32_t T, int32_t H, int32_t I, int32_t S, const uint16_t* x,
                         const moe_ffn* ffn, float swiglu_limit, uint16_t* y, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  if (!ffn || !ffn->w_gate || !ffn->w_up || !ffn->w_down || !ws || ((!x || !y) && T != 0))
    return fail(MOE_ERR_NULL, "moe_dense_ffn: NULL argument (x, ffn, ffn->w_*, y, ws)");
  moe_status st;
  if ((st = check_layout("moe_dense_ffn", "dense FFN", ffn->layout))) return st;
  if ((st = check_dense(T, H, I, S))) return st;
  if (!isfinite(swiglu_limit) || swiglu_limit < 0.f)
    return fail(MOE_ERR_OPTION, "moe_dense_ffn: swiglu_limit must be finite and >= 0");
  if (misaligned(x) || misaligned(ffn->w_gate) || misaligned(ffn->w_up) ||
      misaligned(ffn->w_down) || misaligned(y) || misaligned(ws))
    return fail(MOE_ERR_ALIGN, "moe_dense_ffn: device pointers must be 16-byte aligned");
  if (x == y && T != 0) return fail(MOE_ERR_OPTION, "moe_dense_ffn: x and y must not alias");
  smoe::Plan p;
  smoe::make_plan(T, H, S, S, I / S, 0, &p);
  if (ws_bytes < p.ws_total)
    return fail(MOE_ERR_WORKSPACE, "moe_dense_ffn: workspace %zu bytes < required %zu", ws_bytes,
                p.ws_total);
  if (T == 0) return ok();   // empty batch
  char* w = static_cast<char*>(ws);
  if (p.nb == 1 && S <= 8) {
    // T <= 16: two kernels, no row list and no combine (the down projection
    // sums the slices itself)
    uint16_t* h = reinterpret_cast<uint16_t*>(w + p.ws_h);
    smoe::GateUpArgs ga{};
    ga.wg = ffn->w_gate;
    ga.wu = ffn->w_up;
    ga.x = x;
    ga.h = h;
    ga.limit = swiglu_limit;
    {
      StageMark m(MOE_STAGE_GATE_UP, stream);
      if ((st = launched(smoe::launch_gate_up_dense(p, ga, stream), "gate_up"))) return st;
    }
    StageMark m(MOE_STAGE_DOWN, stream);
    if ((st = launched(smoe::launch_dense_down(p, ffn->w_down, h, y, stream), "down"))) return st;
    return ok();
  }
  int32_t* slot = reinterpret_cast<int32_t*>(w + p.ws_slot);
  {
    StageMark m(MOE_STAGE_DISPATCH, stream);
    if ((st = launched(smoe::launch_dense_rows(
                           p, reinterpret_cast<int32_t*>(w + p.ws_row_token),
                           reinterpret_cast<float*>(w + p.ws_row_w), slot,
                           reinterpret_cast<smoe::RowBlock*>(w + p.ws_rb),
                           reinterpret_cast<int32_t*>(w + p.ws_nrb), stream),
                       "dense_rows")))
      return st;
  }
  moe_opts o = default_opts();
  o.swiglu_limit = swiglu_limit;
  uint16_t* ob = reinterpret_cast<uint16_t*>(w + p.ws_o);
  if ((st = run_experts(p, o, x, ffn->w_gate, ffn->w_up, ffn->w_down, nullptr, w, ob, stream)))
    return st;
  StageMark m(MOE_STAGE_COMBINE, stream);
  if ((st = launched(smoe::launch_combine(p, ob, slot, y, stream), "combine"))) return st;
  return ok();
}

moe_status moe_expert_stats(const moe_dims* d, const int32_t* offsets, const uint16_t* h,
                            float* stats, float* ratios, hipStream_t stream) {
  if (!d || !offsets || !h || !stats)
    return fail(MOE_ERR_NULL, "moe_expert_stats: NULL argument (dims, offsets, h, stats)");
  moe_status st;
  if ((st = check_shape(d))) return st;
  if (d->T < 1) return fail(MOE_ERR_SHAPE, "moe_expert_stats: T=0, an empty batch has no rows");
  if (misaligned(offsets) || misaligned(h) || misaligned(stats) || misaligned(ratios))
    return fail(MOE_ERR_ALIGN, "moe_expert_stats: device pointers must be 16-byte aligned");
  if ((st = launched(smoe::launch_expert_stats(d->T, d->E, d->K, d->I, d->Is, offsets, h, stats,
                                               ratios, stream),
                     "expert_stats")))
    return st;
  return ok();
}

moe_status moe_pack_weights_strided(const uint16_t* src, uint16_t* dst, int32_t n_mats,
                                    int32_t rows, int32_t cols, int64_t ld, int64_t mat_stride,
                                    hipStream_t stream) {
  if (!src || !dst) return fail(MOE_ERR_NULL, "moe_pack_weights: NULL src or dst");
  if (n_mats < 1 || rows < 16 || cols < 32 || rows % 16 || cols % 32)
    return fail(MOE_ERR_SHAPE,
                "moe_pack_weights: n_mats=%d rows=%d cols=%d (need >= 1, rows %% 16 == 0, "
                "cols %% 32 == 0)",
                n_mats, rows, cols);
  if (ld < cols || ld % 8 || mat_stride < 0 || mat_stride % 8)
    return fail(MOE_ERR_SHAPE,
                "moe_pack_weights: ld=%lld must be >= cols=%d, ld and mat_stride=%lld "
                "multiples of 8 and mat_stride >= 0",
                (long long)ld, cols, (long long)mat_stride);
  if (misaligned(src) || misaligned(dst))
    return fail(MOE_ERR_ALIGN, "moe_pack_weights: pointers must be 16-byte aligned");
  const size_t out_bytes = (size_t)n_mats * rows * cols * 2;
  const size_t in_bytes = ((size_t)(n_mats - 1) * mat_stride + (size_t)(rows - 1) * ld + cols) * 2;
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  if (a < b + out_bytes && b < a + in_bytes)
    return fail(MOE_ERR_OPTION, "moe_pack_weights: src and dst overlap");
  moe_status st = launched(
      smoe::launch_pack(src, dst, n_mats, rows, cols, ld, mat_stride, stream), "pack");
  if (st) return st;
  return ok();
}

moe_status moe_pack_weights(const uint16_t* src, uint16_t* dst, int32_t n_mats, int32_t rows,
                            int32_t cols, hipStream_t stream) {
  return moe_pack_weights_strided(src, dst, n_mats, rows, cols, cols, (int64_t)rows * cols,
                                  stream);
}

moe_status moe_read_probe(const void* buf, size_t bytes, int32_t nontemporal, void* sink,
                          hipStream_t stream) {
  if (!buf || !sink) return fail(MOE_ERR_NULL, "moe_read_probe: NULL buffer or sink");
  if (misaligned(buf) || misaligned(sink))
    return fail(MOE_ERR_ALIGN, "moe_read_probe: buf and sink must be 16-byte aligned");
  if (bytes == 0 || bytes % 16384)
    return fail(MOE_ERR_SHAPE, "moe_read_probe: bytes=%zu must be a positive multiple of 16384",
                bytes);
  if (nontemporal != 0 && nontemporal != 1)
    return fail(MOE_ERR_OPTION, "moe_read_probe: nontemporal must be 0 or 1");
  moe_status st;
  if ((st = launched(smoe::launch_read_probe(buf, bytes, nontemporal != 0, sink, stream),
                     "read_probe")))
    return st;
  return ok();
}

moe_status moe_mfma_probe(int32_t iters, uint64_t* clocks, int32_t n_clocks, void* sink,
                          hipStream_t stream) {
  if (!clocks || !sink) return fail(MOE_ERR_NULL, "moe_mfma_probe: NULL clocks or sink");
  if (misaligned(clocks) || misaligned(sink))
    return fail(MOE_ERR_ALIGN, "moe_mfma_probe: clocks and sink must be 16-byte aligned");
  if (iters < 1 || iters > (1 << 24))
    return fail(MOE_ERR_SHAPE, "moe_mfma_probe: iters=%d out of range [1, 16777216]", iters);
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess)
    return fail(MOE_ERR_DEVICE, "moe_mfma_probe: device query failed: %s", hipGetErrorString(e));
  if (n_clocks < 2 * cus)
    return fail(MOE_ERR_SHAPE, "moe_mfma_probe: n_clocks=%d < 2 x %d compute units", n_clocks,
                cus);
  moe_status st;
  if ((st = launched(smoe::launch_mfma_probe(iters, cus,
                                             reinterpret_cast<unsigned long long*>(clocks), sink,
                                             stream),
                     "mfma_probe")))
    return st;
  return ok();
}

moe_status moe_set_stage_events(hipEvent_t* events, int32_t n_events) {
  if (!events) {
    g_stage_events = nullptr;
    return ok();
  }
  if (n_events != 2 * MOE_N_STAGES)
    return fail(MOE_ERR_SHAPE, "moe_set_stage_events: n_events=%d, expected %d", n_events,
                2 * MOE_N_STAGES);
  g_stage_events = events;
  return ok();
}

moe_status moe_residual_rmsnorm(int32_t T, int32_t H, const uint16_t* r_in,
                                const uint16_t* y_add, const float* gamma, float eps,
                                uint16_t* r_out, uint16_t* x_out, hipStream_t stream) {
  if (T < 0 || T > (1 << 20)) return fail(MOE_ERR_SHAPE, "T=%d out of range [0, 1048576]", T);
  if (H < 128 || H > 16384 || H % 128)
    return fail(MOE_ERR_SHAPE, "H=%d must be a multiple of 128 in [128, 16384]", H);
  if (!isfinite(eps) || eps < 0.f) return fail(MOE_ERR_OPTION, "eps must be finite and >= 0");
  if (T == 0) return ok();   // empty batch: no rows, the pointers are not used
  if (!r_in) return fail(MOE_ERR_NULL, "moe_residual_rmsnorm: r_in is NULL");
  if (y_add && !r_out && !x_out)
    return fail(MOE_ERR_NULL, "moe_residual_rmsnorm: y_add given but both r_out and x_out NULL");
  if (!y_add && !x_out) return fail(MOE_ERR_NULL, "moe_residual_rmsnorm: nothing to compute");
  if (misaligned(r_in) || misaligned(y_add) || misaligned(gamma) || misaligned(r_out) ||
      misaligned(x_out))
    return fail(MOE_ERR_ALIGN, "moe_residual_rmsnorm: pointers must be 16-byte aligned");
  moe_status st = launched(
      smoe::launch_residual_rmsnorm(T, H, r_in, y_add, gamma, eps, r_out, x_out, stream),
      "residual_rmsnorm");
  if (st) return st;
  return ok();
}

}  // extern "C"
