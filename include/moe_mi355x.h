/*
 * moe_mi355x.h -- C ABI of the MI355X (gfx950) forward pass of one sparse
 * Mixture-of-Experts FFN layer with the Step-3.5-Flash layer shape.
 *
 * What the layer computes (sources: the Step-3.5-Flash pages):
 *   - hyper.ai summary of arXiv 2602.10604, section "方法" (Method): each token
 *     goes to 8 of 288 routed experts plus one always-on shared expert.
 *   - shd-paper.top summary, "方法详解 / 关键设计": a gating network maps the
 *     token representation to one weight per expert; the highest-weighted
 *     experts are used.
 *   - paperlayer.ai summary, App. B (Detail Analysis of Localized Activation
 *     Blow-up): SwiGLU experts (gate and up activations multiplied
 *     element-wise); the residual stream is normalised with RMSNorm.
 *   - LLM Atlas model card "Step-3.5-Flash", raw config field table:
 *     hidden_size 4096, moe_num_experts 288, moe_top_k 8,
 *     moe_intermediate_size 1280, share_expert_dim 1280, need_fp32_gate,
 *     moe_router_activation sigmoid, use_moe_router_bias,
 *     norm_expert_weight, moe_router_scaling_factor 3, swiglu_limits,
 *     zero_centered, torch_dtype bfloat16.
 *
 *   logits l[t,e] = sum_h float(x[t,h]) * W_r[e,h]          (fp32)
 *   score  s[t,e] = 1 / (1 + exp(-l[t,e]))
 *   key    k[t,e] = s[t,e] + b[e]          (bias steers selection only)
 *   sel[t]        = the K largest keys, equal keys -> lower expert index,
 *                   listed in ascending expert id
 *   w[t,j]        = scale * s[t,sel_j] / sum_j' s[t,sel_j']   (norm_topk=1)
 *   FFN_e(v)      = Wd_e (silu(Wg_e v) * (Wu_e v)),  silu(z) = z/(1+e^-z)
 *   y[t]          = sum_j w[t,j] FFN_{sel_j}(x[t]) + FFN_shared(x[t])
 *
 * Conventions for every entry point:
 *   - Pointers named in the structs and arguments are DEVICE pointers unless
 *     marked "host".  The caller owns every buffer; the library allocates and
 *     frees nothing.  Scratch memory comes from the caller's workspace.
 *   - bf16 tensors are passed as uint16_t bit patterns (IEEE bfloat16).
 *   - Arrays are dense row-major; every device pointer must be 16-byte
 *     aligned.  Weights are read-only; x and y must not alias.
 *   - Calls are asynchronous on `stream` and never synchronise.  Argument
 *     checks run on the host before any HIP call, in the fixed order
 *     null -> layout -> shape -> option -> alignment -> workspace; a failed check
 *     returns a negative moe_status and sets moe_last_error().  A failed
 *     kernel launch returns MOE_ERR_DEVICE.  Faults during execution show
 *     up at the caller's next synchronisation of the stream.
 *   - The same inputs give bitwise-identical outputs (no float atomics).
 *   - Calls that share a workspace must not overlap in time.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 4

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = -1,        /* a required pointer is NULL                   */
  MOE_ERR_SHAPE = -2,       /* a size is out of the supported range         */
  MOE_ERR_DTYPE = -3,       /* weights not in the layout the call reads
                               (a weight struct whose `layout` is not
                               MOE_LAYOUT_PACKED)                           */
  MOE_ERR_WORKSPACE = -4,   /* workspace smaller than moe_workspace_bytes() */
  MOE_ERR_ALIGN = -5,       /* a device pointer is not 16-byte aligned      */
  MOE_ERR_DEVICE = -6,      /* a HIP call or kernel launch failed           */
  MOE_ERR_OPTION = -7       /* an option value is invalid, or buffers alias */
} moe_status;

/* Layer sizes (host struct).
 *   T  tokens, 0 <= T <= 1<<20.  T = 0 is an empty batch: a call reads and
 *      writes no array with a T dimension (those pointers may be NULL; the
 *      rest are checked as usual), moe_route and a routing output still
 *      receive counts = 0 and offsets = 0, and moe_expert_stats rejects it
 *   H  hidden size, a multiple of 128, 128 <= H <= 16384     (Flash: 4096)
 *   E  routed experts, 1 <= E <= 1024                          (Flash: 288)
 *   K  experts per token, 1 <= K <= min(E, 16)                 (Flash: 8)
 *   I  routed intermediate size, a multiple of 64, <= 16384    (Flash: 1280)
 *   Is shared intermediate size, 0 (no shared expert) or a multiple of 64
 *                                                              (Flash: 1280) */
typedef struct { int32_t T, H, E, K, I, Is; } moe_dims;

/* Routing and activation options (host struct).
 *   route_scale      moe_router_scaling_factor (Flash: 3.0); finite, > 0
 *   norm_topk        norm_expert_weight: 1 = normalise the K selected scores
 *                    to sum 1 before scaling (Flash), 0 = w = scale * s
 *   bias_in_weights  0 = the bias steers selection only (default reading);
 *                    1 = the weights also use s + b
 *   swiglu_limit     0 = off.  > 0: the routed experts clamp the gate
 *                    pre-activation from above at +limit and the up
 *                    projection to [-limit, +limit] before the product
 *                    (model card: swiglu_limits, 0 for most layers)
 *   swiglu_limit_shared  the same for the shared expert */
typedef struct {
  float route_scale;
  int32_t norm_topk;
  int32_t bias_in_weights;
  float swiglu_limit;
  float swiglu_limit_shared;
} moe_opts;

/* Router: W [E,H] fp32, b [E] fp32 (learned bias, may be all zero). */
typedef struct { const float* W; const float* b; } moe_router;

/* Packed weight layout.  moe_forward reads every expert matrix in the
 * fragment-packed layout that moe_pack_weights produces from the model's
 * row-major bf16 matrix W[R][C] (R a multiple of 16, C of 32): 16x32 tiles of
 * 512 elements, tile (rt, kt) holding rows 16rt..16rt+15 and columns
 * 32kt..32kt+31 at element offset (rt*(C/32) + kt)*512; inside a tile,
 * W[16rt + r][32kt + c] sits at offset 8*(16*(c/8) + r) + c%8.  A packed
 * matrix has the same size as the row-major one, so the pointer alone cannot
 * tell the two apart: every weight struct therefore states its layout, and
 * the compute calls refuse (MOE_ERR_DTYPE, before any HIP call) a struct that
 * does not declare MOE_LAYOUT_PACKED.  A zero-initialised struct declares
 * MOE_LAYOUT_ROW_MAJOR and is refused. */
#define MOE_LAYOUT_ROW_MAJOR 0   /* the model's row-major matrices (not read by
                                    the compute calls: pack them first)       */
#define MOE_LAYOUT_PACKED 1      /* the output of moe_pack_weights            */

/* Routed experts, bf16: layout (must be MOE_LAYOUT_PACKED), then
 * w_gate E x [I,H], w_up E x [I,H], w_down E x [H,I] in that layout (matrix
 * e at element offset e*I*H). */
typedef struct {
  int32_t layout;
  const uint16_t* w_gate;
  const uint16_t* w_up;
  const uint16_t* w_down;
} moe_experts;

/* Shared expert, bf16: layout (must be MOE_LAYOUT_PACKED), then w_gate
 * [Is,H], w_up [Is,H], w_down [H,Is] in that layout.  Pass NULL (or set
 * dims.Is = 0) for a layer without a shared expert. */
typedef struct {
  int32_t layout;
  const uint16_t* w_gate;
  const uint16_t* w_up;
  const uint16_t* w_down;
} moe_shared;

/* Routing outputs (device buffers owned by the caller).
 *   topk_idx   [T,K] int32  selected experts, ascending per token
 *   topk_w     [T,K] fp32   combine weights
 *   counts     [E]   int32  slots routed to each expert (sum = T*K)
 *   offsets    [E+1] int32  exclusive prefix sum of counts, offsets[E] = T*K
 *   perm_token [T*K] int32  token of each expert-contiguous row; inside an
 *                           expert's block rows are in ascending token order
 *   slot_pos   [T,K] int32  the row that holds token t's slot j
 *   keys       [T,E] fp32   optional (may be NULL): selection keys s + b
 *   scores     [T,E] fp32   optional (may be NULL): sigmoid scores s     */
typedef struct {
  int32_t* topk_idx;
  float* topk_w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm_token;
  int32_t* slot_pos;
  float* keys;
  float* scores;
} moe_routing;

/* The residual stream around one layer, for moe_forward_residual (host
 * struct of device pointers).  Pre-norm reading of paperlayer.ai summary,
 * App. B (the final representation is the sum of the layer outputs followed
 * by RMSNorm) with the model card's zero_centered gain:
 *   r_in    [T,H] bf16  residual stream entering the layer (non-NULL)
 *   r_out   [T,H] bf16  receives r_in + layer output, rounded once to bf16
 *                       (non-NULL; may alias r_in)
 *   x_next  [T,H] bf16  NULL, or receives the next layer's input
 *                       bf16(r / sqrt(mean(r^2) + eps) * (1 + gamma)), r the
 *                       stored bf16 r_out row; must not alias r_in or r_out
 *                       (it may alias the layer's own x)
 *   gamma   [H] fp32    zero-centred gain of that norm, or NULL (gain 1)
 *   eps                 finite, >= 0 */
typedef struct {
  const uint16_t* r_in;
  uint16_t* r_out;
  uint16_t* x_next;
  const float* gamma;
  float eps;
} moe_residual;

/* A dense gated FFN (the model's first, dense layers), bf16, layout
 * MOE_LAYOUT_PACKED: w_gate [I,H], w_up [I,H] as one packed matrix each;
 * w_down as S packed matrices [H, I/S], matrix s being columns
 * s*I/S .. (s+1)*I/S - 1 of the model's Wd [H,I] (see moe_dense_ffn). */
typedef moe_shared moe_ffn;

/* Byte offsets of the intermediates inside a workspace (host struct), for
 * inspection by tests.  h is bf16 [(T*K)*I + T*Is]: routed rows of width I
 * in expert-contiguous order, then the shared expert's T rows of width Is.
 * o is bf16 [T*K + T, H]: each row already multiplied by its combine weight
 * (shared rows by 1). */
typedef struct { size_t h, o, total; } moe_ws_layout;

/* Stages of moe_forward, in launch order (moe_route runs the first three). */
#define MOE_STAGE_ROUTE_LOGITS 0
#define MOE_STAGE_ROUTE_TOPK 1
#define MOE_STAGE_DISPATCH 2
#define MOE_STAGE_GATE_UP 3
#define MOE_STAGE_DOWN 4
#define MOE_STAGE_COMBINE 5
#define MOE_N_STAGES 6

/* ABI version of the library (MOE_ABI_VERSION of the header it was built
 * from). */
int32_t moe_abi_version(void);

/* Message of the last failed call on this thread (host string owned by the
 * library; valid until the next call on this thread; "" after success). */
const char* moe_last_error(void);

/* Workspace bytes that moe_route and moe_forward need for `d` (host; > 0,
 * also for T = 0).  Returns 0 if `d` is NULL or out of range. */
size_t moe_workspace_bytes(const moe_dims* d);

/* Offsets of h and o in a workspace for `d`.  Returns MOE_ERR_NULL or
 * MOE_ERR_SHAPE on bad arguments. */
moe_status moe_workspace_layout(const moe_dims* d, moe_ws_layout* out);

/* Steps 1-4 of the layer: router logits, sigmoid, biased top-K, weights and
 * the expert-contiguous dispatch (counts, offsets, perm_token, slot_pos).
 * Defining passages: LLM Atlas model card "Step-3.5-Flash", raw config field
 * table (need_fp32_gate: the gate in fp32; moe_router_activation sigmoid;
 * use_moe_router_bias; moe_top_k 8; norm_expert_weight;
 * moe_router_scaling_factor 3; moe_num_experts 288), and the shd-paper.top
 * summary, 方法详解 / 关键设计 (a gate gives one weight per expert and the
 * highest-weighted experts are used).  The pages leave open where the bias
 * enters; it is added after the sigmoid and steers the selection only
 * (opts->bias_in_weights = 1 selects the other reading).  Equal keys go to
 * the lower expert index; a token's slots are listed in ascending expert id
 * and an expert's rows in ascending token order.
 *   d, opts  host structs; opts may be NULL (Flash defaults: scale 3,
 *            normalised, bias for selection only, no clamp)
 *   x        [T,H] bf16 token representations
 *   router   host struct holding device pointers W and b
 *   out      host struct; all members except keys/scores must be non-NULL
 *   ws       device workspace of ws_bytes >= moe_workspace_bytes(d) */
moe_status moe_route(const moe_dims* d, const moe_opts* opts, const uint16_t* x,
                     const moe_router* router, const moe_routing* out,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/* The whole layer: moe_route, then per expert the gated FFN on its rows
 * (bf16 MFMA, fp32 accumulation, h rounded to bf16), the shared expert on
 * every token, and the weighted combine back to token order (fp32 sum in
 * slot order, shared last, rounded once to bf16).
 * Defining passages: the routing as for moe_route; the hyper.ai summary,
 * section 方法, and the paperlayer.ai summary, §2.2 (each token goes to 8 of
 * 288 routed experts plus one always-on shared expert); the paperlayer.ai
 * summary, App. B (SwiGLU experts: the gate activation times the up
 * projection); the model card's raw config field table (hidden_size 4096,
 * moe_intermediate_size 1280, share_expert_dim 1280, torch_dtype bfloat16).
 * The shared expert is added with weight 1.
 *   experts      host struct: layout MOE_LAYOUT_PACKED (else MOE_ERR_DTYPE)
 *                and device pointers (all non-NULL)
 *   shared       host struct or NULL; must be non-NULL with non-NULL
 *                members and layout MOE_LAYOUT_PACKED iff d->Is > 0
 *   y            [T,H] bf16 output
 *   routing_out  NULL, or a moe_routing as for moe_route to receive the
 *                routing (then the workspace keeps no copy of it)
 *   ws           device workspace of ws_bytes >= moe_workspace_bytes(d) */
moe_status moe_forward(const moe_dims* d, const moe_opts* opts, const uint16_t* x,
                       const moe_router* router, const moe_experts* experts,
                       const moe_shared* shared, uint16_t* y,
                       const moe_routing* routing_out, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/* Convert n_mats row-major bf16 matrices [rows, cols] (consecutive in src)
 * into the packed layout above (consecutive in dst); a weight struct that
 * points at the result declares layout MOE_LAYOUT_PACKED.  Done once when weights
 * are loaded.  rows must be a multiple of 16, cols of 32; src and dst must
 * not overlap; both 16-byte aligned.  Asynchronous on `stream`. */
moe_status moe_pack_weights(const uint16_t* src, uint16_t* dst, int32_t n_mats, int32_t rows,
                            int32_t cols, hipStream_t stream);

/* moe_pack_weights with a strided source: element (i, j) of source matrix m
 * is src[m*mat_stride + i*ld + j] (elements).  ld >= cols; ld and
 * mat_stride multiples of 8.  moe_pack_weights is the case ld = cols,
 * mat_stride = rows*cols.  Column slices of one wide matrix are packed with
 * mat_stride = the slice width, as moe_dense_ffn's w_down needs: Wd [H,I]
 * into S matrices [H, I/S] is n_mats = S, rows = H, cols = I/S, ld = I,
 * mat_stride = I/S.  dst receives n_mats packed [rows, cols] matrices. */
moe_status moe_pack_weights_strided(const uint16_t* src, uint16_t* dst, int32_t n_mats,
                                    int32_t rows, int32_t cols, int64_t ld, int64_t mat_stride,
                                    hipStream_t stream);

/* Glue between chained layers of a pre-norm residual stream (paperlayer.ai
 * summary, App. B: RMSNorm over the summed layer outputs; model card:
 * zero_centered).  For each of the T rows of width H (T = 0: nothing to do,
 * the pointers are not checked):
 *   r      = r_in + y_add            (fp32 add, stored to r_out as bf16;
 *                                     y_add may be NULL: r = r_in)
 *   x_out  = bf16( r' / sqrt(mean(r'^2) + eps) * (1 + gamma) )
 * where r' is the bf16 value stored for r.  gamma [H] fp32 may be NULL
 * (gain 1).  r_out may be NULL when y_add is NULL; x_out may be NULL (no
 * norm).  r_out may alias r_in.  H must be a multiple of 128 in [128,
 * 16384] (MOE_ERR_SHAPE otherwise); eps >= 0. */
moe_status moe_residual_rmsnorm(int32_t T, int32_t H, const uint16_t* r_in,
                                const uint16_t* y_add, const float* gamma, float eps,
                                uint16_t* r_out, uint16_t* x_out, hipStream_t stream);

/* The whole layer followed by the residual add and, optionally, the next
 * layer's norm (the combine, the add and the norm run as one kernel):
 *   r_out[t]  = bf16( r_in[t] + (sum_j w[t,j] FFN_{sel_j}(x[t]) + FFN_shared(x[t])) )
 *   x_next[t] = bf16( r_out[t] / sqrt(mean(r_out[t]^2) + eps) * (1 + gamma) )
 * The layer output is summed in fp32 in slot order (shared last) and added
 * to r_in in fp32 before the one rounding, so it is never stored on its own.
 * x is the layer's (already normalised) input; it must not alias r_in or
 * r_out.  Other arguments, the workspace and the errors are as for
 * moe_forward; res and, unless T = 0, its r_in, r_out must be non-NULL. */
moe_status moe_forward_residual(const moe_dims* d, const moe_opts* opts, const uint16_t* x,
                                const moe_router* router, const moe_experts* experts,
                                const moe_shared* shared, const moe_residual* res,
                                const moe_routing* routing_out, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/* Workspace bytes for moe_dense_ffn (host); 0 if the sizes are out of range. */
size_t moe_dense_workspace_bytes(int32_t T, int32_t H, int32_t I, int32_t S);

/* A dense gated FFN, y[t] = Wd (silu(Wg x[t]) * (Wu x[t])) (hyper.ai summary,
 * 方法, and paperlayer.ai summary, §2.2: the first three of the 45 layers
 * are dense; model card: intermediate_size 11264).  The intermediate
 * dimension is cut into S slices that run as S groups of the grouped
 * expert GEMMs, every token in every group with weight 1.  For T <= 16 and
 * S <= 8 the down projection adds the S slices' fp32 partial sums in slice
 * order and rounds y once to bf16; otherwise the S partial outputs of a
 * token are rounded to bf16 and added in fp32 in slice order, then rounded
 * once more.
 *   T, H     as in moe_dims
 *   I        intermediate size; I/S must be a multiple of 64, <= 16384
 *   S        slices, 1 <= S <= 16; T*S <= 1<<24.  w_down must have been
 *            packed for the same S.  More slices give small batches more
 *            workgroups (S = 8 for I = 11264).
 *   ffn      packed weights (moe_ffn above)
 *   swiglu_limit  as moe_opts.swiglu_limit (0 = off)
 *   y        [T,H] bf16 output, must not alias x
 *   ws       device workspace of ws_bytes >= moe_dense_workspace_bytes */
moe_status moe_dense_ffn(int32_t T, int32_t H, int32_t I, int32_t S, const uint16_t* x,
                         const moe_ffn* ffn, float swiglu_limit, uint16_t* y, void* ws,
                         size_t ws_bytes, hipStream_t stream);

/* Per-expert activation statistics for monitoring (T >= 1; paperlayer.ai summary,
 * §4.1.2 and §4.1.3: per-expert activation norms, whose maximum-to-median
 * ratio exposes localized blow-up and whose falling minimum-to-median ratio
 * warns of expert death; App. B: the blow-up is in the SwiGLU product h).
 * Reads h and offsets of a finished moe_forward / moe_forward_residual call
 * with the same d: h at workspace offset moe_ws_layout.h, offsets from the
 * routing output (or the caller's copy).  With ||h_r|| the L2 norm of row r
 * of h (bf16 values, squares summed in fp32), for each routed expert g < E,
 * then the shared expert g = E when d->Is > 0:
 *   stats[4g..4g+3] = { rows, sum ||h_r||, sum ||h_r||^2, max ||h_r|| }  fp32
 * and, when ratios is non-NULL, over the routed experts with rows, m_e =
 * stats[4e+1] / stats[4e] and M their median (mean of the two middle values
 * for an even count):
 *   ratios[0] = max m_e / M,  ratios[1] = min m_e / M                   fp32
 * stats has 4*(E+1) floats (4*E without a shared expert), ratios 2.
 * Deterministic (fixed-order sums).  Errors as for moe_forward. */
moe_status moe_expert_stats(const moe_dims* d, const int32_t* offsets, const uint16_t* h,
                            float* stats, float* ratios, hipStream_t stream);

/* Per-stage timing hook for benchmarks and profilers (thread-local, host).
 * `events` is a host array of 2*MOE_N_STAGES hipEvent_t created by the
 * caller (hipEventCreate); while it is set, every moe_route / moe_forward on
 * this thread records events[2*i] just before and events[2*i+1] just after
 * stage i on the call's stream, so hipEventElapsedTime(events[2*i],
 * events[2*i+1]) is that kernel's duration.  Pass NULL (n_events ignored) to
 * stop.  Returns MOE_ERR_SHAPE unless n_events == 2*MOE_N_STAGES. */
moe_status moe_set_stage_events(hipEvent_t* events, int32_t n_events);

/* Measurement aid, not part of the layer: reads `bytes` of device memory at
 * `buf` once with 16-byte loads (`nontemporal` = 1: non-temporal loads, the
 * kind the weight streams use; 0: ordinary loads), two 256-thread
 * workgroups per CU in a grid-stride loop, enqueued on `stream`.  It gives
 * the HBM read rate a plain stream reaches, the practical ceiling the GEMMs'
 * weight streams are compared with.  `sink` (16 bytes, device) is written
 * only in a case that does not occur, so the kernel moves no data but the
 * reads.  Returns MOE_ERR_NULL, MOE_ERR_ALIGN (buf or sink not 16-byte
 * aligned), MOE_ERR_SHAPE (bytes not a positive multiple of 16384),
 * MOE_ERR_OPTION, or MOE_ERR_DEVICE (launch failed). */
moe_status moe_read_probe(const void* buf, size_t bytes, int32_t nontemporal, void* sink,
                          hipStream_t stream);

/* Measurement aid, not part of the layer: the bf16 matrix-core rate the
 * chip sustains on work without memory traffic, the practical ceiling the
 * GEMMs' MFMA figures are compared with next to the nominal peak.  One
 * workgroup of 8 waves (two per SIMD) on each compute unit; each wave runs
 * `iters` rounds of four independent v_mfma_f32_32x32x16_bf16 on register
 * operands: CUs x 8 x iters x 4 x 32768 FLOPs, enqueued on `stream`.
 * `clocks` (device, n_clocks >= 2 x the CU count uint64 values) receives for
 * each workgroup the shader clock counter (s_memtime) and the 100 MHz
 * real-time counter (s_memrealtime) elapsed over its loop: their ratio
 * times 100 MHz is the clock the matrix cores ran at.  `sink` (16 bytes,
 * device) is written only in a case that does not occur.  Returns
 * MOE_ERR_NULL, MOE_ERR_ALIGN (clocks or sink not 16-byte aligned),
 * MOE_ERR_SHAPE (iters outside [1, 1 << 24], or n_clocks too small), or
 * MOE_ERR_DEVICE (device query or launch failed). */
moe_status moe_mfma_probe(int32_t iters, uint64_t* clocks, int32_t n_clocks, void* sink,
                          hipStream_t stream);

/* For callers that cannot allocate: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  moe_forward with the
 * same arguments minus the workspace: the scratch memory comes from a fixed
 * device array of MOE_NOALLOC_SCRATCH_BYTES inside the library (one per GPU,
 * held until the process ends), so the call allocates nothing.
 *   - The stream must belong to the current device (MOE_ERR_DEVICE
 *     otherwise); the first call on a device looks up that device's array.
 *   - Layers whose moe_workspace_bytes(d) exceeds MOE_NOALLOC_SCRATCH_BYTES
 *     are refused with MOE_ERR_WORKSPACE (at the Flash shape: T > 290);
 *     use moe_forward with a workspace for them.
 *   - Every call on one GPU shares that GPU's array: calls that overlap in
 *     time on one GPU (two streams, two threads) race and must not be made.
 *     Nothing in it needs clearing between calls: no call depends on what
 *     an earlier one left there (every scratch value a call uses, the same
 *     call wrote first).  A routing output, if asked for, goes to the
 *     caller's buffers as for moe_forward; the h and o intermediates stay in
 *     the array (moe_ws_layout gives their offsets in it).
 * Checks and errors are as for moe_forward. */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
moe_status moe_forward_noalloc(const moe_dims* d, const moe_opts* opts, const uint16_t* x,
                               const moe_router* router, const moe_experts* experts,
                               const moe_shared* shared, uint16_t* y,
                               const moe_routing* routing_out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
