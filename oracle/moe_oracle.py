"""CPU oracle for the forward pass of one Step-3.5-Flash sparse MoE FFN layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
`cpu_baseline` leg may import this module.  The HIP library never calls it,
and it shares no code with the HIP library.

Plain, slow, float64 NumPy.  Inputs are the exact values the GPU received
(bf16 / fp32), widened to float64 without change.

Sources (the pages this follows; short tags used below):
  [P1 Method]  hyper.ai summary of arXiv 2602.10604 (Chinese), section 方法:
               every MoE layer routes each token to 8 of 288 routed experts
               plus one shared expert.
  [P2 Design]  shd-paper.top summary, 方法详解 / 关键设计: a gating network
               takes the token representation, gives one weight per expert,
               and the highest-weighted experts are used.
  [P3 2.2]     paperlayer.ai summary, §2.2 Sparse MoE Backbone with Hybrid
               Attention: 288 routed + 1 shared expert per MoE layer, top-8.
  [P3 App.B]   paperlayer.ai summary, App. B Detail Analysis of Localized
               Activation Blow-up: SwiGLU experts (gate and up activations,
               element-wise product); final representation = sum of layer
               outputs followed by RMSNorm.
  [P4 config]  LLM Atlas model card "Step-3.5-Flash" (zh-TW), raw config field
               table: moe_router_activation sigmoid, use_moe_router_bias true,
               need_fp32_gate true, moe_top_k 8, norm_expert_weight true,
               moe_router_scaling_factor 3, moe_intermediate_size 1280,
               share_expert_dim 1280, hidden_size 4096, zero_centered true,
               swiglu_limits mostly 0.0.

Readings taken where the pages are silent (each is an explicit switch or
constant below):
  A2  router bias enters after the sigmoid and steers selection only;
      `bias_in_weights=True` is the alternative reading (weights from s+b).
  A3  weights are normalised over the selected K and then scaled by 3.
  A4  a token's K slots are listed in ascending expert id.
  A5  inside one expert's block, rows are in ascending token order.
  A6  SwiGLU: h = silu(Wg x) * (Wu x), silu(z) = z / (1 + exp(-z)).
  A7  the shared expert is added with weight 1 (not scaled by 3).
  A8  no SwiGLU clamp on the hot path (a limit of 0 means "off").
  A17 a positive SwiGLU limit clamps the gate from above and the up
      projection to [-limit, limit].
  A12 if the selected scores sum to 0, weights are uniform scale/K.
  A13 no capacity limit, no token dropping.  A14 no group-limited routing.
  A15 RMSNorm epsilon 1e-6, zero-centred gain (1 + gamma).
  Ties between equal keys go to the lower expert index.

  [P3 4.1.2], [P3 4.1.3]  paperlayer.ai summary, §4.1.2 (expert collapse:
               monitor per-expert activation norms; a falling
               minimum-to-median ratio warns of expert death) and §4.1.3
               (localized activation blow-up: the maximum-to-median
               activation-norm ratio exposes it).
  A18 an expert's activation norm is the L2 norm of a token's SwiGLU
      activation h (the product the blow-up appears in); per expert the
      mean over the tokens routed to it; the ratios compare those means
      over the experts with tokens, against their median.

Parity status: every function here is pinned by the CPU tests (dense brute
force, closed forms, invariants, hand-computed cases); none is unpinned.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

__all__ = [
    "bf16_bits_to_f64", "router_logits", "router_scores", "selection_keys",
    "select_topk", "routing_weights", "dispatch", "swiglu_hidden", "swiglu_ffn", "route",
    "moe_layer", "rmsnorm", "moe_chain", "dense_ffn", "activation_stats", "norm_ratios",
    "expert_activation_stats",
]


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly: a bf16 value is the
    top 16 bits of the float32 with the same sign, exponent and leading
    mantissa bits."""
    b = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def router_logits(x, Wr) -> np.ndarray:
    """l[t,e] = sum_h x[t,h] * Wr[e,h].  [P4 config] need_fp32_gate: the gate
    runs on x widened to fp32 (exact for bf16) with an fp32 weight; here the
    same values are multiplied in float64.  [P2 Design]: the gate's input is
    the token representation, its output one value per expert."""
    return _f64(x) @ _f64(Wr).T


def router_scores(logits) -> np.ndarray:
    """s = sigmoid(l) = 1 / (1 + exp(-l)).  [P4 config] moe_router_activation."""
    l = _f64(logits)
    return 1.0 / (1.0 + np.exp(-l))


def selection_keys(scores, bias) -> np.ndarray:
    """key = s + b (reading A2: the learned bias of [P4 config]
    use_moe_router_bias is added after the sigmoid)."""
    return _f64(scores) + _f64(bias)[None, :]


def select_topk(keys, K: int) -> np.ndarray:
    """The K experts with the largest keys per token; equal keys go to the
    lower expert index.  Returned in ascending expert id (reading A4).
    [P4 config] moe_top_k; [P2 Design] the highest-weighted experts are used.

    Comparisons are exact in whatever precision `keys` carries, so feeding the
    GPU's own fp32 keys reproduces its discrete decision exactly."""
    keys = np.asarray(keys)
    T, E = keys.shape
    sel = np.empty((T, K), dtype=np.int64)
    for t in range(T):
        # lexsort: last key is primary -> (-key ascending, index ascending)
        order = np.lexsort((np.arange(E), -keys[t].astype(np.float64)))
        sel[t] = np.sort(order[:K])
    return sel


def routing_weights(scores, sel, scale: float = 3.0, norm: bool = True,
                    bias=None, bias_in_weights: bool = False) -> np.ndarray:
    """w[t,j] = scale * g[t,sel_j] / sum_j' g[t,sel_j'] with g = s (reading A2)
    or g = s + b (alternative reading).  [P4 config] norm_expert_weight true,
    moe_router_scaling_factor 3.  Without normalisation w = scale * g.
    A zero denominator gives uniform scale / K (reading A12)."""
    g = _f64(scores)
    if bias_in_weights:
        g = g + _f64(bias)[None, :]
    gs = np.take_along_axis(g, sel, axis=1)
    if not norm:
        return scale * gs
    den = gs.sum(axis=1, keepdims=True)
    K = sel.shape[1]
    safe = np.where(den == 0.0, 1.0, den)
    w = scale * gs / safe
    return np.where(den == 0.0, scale / K, w)


def dispatch(sel, E: int) -> Dict[str, np.ndarray]:
    """Expert-contiguous dispatch structures (the grouping [P2 Design] implies;
    the pages fix no layout):
      counts[e]      slots routed to expert e
      offsets[e]     exclusive prefix sum of counts, offsets[E] = T*K
      perm_token[r]  token of expert-contiguous row r; inside an expert's block
                     rows are in ascending token order (reading A5)
      slot_pos[t,j]  the row that holds token t's slot j
    """
    sel = np.asarray(sel)
    T, K = sel.shape
    counts = np.zeros(E, dtype=np.int64)
    for t in range(T):
        for j in range(K):
            counts[sel[t, j]] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    fill = offsets[:E].copy()
    perm_token = np.empty(T * K, dtype=np.int64)
    slot_pos = np.empty((T, K), dtype=np.int64)
    for t in range(T):            # ascending t -> token-ascending blocks
        for j in range(K):
            e = sel[t, j]
            r = fill[e]
            fill[e] += 1
            perm_token[r] = t
            slot_pos[t, j] = r
    return dict(counts=counts, offsets=offsets, perm_token=perm_token,
                slot_pos=slot_pos)


def silu(z) -> np.ndarray:
    z = _f64(z)
    return z / (1.0 + np.exp(-z))


def swiglu_hidden(xr, Wg, Wu, limit: float = 0.0) -> np.ndarray:
    """The SwiGLU activation of one gated expert on rows xr [m, H]:
    h = silu(xr Wg^T) * (xr Wu^T), with Wg, Wu [I, H].  [P3 App.B]: the
    element-wise product of the gate and up activations.

    `limit` is [P4 config] swiglu_limits: 0 = no clamp (reading A8, the
    value of almost every layer).  A positive limit clamps the gate
    pre-activation from above and the up projection to [-limit, limit]
    before the product (reading A17; the pages name the limit, not its
    form)."""
    xr = _f64(xr)
    g = xr @ _f64(Wg).T
    u = xr @ _f64(Wu).T
    if limit > 0:
        g = np.minimum(g, limit)
        u = np.clip(u, -limit, limit)
    return silu(g) * u


def swiglu_ffn(xr, Wg, Wu, Wd, return_hidden: bool = False, limit: float = 0.0):
    """One gated expert on rows xr [m, H]: o = h Wd^T with h the SwiGLU
    activation (swiglu_hidden); Wd is [H, I].  The three matrices of size
    4096 x 1280 per expert are what the 196B/11B parameter counts of
    [P3 2.2] add up to."""
    h = swiglu_hidden(xr, Wg, Wu, limit)
    o = h @ _f64(Wd).T
    return (o, h) if return_hidden else o


def dense_ffn(x, Wg, Wu, Wd, limit: float = 0.0) -> np.ndarray:
    """The dense FFN of the model's first layers ([P3 2.2]: 3 dense and 42
    MoE layers; [P4 config] intermediate_size 11264): the same gated form as
    an expert, on every token, with no router."""
    return swiglu_ffn(x, Wg, Wu, Wd, limit=limit)


def activation_stats(h) -> np.ndarray:
    """[rows, sum ||h_r||, sum ||h_r||^2, max ||h_r||] over the rows of one
    expert's SwiGLU activations h [m, I] (zeros for m = 0).  [P3 4.1.2],
    [P3 4.1.3]: per-expert activation norms are what is monitored; [P3
    App.B]: the blow-up is in the SwiGLU product."""
    h = _f64(h)
    if h.shape[0] == 0:
        return np.zeros(4)
    n = np.sqrt(np.sum(h * h, axis=1))
    return np.array([h.shape[0], n.sum(), np.sum(n * n), n.max()])


def norm_ratios(stats) -> np.ndarray:
    """[max m_e / M, min m_e / M] over the experts with rows, m_e = mean
    activation norm (stats[e,1] / stats[e,0]) and M the median of the m_e.
    [P3 4.1.3]: the maximum-to-median ratio reveals localized blow-up;
    [P3 4.1.2]: a falling minimum-to-median ratio warns of expert death."""
    st = _f64(stats)
    act = st[:, 0] > 0
    m = st[act, 1] / st[act, 0]
    med = np.median(m)
    return np.array([m.max() / med, m.min() / med])


def expert_activation_stats(x, sel, Wg, Wu, Ws_g=None, Ws_u=None, limit: float = 0.0,
                            limit_shared: float = 0.0, E: Optional[int] = None) -> np.ndarray:
    """activation_stats of every routed expert e < E over the tokens that
    selected it, then of the shared expert over all tokens (when given):
    an [E (+1), 4] array."""
    x = _f64(x)
    sel = np.asarray(sel, dtype=np.int64)
    E = int(sel.max()) + 1 if E is None else E
    rows = []
    for e in range(E):
        t = np.nonzero((sel == e).any(axis=1))[0]
        rows.append(activation_stats(swiglu_hidden(x[t], Wg[e], Wu[e], limit)) if t.size
                    else np.zeros(4))
    if Ws_g is not None:
        rows.append(activation_stats(swiglu_hidden(x, Ws_g, Ws_u, limit_shared)))
    return np.stack(rows)


def route(x, Wr, b, K: int, scale: float = 3.0, norm: bool = True,
          bias_in_weights: bool = False) -> Dict[str, np.ndarray]:
    """Steps a1-a4: logits, sigmoid, biased top-K, weights, dispatch."""
    logits = router_logits(x, Wr)
    s = router_scores(logits)
    keys = selection_keys(s, b)
    sel = select_topk(keys, K)
    w = routing_weights(s, sel, scale, norm, b, bias_in_weights)
    out = dict(logits=logits, scores=s, keys=keys, topk_idx=sel, topk_w=w)
    out.update(dispatch(sel, np.asarray(Wr).shape[0]))
    return out


def moe_layer(x, Wr, b, Wg, Wu, Wd, Ws_g=None, Ws_u=None, Ws_d=None, K: int = 8,
              scale: float = 3.0, norm: bool = True, bias_in_weights: bool = False,
              sel: Optional[np.ndarray] = None, return_parts: bool = False,
              limit: float = 0.0, limit_shared: float = 0.0):
    """y_t = sum_j w[t,j] * FFN_{sel_j}(x_t) + S(x_t), computed expert by
    expert over the dispatch of `route`.  [P1 Method], [P3 2.2]: 8 of 288
    routed experts plus one always-on shared expert; the shared expert adds
    with weight 1 (reading A7).  No capacity limit (A13).

    Wg/Wu/Wd may be any object whose [e] returns expert e's matrix, so callers
    can stream large weight stacks one expert at a time.  `sel` overrides the
    selection (used to follow a given routing of near-tied tokens)."""
    x = _f64(x)
    T = x.shape[0]
    r = route(x, Wr, b, K, scale, norm, bias_in_weights)
    if sel is not None:
        sel = np.asarray(sel, dtype=np.int64)
        r["topk_idx"] = sel
        r["topk_w"] = routing_weights(r["scores"], sel, scale, norm, b, bias_in_weights)
        r.update(dispatch(sel, np.asarray(Wr).shape[0]))
    sel, w = r["topk_idx"], r["topk_w"]
    routed = np.zeros_like(x)
    for e in np.unique(sel):
        rows_t, rows_j = np.nonzero(sel == e)
        o = swiglu_ffn(x[rows_t], Wg[e], Wu[e], Wd[e], limit=limit)
        routed[rows_t] += w[rows_t, rows_j][:, None] * o
    shared = np.zeros_like(x)
    if Ws_g is not None:
        shared = swiglu_ffn(x, Ws_g, Ws_u, Ws_d, limit=limit_shared)
    y = routed + shared
    if return_parts:
        r.update(y=y, routed=routed, shared=shared)
        return r
    return y


def rmsnorm(v, eps: float = 1e-6, gamma=None) -> np.ndarray:
    """Zero-centred RMSNorm: v / sqrt(mean(v^2) + eps) * (1 + gamma).
    [P4 config] zero_centered true (gain stored as an offset from 1);
    [P3 App.B] RMSNorm over the summed layer outputs.  eps: reading A15."""
    v = _f64(v)
    ms = np.mean(v * v, axis=-1, keepdims=True)
    g = 1.0 if gamma is None else (1.0 + _f64(gamma))
    return v / np.sqrt(ms + eps) * g


def moe_chain(r0, layers: Sequence[dict], K: int = 8, scale: float = 3.0,
              eps: float = 1e-6) -> np.ndarray:
    """Pre-norm residual stream through several MoE layers (reading A10):
    x_l = RMSNorm(r_l); r_{l+1} = r_l + MoE_l(x_l).  Returns the last r.
    Each element of `layers` holds Wr, b, Wg, Wu, Wd, Ws_g, Ws_u, Ws_d."""
    r = _f64(r0)
    for L in layers:
        xl = rmsnorm(r, eps)
        r = r + moe_layer(xl, L["Wr"], L["b"], L["Wg"], L["Wu"], L["Wd"],
                          L.get("Ws_g"), L.get("Ws_u"), L.get("Ws_d"), K=K, scale=scale)
    return r
