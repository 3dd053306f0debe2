"""Pins for the CPU oracle: checks against what the pages and the mathematics
fix, never against the oracle itself (CPU only)."""
import math
import os

import numpy as np
import pytest

import oracle
from tests.brute import brute_moe, brute_mask, textbook_swiglu_row
from sparse_moe_transformer_fp32_amd.inputs import (
    WORKLOADS, FLASH, make_inputs, random_tiny)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _np(t):
    return t.detach().cpu().double().numpy()


def _args(inp, li=0):
    L = inp.layers[li]
    sh = (None, None, None) if L.ws_gate is None else (_np(L.ws_gate), _np(L.ws_up), _np(L.ws_down))
    return (_np(inp.x), _np(inp.router_ws[li]), _np(inp.router_bs[li]),
            _np(L.w_gate), _np(L.w_up), _np(L.w_down)) + sh


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


TINY_SHAPES = [  # (seed, T, H, E, K, I, Is)
    (11, 5, 8, 6, 2, 4, 4),
    (12, 9, 16, 7, 3, 5, 6),
    (13, 3, 12, 4, 4, 12, 0),      # K == E, I == H (square: catches transposes)
    (14, 17, 10, 9, 1, 3, 2),
    (15, 8, 6, 12, 5, 6, 6),
]


# P1: oracle == dense brute force -------------------------------------------
def test_p1_tiny_workload_matches_brute_force():
    inp = make_inputs(WORKLOADS["tiny"])
    a = _args(inp)
    y = oracle.moe_layer(*a, K=2)
    yb, _, _ = brute_moe(*a, K=2)
    assert _rel(y, yb) < 1e-12


@pytest.mark.parametrize("shape", TINY_SHAPES)
def test_p1_random_tiny_matches_brute_force(shape):
    seed, T, H, E, K, I, Is = shape
    inp = random_tiny(seed, T, H, E, K, I, Is)
    a = _args(inp)
    if Is == 0:
        a = a[:6]
    for biw in (False, True):
        r = oracle.moe_layer(*a, K=K, bias_in_weights=biw, return_parts=True)
        yb, mb, wb = brute_moe(*a, K=K, bias_in_weights=biw)
        assert _rel(r["y"], yb) < 1e-12
        m = np.zeros_like(mb)
        np.put_along_axis(m, r["topk_idx"], True, axis=1)
        assert (m == mb).all()
        wd = np.zeros_like(wb)
        np.put_along_axis(wd, r["topk_idx"], r["topk_w"], axis=1)
        assert np.allclose(wd, wb, rtol=1e-13, atol=1e-15)


# P2 / P3: invariants of weights and dispatch --------------------------------
@pytest.mark.parametrize("shape", TINY_SHAPES + [(21, 64, 32, 16, 2, 8, 8), (22, 40, 16, 33, 8, 4, 4)])
def test_p2_p3_weights_and_dispatch(shape):
    seed, T, H, E, K, I, Is = shape
    inp = random_tiny(seed, T, H, E, K, I, Is)
    r = oracle.route(_np(inp.x), _np(inp.router_w), _np(inp.router_b), K)
    assert np.allclose(r["topk_w"].sum(axis=1), 3.0, rtol=0, atol=1e-12)     # P2
    sel, counts, off = r["topk_idx"], r["counts"], r["offsets"]
    perm, pos = r["perm_token"], r["slot_pos"]
    assert (np.diff(sel, axis=1) > 0).all()          # distinct, ascending ids
    assert counts.sum() == K * T
    assert off[0] == 0 and off[E] == K * T and (np.diff(off) == counts).all()
    assert sorted(pos.ravel().tolist()) == list(range(K * T))  # each row once
    for t in range(T):
        for j in range(K):
            rr = pos[t, j]
            assert perm[rr] == t
            assert off[sel[t, j]] <= rr < off[sel[t, j] + 1]
    for e in range(E):
        blk = perm[off[e]:off[e + 1]]
        assert (np.diff(blk) > 0).all()                # token-ascending blocks
    # counts equal a plain histogram
    assert (counts == np.bincount(sel.ravel(), minlength=E)).all()


# P4: token-permutation equivariance ----------------------------------------
def test_p4_permutation_equivariance():
    inp = random_tiny(31, 23, 16, 10, 3, 8, 8)
    a = list(_args(inp))
    y = oracle.moe_layer(*a, K=3)
    p = np.random.default_rng(0).permutation(23)
    a[0] = a[0][p]
    y2 = oracle.moe_layer(*a, K=3)
    assert _rel(y2, y[p]) < 1e-12


# P5: identical routed experts -> y = 3 FFN(x) + S(x) -----------------------
def test_p5_identical_experts_closed_form():
    rng = np.random.default_rng(5)
    T, H, E, K, I = 7, 12, 9, 4, 6
    x = rng.normal(size=(T, H))
    Wr = rng.normal(size=(E, H)); b = rng.normal(size=E)
    g1, u1, d1 = rng.normal(size=(I, H)), rng.normal(size=(I, H)), rng.normal(size=(H, I))
    Wg, Wu, Wd = (np.repeat(m[None], E, 0) for m in (g1, u1, d1))
    sg, su, sd = rng.normal(size=(5, H)), rng.normal(size=(5, H)), rng.normal(size=(H, 5))
    y = oracle.moe_layer(x, Wr, b, Wg, Wu, Wd, sg, su, sd, K=K)
    ffn = lambda W1, W2, W3: np.array([textbook_swiglu_row(xv, W1, W2, W3) for xv in x])
    assert _rel(y, 3.0 * ffn(g1, u1, d1) + ffn(sg, su, sd)) < 1e-12


# P6: K=1 gives weight 3; K=E gives the dense normalised mixture -------------
def test_p6_k1_and_k_equals_e():
    rng = np.random.default_rng(6)
    x = rng.normal(size=(6, 8)); Wr = rng.normal(size=(5, 8)); b = rng.normal(size=5) * 0.1
    r1 = oracle.route(x, Wr, b, 1)
    assert np.all(r1["topk_w"] == 3.0)
    rE = oracle.route(x, Wr, b, 5)
    s = np.array([[1.0 / (1.0 + math.exp(-float(v))) for v in row] for row in x @ Wr.T])
    assert (rE["topk_idx"] == np.arange(5)[None]).all()
    assert np.allclose(rE["topk_w"], 3.0 * s / s.sum(1, keepdims=True), rtol=1e-14)


# P7: bias forcing; A2 (selection only) vs A2' (weights from s + b) ----------
def test_p7_bias_forcing_and_reading():
    rng = np.random.default_rng(7)
    T, H, E, K = 11, 8, 10, 3
    x = rng.normal(size=(T, H)); Wr = rng.normal(size=(E, H))
    forced = np.array([1, 4, 8])
    b = np.zeros(E); b[forced] = 10.0
    r = oracle.route(x, Wr, b, K)
    assert (r["topk_idx"] == forced[None]).all()
    s = 1.0 / (1.0 + np.exp(-(x @ Wr.T)))
    want = 3.0 * s[:, forced] / s[:, forced].sum(1, keepdims=True)
    assert np.allclose(r["topk_w"], want, rtol=1e-14)
    r2 = oracle.route(x, Wr, b, K, bias_in_weights=True)
    assert (r2["topk_idx"] == forced[None]).all()
    g = s[:, forced] + 10.0
    assert np.allclose(r2["topk_w"], 3.0 * g / g.sum(1, keepdims=True), rtol=1e-14)
    assert not np.allclose(r2["topk_w"], r["topk_w"], rtol=1e-3)


# Ties: all keys equal -> lowest K indices, uniform weights ------------------
def test_ties_go_to_lower_index():
    rng = np.random.default_rng(8)
    T, H, E, K, I = 4, 6, 7, 3, 5
    x = rng.normal(size=(T, H)); Wr = np.zeros((E, H)); b = np.zeros(E)
    Wg, Wu, Wd = rng.normal(size=(E, I, H)), rng.normal(size=(E, I, H)), rng.normal(size=(E, H, I))
    r = oracle.moe_layer(x, Wr, b, Wg, Wu, Wd, K=K, return_parts=True)
    assert (r["topk_idx"] == np.arange(K)[None]).all()
    assert np.all(r["topk_w"] == 1.0)                 # 3 * 0.5 / (3 * 0.5)
    want = sum(np.array([textbook_swiglu_row(xv, Wg[e], Wu[e], Wd[e]) for xv in x])
               for e in range(K))
    assert _rel(r["y"], want) < 1e-12
    # two equal keys straddling the K boundary: the lower index wins
    keys = np.array([[0.1, 0.7, 0.5, 0.7, 0.5, 0.2]])
    assert oracle.select_topk(keys, 3).tolist() == [[1, 2, 3]]
    assert oracle.select_topk(keys.astype(np.float32), 3).tolist() == [[1, 2, 3]]


# P8: zero down weights isolate each half; shared == textbook dense FFN -------
def test_p8_routed_and_shared_halves():
    inp = random_tiny(41, 6, 10, 8, 2, 4, 5)
    a = list(_args(inp))
    full = oracle.moe_layer(*a, K=2)
    a_noshared = a[:8] + [np.zeros_like(a[8])]
    a_norouted = a[:5] + [np.zeros_like(a[5])] + a[6:]
    y_r = oracle.moe_layer(*a_noshared, K=2)
    y_s = oracle.moe_layer(*a_norouted, K=2)
    dense = np.array([textbook_swiglu_row(xv, a[6], a[7], a[8]) for xv in a[0]])
    assert _rel(y_s, dense) < 1e-12
    assert _rel(y_r + y_s, full) < 1e-12


# P9: one expert row == textbook formula -------------------------------------
def test_p9_single_row_textbook():
    rng = np.random.default_rng(9)
    H, I = 7, 5
    xv = rng.normal(size=(1, H))
    Wg, Wu, Wd = rng.normal(size=(I, H)), rng.normal(size=(I, H)), rng.normal(size=(H, I))
    o, h = oracle.swiglu_ffn(xv, Wg, Wu, Wd, return_hidden=True)
    assert _rel(o[0], np.array(textbook_swiglu_row(xv[0], Wg, Wu, Wd))) < 1e-13
    # hand value: silu(2) * 3 with one-element matrices
    o1 = oracle.swiglu_ffn(np.array([[1.0]]), np.array([[2.0]]), np.array([[3.0]]), np.array([[0.5]]))
    assert abs(o1[0, 0] - 0.5 * 3.0 * 2.0 / (1.0 + math.exp(-2.0))) < 1e-15


# P10: parameter-count identity pins the gated 3-matrix expert --------------
def _golden():
    vals = {}
    with open(os.path.join(GOLDEN, "step35_flash_moe_config.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split(None, 1)
                vals[k] = v
    return vals


def test_p10_config_constants_and_parameter_count():
    g = _golden()
    assert int(g["hidden_size"]) == FLASH["H"]
    assert int(g["moe_num_experts"]) == FLASH["E"]
    assert int(g["moe_top_k"]) == FLASH["K"]
    assert int(g["moe_intermediate_size"]) == FLASH["I"]
    assert int(g["share_expert_dim"]) == FLASH["Is"]
    assert float(g["moe_router_scaling_factor"]) == 3.0
    assert g["moe_router_activation"] == "sigmoid" and g["norm_expert_weight"] == "true"
    lo, hi = (int(v) for v in g["moe_layers_enum"].split("-"))
    n_moe = hi - lo + 1
    assert n_moe == 42
    per_expert_gated = 3 * FLASH["H"] * FLASH["I"]
    moe_total = n_moe * (FLASH["E"] + 1) * per_expert_gated
    assert abs(moe_total / 1e9 - 190.9) < 0.1
    total = float(g["total_params_b"]) * 1e9
    # gated experts fit under the printed total with a few billion left for
    # attention, embeddings, dense layers and MTP; a 2-matrix expert cannot
    assert 0.9 * total < moe_total < total
    assert n_moe * (FLASH["E"] + 1) * 2 * FLASH["H"] * FLASH["I"] < 0.7 * total
    # active: 8 routed + 1 shared gated experts per MoE layer stay under 11B
    active_moe = n_moe * (FLASH["K"] + 1) * per_expert_gated
    assert active_moe < float(g["active_params_b"]) * 1e9 < active_moe + 6e9


# P11: linearity in the down projections -------------------------------------
def test_p11_linearity():
    inp = random_tiny(51, 9, 12, 8, 3, 6, 6)
    a = list(_args(inp))
    y = oracle.moe_layer(*a, K=3)
    c = -2.5
    a[5] = a[5] * c; a[8] = a[8] * c
    assert _rel(oracle.moe_layer(*a, K=3), c * y) < 1e-12


# Normalisation switch and zero denominator ---------------------------------
def test_unnormalised_and_zero_denominator():
    s = np.array([[0.2, 0.5, 0.1]])
    sel = np.array([[0, 1]])
    assert np.allclose(oracle.routing_weights(s, sel, 3.0, norm=False), [[0.6, 1.5]])
    z = np.zeros((1, 3))
    assert np.allclose(oracle.routing_weights(z, sel, 3.0), [[1.5, 1.5]])


# Sigmoid special values --------------------------------------------------------
def test_sigmoid_values():
    s = oracle.router_scores(np.array([0.0, math.log(3.0), -math.log(3.0)]))
    assert np.allclose(s, [0.5, 0.75, 0.25], rtol=0, atol=1e-15)


# RMSNorm closed forms ----------------------------------------------------------
def test_rmsnorm_closed_forms():
    v = np.array([[3.0, 4.0]])
    got = oracle.rmsnorm(v, eps=0.0)
    assert np.allclose(got, v / math.sqrt(12.5), rtol=1e-15)
    got = oracle.rmsnorm(v, eps=0.0, gamma=np.array([1.0, -0.5]))
    assert np.allclose(got, v / math.sqrt(12.5) * np.array([2.0, 0.5]), rtol=1e-15)
    rng = np.random.default_rng(3)
    w = rng.normal(size=(5, 64)) * 7
    out = oracle.rmsnorm(w, eps=1e-6)
    assert np.allclose(np.sqrt(np.mean(out ** 2, axis=1)), 1.0, atol=1e-6)
    assert np.allclose(oracle.rmsnorm(w, eps=1e-6), oracle.rmsnorm(3.0 * w, eps=9e-6), rtol=1e-12)


# Chain: zero down weights keep the stream; one layer is x + MoE(norm(x)) ------
def test_chain_closed_forms():
    inp = random_tiny(61, 7, 8, 6, 2, 4, 4)
    a = _args(inp)
    L = dict(Wr=a[1], b=a[2], Wg=a[3], Wu=a[4], Wd=a[5], Ws_g=a[6], Ws_u=a[7], Ws_d=a[8])
    r1 = oracle.moe_chain(a[0], [L], K=2)
    xn = a[0] / np.sqrt(np.mean(a[0] ** 2, axis=1, keepdims=True) + 1e-6)
    yb, _, _ = brute_moe(xn, *a[1:], K=2)
    assert _rel(r1, a[0] + yb) < 1e-12
    Z = dict(L, Wd=np.zeros_like(a[5]), Ws_d=np.zeros_like(a[8]))
    assert np.array_equal(oracle.moe_chain(a[0], [Z, Z, Z], K=2), a[0])


# bf16 decoding ---------------------------------------------------------------
def test_bf16_decode_exact():
    import torch
    vals = torch.tensor([0.0, -0.0, 1.0, -2.5, 3.140625, 1e-30, 65280.0, -1.0e38])
    bits = vals.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_bits_to_f64(bits)
    assert np.array_equal(got, vals.to(torch.bfloat16).double().numpy())
    assert oracle.bf16_bits_to_f64(np.array([0x3F80], np.uint16))[0] == 1.0
    assert oracle.bf16_bits_to_f64(np.array([0xC020], np.uint16))[0] == -2.5


# SwiGLU clamp (reading A17): hand values and the no-op limit ----------------
def test_swiglu_limit_closed_forms():
    x = np.array([[1.0]])
    Wd = np.array([[1.0]])
    # g = 9 -> clamped to 7; u = -12 -> clamped to -7
    o = oracle.swiglu_ffn(x, np.array([[9.0]]), np.array([[-12.0]]), Wd, limit=7.0)
    assert abs(o[0, 0] - 7.0 / (1.0 + math.exp(-7.0)) * -7.0) < 1e-14
    # the gate is clamped from above only: g = -9 stays
    o = oracle.swiglu_ffn(x, np.array([[-9.0]]), np.array([[3.0]]), Wd, limit=7.0)
    assert abs(o[0, 0] - (-9.0) / (1.0 + math.exp(9.0)) * 3.0) < 1e-15
    # a limit above every activation changes nothing
    inp = random_tiny(71, 6, 10, 8, 2, 4, 5)
    a = _args(inp)
    y0 = oracle.moe_layer(*a, K=2)
    y1 = oracle.moe_layer(*a, K=2, limit=1e6, limit_shared=1e6)
    assert np.array_equal(y0, y1)
    y2 = oracle.moe_layer(*a, K=2, limit=1e-3, limit_shared=1e-3)
    assert not np.allclose(y0, y2)


# Dense FFN of the first layers: the gated form on every token ---------------
def test_dense_ffn_textbook():
    rng = np.random.default_rng(21)
    T, H, I = 3, 6, 9
    x = rng.normal(size=(T, H))
    Wg, Wu, Wd = rng.normal(size=(I, H)), rng.normal(size=(I, H)), rng.normal(size=(H, I))
    y = oracle.dense_ffn(x, Wg, Wu, Wd)
    for t in range(T):
        assert _rel(y[t], np.array(textbook_swiglu_row(x[t], Wg, Wu, Wd))) < 1e-13
    # cutting the intermediate dimension into slices and adding the partial
    # outputs gives the same result (the slicing the HIP path uses)
    parts = sum(oracle.dense_ffn(x, Wg[s:s + 3], Wu[s:s + 3], Wd[:, s:s + 3]) for s in (0, 3, 6))
    assert _rel(parts, y) < 1e-13


# Per-expert activation statistics -------------------------------------------
def test_activation_stats_hand_computed():
    h = np.array([[3.0, 4.0], [0.0, 0.0], [6.0, 8.0]])
    assert np.allclose(oracle.activation_stats(h), [3, 15, 125, 10], rtol=0, atol=1e-12)
    assert np.array_equal(oracle.activation_stats(np.zeros((0, 2))), np.zeros(4))


def test_norm_ratios_hand_computed():
    # mean norms 1, (empty), 2, 4 -> median 2 over the three with rows
    st = np.array([[2, 2, 0, 1], [0, 0, 0, 0], [1, 2, 0, 2], [4, 16, 0, 4]], float)
    assert np.allclose(oracle.norm_ratios(st), [2.0, 0.5], rtol=0, atol=1e-15)
    # even count: means 1, 2, 3, 10 -> median 2.5
    st = np.array([[1, 1, 0, 1], [1, 2, 0, 2], [1, 3, 0, 3], [1, 10, 0, 10]], float)
    assert np.allclose(oracle.norm_ratios(st), [4.0, 0.4], rtol=0, atol=1e-15)


@pytest.mark.parametrize("shape", TINY_SHAPES)
def test_expert_stats_brute_force(shape):
    """Dense over every (token, expert): norms of the SwiGLU activation with
    the tanh-form sigmoid, masked by the counting top-K of tests/brute.py."""
    from tests.brute import _sig
    seed, T, H, E, K, I, Is = shape
    inp = random_tiny(seed, T, H, E, K, I, Is)
    x, Wr, b, Wg, Wu, Wd, Wsg, Wsu, Wsd = _args(inp)
    keys = _sig(x @ Wr.T) + b[None, :]
    m = brute_mask(keys, K)
    G = np.einsum("th,eih->tei", x, Wg)
    U = np.einsum("th,eih->tei", x, Wu)
    n = np.sqrt(np.einsum("tei,tei->te", G * _sig(G) * U, G * _sig(G) * U))
    want = np.stack([m.sum(0), (n * m).sum(0), (n * n * m).sum(0), (n * m).max(0)], axis=1)
    if Is:
        gs, us = x @ Wsg.T, x @ Wsu.T
        ns = np.sqrt(((gs * _sig(gs) * us) ** 2).sum(1))
        want = np.vstack([want, [T, ns.sum(), (ns * ns).sum(), ns.max()]])
    sel = oracle.select_topk(oracle.selection_keys(oracle.router_scores(
        oracle.router_logits(x, Wr)), b), K)
    got = oracle.expert_activation_stats(x, sel, Wg, Wu, Wsg if Is else None,
                                         Wsu if Is else None, E=E)
    assert got.shape == want.shape
    assert np.allclose(got, want, rtol=1e-12, atol=1e-14)


def test_norm_ratios_closed_forms():
    """Identical experts that see the same tokens have equal mean norms (both
    ratios 1); scaling one expert's up projection by c scales its norms by c."""
    rng = np.random.default_rng(31)
    T, H, E, I = 7, 6, 3, 4
    x = rng.normal(size=(T, H))
    wg, wu = rng.normal(size=(I, H)), rng.normal(size=(I, H))
    sel = np.tile(np.arange(E), (T, 1))                  # K = E: every token on every expert
    Wg = np.stack([wg] * E)
    st = oracle.expert_activation_stats(x, sel, Wg, np.stack([wu] * E), E=E)
    assert np.allclose(oracle.norm_ratios(st), [1.0, 1.0], rtol=0, atol=1e-13)
    st = oracle.expert_activation_stats(x, sel, Wg, np.stack([wu, wu, 3.0 * wu]), E=E)
    assert np.allclose(oracle.norm_ratios(st), [3.0, 1.0], rtol=0, atol=1e-13)
    st = oracle.expert_activation_stats(x, sel, Wg, np.stack([0.5 * wu, wu, wu]), E=E)
    assert np.allclose(oracle.norm_ratios(st), [1.0, 0.5], rtol=0, atol=1e-13)
