"""HIP path vs CPU oracle, element by element, through the C-ABI (gfx950 GPU).

Small cases cover every tiling variant (row blocks of 16/32/64 tokens with
split-K 1/2/4 in the register-streaming kernels, 192-token blocks in the
LDS-pipelined kernels, and the fallback when shapes exclude them; the
64-token and the 256-token router tiles), ragged tails, T=1, K=1, K=E, E not a multiple of 64, the
largest E and K, no shared expert, the SwiGLU clamp and the alternative bias
reading.  Flash-shaped cases run the same launch configuration as the
benchmark: full outputs at T=16 and T=4096, sampled rows at T=8192.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_moe_transformer_fp32_amd import binding as B
from sparse_moe_transformer_fp32_amd.inputs import WORKLOADS, make_inputs, random_tiny
from tests.parity import LazyStack, check_output, check_routing, gpu_routing_np, host_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _to_gpu_bf16(inp):
    """Small CPU-drawn case -> device tensors; x and expert weights cast to
    bf16 (round to nearest even), router kept fp32."""
    L = inp.layers[0]
    bf = lambda t: None if t is None else t.to(torch.bfloat16).to(DEV).contiguous()
    f32 = lambda t: t.to(torch.float32).to(DEV).contiguous()
    return dict(x=bf(inp.x), Wr=f32(inp.router_w), b=f32(inp.router_b), wg=bf(L.w_gate),
                wu=bf(L.w_up), wd=bf(L.w_down), sg=bf(L.ws_gate), su=bf(L.ws_up),
                sd=bf(L.ws_down))


def _run(g, K, keys=True, **opts):
    y, r, layer = B.forward(g["x"], g["Wr"], g["b"], g["wg"], g["wu"], g["wd"], g["sg"], g["su"],
                            g["sd"], K=K, routing=True, keys=keys, **opts)
    torch.cuda.synchronize()
    return host_f64(y), gpu_routing_np(r), layer


def _oracle_full(g, K, sel=None, **kw):
    f = {k: (None if v is None else host_f64(v)) for k, v in g.items()}
    return oracle.moe_layer(f["x"], f["Wr"], f["b"], f["wg"], f["wu"], f["wd"], f["sg"], f["su"],
                            f["sd"], K=K, sel=sel, return_parts=True, **kw)


def _check_case(g, K, **opts):
    print(f"case T={g['x'].shape[0]} H={g['x'].shape[1]} E={g['Wr'].shape[0]} K={K} "
          f"I={g['wg'].shape[1]} Is={0 if g['sg'] is None else g['sg'].shape[0]} {opts}", flush=True)
    y, rg, _ = _run(g, K, **opts)
    scale = opts.get("route_scale", 3.0)
    norm = opts.get("norm_topk", True)
    biw = opts.get("bias_in_weights", False)
    okw = dict(scale=scale, norm=norm, bias_in_weights=biw,
               limit=opts.get("swiglu_limit", 0.0), limit_shared=opts.get("swiglu_limit_shared", 0.0))
    ref = _oracle_full(g, K, **okw)
    E = g["Wr"].shape[0]
    check_routing(rg, ref, K, E, host_f64(g["b"]), scale, norm, biw)
    # the oracle on the GPU's selection (identical except for near ties)
    ref2 = _oracle_full(g, K, sel=rg["topk_idx"].astype(np.int64), **okw)
    return check_output(y, ref2["y"])


def _small(seed, T, H, E, K, I, Is, bias_std=0.1, w_std=0.05):
    return _to_gpu_bf16(random_tiny(seed, T, H, E, K, I, Is, bias_std=bias_std, w_std=w_std))


def test_tiny_workload():
    g = _to_gpu_bf16(make_inputs(WORKLOADS["tiny"]))
    _check_case(g, 2)


SMALL = {  # name: (seed, T, H, E, K, I, Is)
    "ragged_nb1_ksplit2": (101, 37, 384, 40, 6, 192, 128),
    "nb2": (102, 100, 256, 8, 2, 128, 64),
    "nb4": (103, 200, 256, 8, 2, 128, 128),
    "lds_block": (104, 300, 256, 8, 2, 128, 128),
    "lds_fallback_nb4": (105, 300, 384, 8, 2, 192, 64),
    "lds_I_ne_Is": (114, 400, 256, 8, 2, 128, 256),
    "no_shared": (106, 50, 256, 16, 4, 64, 0),
    "T1": (107, 1, 256, 16, 4, 64, 64),
    "K1": (108, 40, 256, 16, 1, 64, 64),
    "K_eq_E": (109, 20, 256, 8, 8, 64, 64),
    "E100": (110, 33, 256, 100, 8, 64, 64),
    "E1024_K16": (111, 20, 256, 1024, 16, 64, 64),
    "I_ne_Is": (112, 70, 256, 12, 3, 128, 192),
    "lds_multi_block": (113, 1000, 256, 6, 2, 128, 128),
    "dispatch_blocks_ragged": (115, 1500, 256, 16, 4, 128, 64),
    "dispatch_blocks_E1024": (116, 1300, 256, 1024, 16, 64, 64),
    "wide_router_E100": (117, 1100, 2048, 100, 6, 128, 128),
    # wide router, 8 H splits, E % 4 != 0: its partial sums go out as scalar stores
    "wide_router_E30": (123, 1100, 1024, 30, 3, 64, 64),
    "max_H_lds": (119, 400, 16384, 8, 2, 128, 128),
    "max_I_lds": (120, 400, 256, 8, 2, 16384, 128),
    "max_I_Is_decode": (122, 12, 256, 8, 2, 16384, 16384),
    # H % 512 == 0: 512-row down items, one 512-row pass for blocks of at
    # most 128 rows and two 256-row passes above (shared expert: 175 rows)
    "lds_wide_down": (130, 700, 512, 8, 2, 128, 128),
    # T >= 1024 with T % 4 != 0: the top-K kernel's four-token workgroups end
    # in a part-filled one (three tokens)
    "topk_ragged_T1027": (131, 1027, 512, 20, 4, 64, 64),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_cases(name):
    _check_case(_small(*SMALL[name]), SMALL[name][4])


def test_options_clamp_and_biased_weights():
    g = _small(120, 60, 256, 16, 4, 64, 64, w_std=0.3)
    _check_case(g, 4, swiglu_limit=0.5, swiglu_limit_shared=0.7)
    _check_case(g, 4, bias_in_weights=True)
    _check_case(g, 4, norm_topk=False, route_scale=2.5)


def test_bias_forcing_selects_the_forced_set():
    g = _small(121, 64, 256, 32, 4, 64, 64)
    forced = torch.tensor([3, 9, 17, 30])
    b = torch.zeros(32)
    b[forced] = 10.0
    g["b"] = b.to(DEV)
    y, rg, _ = _run(g, 4)
    assert (rg["topk_idx"] == forced.numpy()[None]).all()
    assert (rg["counts"][forced.numpy()] == 64).all() and rg["counts"].sum() == 256


def test_mixed_single_and_multi_block_groups():
    """One launch with both weight-load kinds: a biased hot expert spans
    several row blocks (ordinary loads, shared through L2) while the other
    experts fit one block each (non-temporal loads); register-streaming
    (16-row blocks) and LDS-pipelined (192-row blocks) kernels."""
    for seed, T, H, E, K, I, Is, hot, bn in ((124, 48, 256, 24, 4, 64, 64, (5, 17), 16),
                                              (125, 1200, 256, 8, 2, 128, 128, (3,), 192)):
        g = _small(seed, T, H, E, K, I, Is)
        b = g["b"].clone()
        b[list(hot)] += 3.0
        g["b"] = b
        counts = _run(g, K)[1]["counts"]
        cold = np.delete(counts, list(hot))
        assert (counts[list(hot)] > bn).all() and ((cold > 0) & (cold <= bn)).any(), counts
        _check_case(g, K)


def test_all_ties_take_lowest_indices():
    g = _small(122, 16, 256, 20, 5, 64, 64, bias_std=0.0)
    g["Wr"] = torch.zeros_like(g["Wr"])
    y, rg, _ = _run(g, 5)
    assert (rg["topk_idx"] == np.arange(5)[None]).all()
    assert np.all(rg["topk_w"] == np.float32(3.0) * np.float32(0.5) / np.float32(2.5))


def _bitwise_twice_and_permuted(g, K, seed=0):
    """Run the layer twice on the same inputs (outputs and routing must be
    bitwise equal), then once on a seeded permutation of the tokens: y(P x)
    must equal P y(x) bit for bit, and each token keep its experts."""
    T = g["x"].shape[0]
    y1, r1, _ = _run(g, K)
    y2, r2, _ = _run(g, K)
    assert np.array_equal(y1, y2), "two runs on the same inputs differ"
    for k in r1:
        assert np.array_equal(r1[k], r2[k]), f"routing {k} differs between two runs"
    p = torch.randperm(T, generator=torch.Generator().manual_seed(seed))
    gp = dict(g, x=g["x"][p.to(g["x"].device)].contiguous())
    y3, r3, _ = _run(gp, K)
    pn = p.numpy()
    assert np.array_equal(y3, y1[pn]), "y(P x) != P y(x)"
    assert np.array_equal(r3["topk_idx"], r1["topk_idx"][pn])
    assert np.array_equal(r3["topk_w"], r1["topk_w"][pn])
    assert np.array_equal(r3["counts"], r1["counts"])
    return r1


@pytest.mark.parametrize("case", [
    # 16 rows per expert: the register-streaming kernels
    (123, 96, 512, 24, 4, 128, 128),
    # 300 rows per expert on average: the LDS-pipelined kernels (192-row
    # blocks of 32-row fragments), experts over several row blocks, ragged
    # last fragments
    (126, 1200, 256, 8, 2, 128, 128),
])
def test_deterministic_and_permutation_equivariant(case):
    print(f"case bitwise {case}", flush=True)
    r = _bitwise_twice_and_permuted(_small(*case), case[4])
    if case[1] == 1200:
        assert (r["counts"] > 192).any(), r["counts"]   # experts over >= 2 row blocks


def test_max_tokens_sampled():
    """T = 2^20, the largest batch the ABI takes (H=256, E=16, K=2, I=Is=128:
    the 256-token router tiles, the three-kernel dispatch over 4096 blocks,
    ~131k rows per expert in the LDS kernels).  Routing is checked on every
    token, the output on 512 sampled rows."""
    T, H, E, K, I, Is = 1 << 20, 256, 16, 2, 128, 128
    print(f"case max tokens T={T} H={H} E={E} K={K} I={I} Is={Is}", flush=True)
    g = _small(121, T, H, E, K, I, Is)
    y, rg, _ = _run(g, K)
    x64 = host_f64(g["x"])
    Wr, b = host_f64(g["Wr"]), host_f64(g["b"])
    check_routing(rg, oracle.route(x64, Wr, b, K), K, E, b)
    rng = np.random.default_rng(121)
    rows = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 510, replace=False)]))
    yref = oracle.moe_layer(x64[rows], Wr, b, host_f64(g["wg"]), host_f64(g["wu"]),
                            host_f64(g["wd"]), host_f64(g["sg"]), host_f64(g["su"]),
                            host_f64(g["sd"]), K=K, sel=rg["topk_idx"].astype(np.int64)[rows])
    res = check_output(y[rows], yref)
    print(f"  rows={len(rows)} max_rel={res[0]:.3e} l2_rel={res[1]:.3e}", flush=True)


# ---------------------------------------------------------------- Flash shape
def _flash(wl_name, T=None):
    inp = make_inputs(WORKLOADS[wl_name], device=DEV, T=T)
    L = inp.layers[0]
    return dict(x=inp.x, Wr=inp.router_w, b=inp.router_b, wg=L.w_gate, wu=L.w_up, wd=L.w_down,
                sg=L.ws_gate, su=L.ws_up, sd=L.ws_down), inp


def _flash_check(wl_name, n_sample=None, T=None):
    g, inp = _flash(wl_name, T)
    K = inp.wl.K
    Tn = g["x"].shape[0]
    print(f"flash case {wl_name} T={Tn}", flush=True)
    y, rg, _ = _run(g, K)
    x64 = host_f64(g["x"])
    Wr, b = host_f64(g["Wr"]), host_f64(g["b"])
    ref_route = oracle.route(x64, Wr, b, K)
    check_routing(rg, ref_route, K, inp.wl.E, b)
    rows = np.arange(Tn)
    if n_sample and n_sample < Tn:
        rng = np.random.default_rng(inp.wl.seed)
        rows = np.unique(np.concatenate([[0, Tn - 1], rng.choice(Tn, n_sample - 2, replace=False)]))
    sel = rg["topk_idx"].astype(np.int64)[rows]
    yref = oracle.moe_layer(x64[rows], Wr, b, LazyStack(g["wg"]), LazyStack(g["wu"]),
                            LazyStack(g["wd"]), host_f64(g["sg"]), host_f64(g["su"]),
                            host_f64(g["sd"]), K=K, sel=sel)
    res = check_output(y[rows], yref)
    print(f"  rows={len(rows)} max_rel={res[0]:.3e} l2_rel={res[1]:.3e}", flush=True)
    return rg


def test_flash_decode_full():
    rg = _flash_check("decode")
    assert rg["counts"].sum() == 16 * 8


def test_flash_decode_bitwise_deterministic_and_permutation_equivariant():
    """The headline decode batch (T = 16, register kernels with their pooled
    tail: which workgroup claims a pooled item varies from run to run), run
    twice (bitwise equal) and once on permuted tokens."""
    g, inp = _flash("decode")
    print("flash case decode: run twice + permuted", flush=True)
    _bitwise_twice_and_permuted(g, inp.wl.K, seed=5)


def test_flash_prefill_full():
    """T = 4096 at the Flash shape (the LDS-pipelined kernels, every expert
    touched, ~114 rows each): routing on every token and the output on all
    4096 rows against the float64 oracle."""
    _flash_check("prefill")


def test_flash_prefill_bitwise_deterministic_and_permutation_equivariant():
    """The full-size prefill in the benchmark's launch configuration, run
    twice (bitwise equal) and once on permuted tokens (y(P x) = P y(x) bit
    for bit)."""
    g, inp = _flash("prefill")
    print("flash case prefill: run twice + permuted", flush=True)
    _bitwise_twice_and_permuted(g, inp.wl.K, seed=3)


def test_flash_skew_sampled():
    rg = _flash_check("skew", n_sample=512)
    from sparse_moe_transformer_fp32_amd.inputs import boosted_experts
    boost = boosted_experts(WORKLOADS["skew"])
    share = rg["counts"][boost].sum() / rg["counts"].sum()
    print(f"  share of slots on the 29 boosted experts: {share:.3f}", flush=True)
    assert share > 0.99


def test_flash_skew_mild_sampled():
    rg = _flash_check("skew_mild", n_sample=512)
    from sparse_moe_transformer_fp32_amd.inputs import boosted_experts
    boost = boosted_experts(WORKLOADS["skew_mild"])
    share = rg["counts"][boost].sum() / rg["counts"].sum()
    print(f"  share of slots on the 29 boosted experts: {share:.3f}", flush=True)
    assert 0.3 < share < 0.8


# ---------------------------------------------------------------- RMSNorm glue
@pytest.mark.parametrize("H", [1152, 9216, 16384])
def test_residual_rmsnorm_matches_oracle(H):
    """H = 1152: a partly filled last wave; above 8192 each thread takes a
    second 8-column chunk (9216: only part of the workgroup)."""
    print(f"residual_rmsnorm H={H}", flush=True)
    gen = torch.Generator().manual_seed(7)
    T = 50
    r = (torch.randn(T, H, generator=gen) * 3).to(torch.bfloat16).to(DEV)
    yv = torch.randn(T, H, generator=gen).to(torch.bfloat16).to(DEV)
    gamma = (torch.randn(H, generator=gen) * 0.1).to(DEV)
    r_out, x_out = B.residual_rmsnorm(r, yv, gamma, eps=1e-6)
    torch.cuda.synchronize()
    r_ref = host_f64(r) + host_f64(yv)
    r_got = host_f64(r_out)
    assert np.abs(r_got - r_ref).max() <= np.abs(r_ref).max() * 2 ** -8
    x_ref = oracle.rmsnorm(r_got, 1e-6, host_f64(gamma))
    check_output(host_f64(x_out), x_ref, "rmsnorm")
    assert np.abs(host_f64(x_out) - x_ref).max() <= np.abs(x_ref).max() * 2 ** -7
    # norm only, in place residual
    _, x2 = B.residual_rmsnorm(r, None, None, eps=1e-6)
    torch.cuda.synchronize()
    check_output(host_f64(x2), oracle.rmsnorm(host_f64(r), 1e-6), "rmsnorm-only")


def test_chain_teacher_forced_small():
    """Three chained small layers; each GPU step is checked against the
    oracle fed the GPU's own input of that step."""
    T, H, E, K, I, Is = 80, 256, 16, 4, 64, 64
    layers = [_small(130 + i, T, H, E, K, I, Is) for i in range(3)]
    r = layers[0]["x"]
    x = None
    for li, g in enumerate(layers):
        _, x = B.residual_rmsnorm(r, None, None, eps=1e-6)
        gx = dict(g, x=x)
        y, rg, _ = _run(gx, K)
        ref = _oracle_full(gx, K, sel=rg["topk_idx"].astype(np.int64))
        check_output(y, ref["y"], f"layer {li}")
        check_output(host_f64(x), oracle.rmsnorm(host_f64(r), 1e-6), f"norm {li}")
        r_new, _ = B.residual_rmsnorm(r, torch.from_numpy(y).to(torch.bfloat16).to(DEV), None,
                                      want_x=False)
        torch.cuda.synchronize()
        check_output(host_f64(r_new), host_f64(r) + y, f"residual {li}")
        r = r_new


# ---------------------------------------------------------------- packing
def test_pack_layout_bit_exact():
    """moe_pack_weights against the layout formula in the header."""
    n, R, C = 3, 48, 96
    w = torch.randn(n, R, C, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    got = B.pack_weights(w.to(DEV)).cpu().view(torch.int16).numpy().reshape(-1)
    src = w.view(torch.int16).numpy()
    want = np.empty(n * R * C, np.int16)
    for m in range(n):
        for row in range(R):
            for col in range(C):
                rt, kt, r, c = row // 16, col // 32, row % 16, col % 32
                off = m * R * C + (rt * (C // 32) + kt) * 512 + 8 * (16 * (c // 8) + r) + c % 8
                want[off] = src[m, row, col]
    assert np.array_equal(got, want)


# ---------------------------------------------------------------- chained layers
def test_flash_long_chain_teacher_forced_sampled():
    """Four chained Flash-shaped layers at T=32768 (the long-context prefill
    chunk): every GPU step is checked against the oracle fed the GPU's own
    input of that step (teacher forcing): the norm on sampled rows, the
    routing bit-exactly on every token (R1) and by the margin rule on sampled
    tokens (R2/R3), the layer output on sampled rows, and the residual add
    on every row."""
    wl = WORKLOADS["long"]
    inp = make_inputs(wl, device=DEV)
    layers = []
    for li, L in enumerate(inp.layers):
        layers.append(B.MoELayer(inp.router_ws[li], inp.router_bs[li], L.w_gate, L.w_up, L.w_down,
                                 L.ws_gate, L.ws_up, L.ws_down, K=wl.K, T_max=wl.T))
    chain = B.MoEChain(layers)
    r_final, trace = chain.forward(inp.x, capture=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    T = wl.T
    rows = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 510, replace=False)]))
    route_rows = np.unique(np.concatenate([rows, rng.choice(T, 1024, replace=False)]))
    for li, (r_l, x_l, rt) in enumerate(trace):
        print(f"layer {li}", flush=True)
        L = inp.layers[li]
        Wr, b = host_f64(inp.router_ws[li]), host_f64(inp.router_bs[li])
        r_rows = host_f64(r_l[torch.as_tensor(route_rows, device=DEV)])
        x_rows = host_f64(x_l[torch.as_tensor(route_rows, device=DEV)])
        check_output(x_rows, oracle.rmsnorm(r_rows, 1e-6), f"norm {li}")
        rg = gpu_routing_np(rt)
        # R1 on every token; R2/R3 on the sampled tokens
        ref = oracle.route(x_rows, Wr, b, wl.K)
        check_routing(rg, ref, wl.K, wl.E, b, tokens=route_rows)
        sel = rg["topk_idx"].astype(np.int64)[rows]
        xs = host_f64(x_l[torch.as_tensor(rows, device=DEV)])
        yref = oracle.moe_layer(xs, Wr, b, LazyStack(L.w_gate), LazyStack(L.w_up),
                                LazyStack(L.w_down), host_f64(L.ws_gate), host_f64(L.ws_up),
                                host_f64(L.ws_down), K=wl.K, sel=sel)
        # the layer output is fused into the residual add: r_{l+1} = r_l + y_l
        r_next = trace[li + 1][0] if li + 1 < len(trace) else r_final
        rs = host_f64(r_l[torch.as_tensor(rows, device=DEV)])
        rn = host_f64(r_next[torch.as_tensor(rows, device=DEV)])
        res = check_output(rn, rs + yref, f"layer {li} residual stream")
        print(f"  rows={len(rows)} max_rel={res[0]:.3e} l2_rel={res[1]:.3e}", flush=True)
        # the layer's contribution alone, within the stream's bf16 rounding
        err = np.abs((rn - rs) - yref)
        assert (err <= 2e-2 * np.abs(yref).max() + np.abs(rn) * 2 ** -8).all(), f"layer {li}"


# ---------------------------------------------------------------- fused residual
FUSED = {  # name: (seed, T, H, E, K, I, Is)
    "nb1": (140, 40, 384, 24, 4, 128, 64),
    "lds": (141, 600, 256, 8, 2, 128, 128),
    "no_shared": (142, 30, 256, 16, 4, 64, 0),
    "wide_h": (143, 24, 9216, 8, 2, 64, 64),   # two column chunks per thread
}


@pytest.mark.parametrize("name", sorted(FUSED))
def test_forward_residual_fused(name):
    """moe_forward_residual: r_out against r_in + the oracle's layer output,
    x_next against the oracle's norm of the GPU's stored r_out, and r_out
    against the unfused GPU path (moe_forward then moe_residual_rmsnorm),
    which rounds once more."""
    seed, T, H, E, K, I, Is = FUSED[name]
    print(f"fused {name}", flush=True)
    g = _small(seed, T, H, E, K, I, Is)
    gen = torch.Generator().manual_seed(seed)
    r_in = (torch.randn(T, H, generator=gen) * 0.5).to(torch.bfloat16).to(DEV)
    gamma = (torch.randn(H, generator=gen) * 0.1).to(DEV)
    layer = B.MoELayer(g["Wr"], g["b"], g["wg"], g["wu"], g["wd"], g["sg"], g["su"], g["sd"], K=K)
    rt = B.alloc_routing(T, E, K, DEV)
    x_next = torch.empty_like(r_in)
    r_out = layer.forward_residual(g["x"], r_in, None, x_next, gamma, 1e-6, rt)
    y = layer.forward(g["x"])
    r_unf, x_unf = B.residual_rmsnorm(r_in, y, gamma, 1e-6)
    torch.cuda.synchronize()
    sel = rt["topk_idx"].cpu().numpy().astype(np.int64)
    ref = _oracle_full(g, K, sel=sel)
    r_ref = host_f64(r_in) + ref["y"]
    check_output(host_f64(r_out), r_ref, f"{name} r_out")
    x_ref = oracle.rmsnorm(host_f64(r_out), 1e-6, host_f64(gamma))
    assert np.abs(host_f64(x_next) - x_ref).max() <= np.abs(x_ref).max() * 2 ** -7
    # against the unfused path: each side rounds r once (half an ulp, at most
    # 2^-8 relative for bf16's 8-bit significand) and the unfused side also
    # rounds y once
    d = np.abs(host_f64(r_out) - host_f64(r_unf))
    bound = (2 * np.abs(host_f64(r_unf)) + np.abs(host_f64(y))) * 2 ** -8 + 1e-30
    assert (d <= bound).all(), f"fused vs unfused off by {(d / bound).max():.2f} of the bound"


def test_forward_residual_in_place():
    """r_out aliasing r_in and x_next aliasing x (how a chain reuses its
    buffers) give the same bits as separate buffers."""
    seed, T, H, E, K, I, Is = FUSED["nb1"]
    g = _small(seed, T, H, E, K, I, Is)
    layer = B.MoELayer(g["Wr"], g["b"], g["wg"], g["wu"], g["wd"], g["sg"], g["su"], g["sd"], K=K)
    r = (torch.randn(T, H, generator=torch.Generator().manual_seed(1)) * 0.5).to(
        torch.bfloat16).to(DEV)
    x = g["x"].clone()
    xn = torch.empty_like(x)
    r_sep = layer.forward_residual(x, r, None, xn)
    r2 = r.clone()
    layer.forward_residual(x, r2, r2, x)
    torch.cuda.synchronize()
    assert torch.equal(r2, r_sep) and torch.equal(x, xn)


# ---------------------------------------------------------------- dense FFN
DENSE = {  # name: (seed, T, H, I, S)
    "nb1_S4": (150, 9, 256, 512, 4),
    "T1_S1": (151, 1, 256, 256, 1),
    "nb4_S2": (152, 60, 384, 256, 2),
    "lds_S4": (153, 300, 512, 1024, 4),
    "lds_ragged_S8": (154, 777, 256, 2048, 8),
    "fallback_S16": (155, 100, 256, 1024, 16),
    # T <= 16 and S <= 8: two-kernel path (slice sum inside the down kernel)
    "two_kernel_T13_S8": (156, 13, 512, 2048, 8),
    "two_kernel_T16_S2": (157, 16, 384, 768, 2),
    # H above 4096: x does not fit in LDS, the one-pair-per-workgroup gate/up
    "two_kernel_T3_H8192_S2": (159, 3, 8192, 256, 2),
    # T <= 16 with S > 8: the row list, the grouped kernels and the combine
    "small_T8_S16": (158, 8, 256, 1024, 16),
}


def _dense_case(x, wg, wu, wd, S, limit=0.0, rows=None):
    ffn = B.DenseFFN(wg, wu, wd, S=S, swiglu_limit=limit)
    y = ffn(x)
    torch.cuda.synchronize()
    sl = slice(None) if rows is None else torch.as_tensor(rows, device=x.device)
    ref = oracle.dense_ffn(host_f64(x[sl]), host_f64(wg), host_f64(wu), host_f64(wd), limit=limit)
    return check_output(host_f64(y[sl]), ref, "dense")


@pytest.mark.parametrize("name", sorted(DENSE))
def test_dense_small(name):
    seed, T, H, I, S = DENSE[name]
    print(f"dense {name}", flush=True)
    gen = torch.Generator().manual_seed(seed)
    x = torch.randn(T, H, generator=gen).to(torch.bfloat16).to(DEV)
    w = [(torch.randn(*s, generator=gen) * 0.05).to(torch.bfloat16).to(DEV)
         for s in ((I, H), (I, H), (H, I))]
    _dense_case(x, *w, S)
    if name == "nb1_S4":
        _dense_case(x, *w, S, limit=0.3)


def test_pack_column_slices_bit_exact():
    R, C, S = 32, 256, 4
    w = torch.randn(R, C, generator=torch.Generator().manual_seed(6)).to(torch.bfloat16)
    got = B.pack_column_slices(w.to(DEV), S).cpu()
    want = torch.stack([B.pack_weights(w[:, s * C // S:(s + 1) * C // S].contiguous().to(DEV)).cpu()
                        for s in range(S)])
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))


@pytest.mark.parametrize("name", ["dense_decode", "dense_prefill"])
def test_dense_flash_shape(name):
    """The model's dense FFN (H=4096, I=11264) with the benchmark's slice
    counts (8 at T=16, 4 at T=4096): every token at T=16, sampled tokens at
    T=4096."""
    from sparse_moe_transformer_fp32_amd.inputs import DENSE_WORKLOADS, make_dense_inputs
    wl = DENSE_WORKLOADS[name]
    x, wg, wu, wd = make_dense_inputs(wl, DEV)
    rows = None if wl.T <= 16 else np.unique(np.concatenate(
        [[0, wl.T - 1], np.random.default_rng(wl.seed).choice(wl.T, 62, replace=False)]))
    res = _dense_case(x, wg, wu, wd, wl.slices, rows=rows)
    print(f"{name}: max_rel={res[0]:.3e} l2_rel={res[1]:.3e}", flush=True)


# ---------------------------------------------------------------- expert statistics
def _stats_case(g, K):
    T, H = g["x"].shape
    E = g["Wr"].shape[0]
    I = g["wg"].shape[1]
    Is = 0 if g["sg"] is None else g["sg"].shape[0]
    layer = B.MoELayer(g["Wr"], g["b"], g["wg"], g["wu"], g["wd"], g["sg"], g["su"], g["sd"], K=K)
    rt = B.alloc_routing(T, E, K, DEV)
    layer.forward(g["x"], routing=rt)
    stats, ratios = layer.expert_stats(T, rt["offsets"])
    stats2, _ = layer.expert_stats(T, rt["offsets"])
    torch.cuda.synchronize()
    assert torch.equal(stats, stats2)                        # deterministic
    st = stats.cpu().numpy().astype(np.float64)
    counts = rt["counts"].cpu().numpy()
    assert np.array_equal(st[:E, 0], counts)
    if Is:
        assert st[E, 0] == T
    # teacher-forced: the oracle's statistics of the GPU's own bf16 h
    lay = B.workspace_layout(T, H, E, K, I, Is)
    hb = layer.workspace()[lay.h:lay.h + (T * K * I + T * Is) * 2].view(torch.bfloat16)
    h = host_f64(hb)
    off = rt["offsets"].cpu().numpy()
    want = [oracle.activation_stats(h[:T * K * I].reshape(T * K, I)[off[e]:off[e + 1]])
            for e in range(E)]
    if Is:
        want.append(oracle.activation_stats(h[T * K * I:].reshape(T, Is)))
    want = np.stack(want)
    assert np.allclose(st, want, rtol=2e-5, atol=1e-6), np.abs(st - want).max()
    rat = ratios.cpu().numpy().astype(np.float64)
    assert np.allclose(rat, oracle.norm_ratios(want[:E]), rtol=2e-5)
    # end to end: the float64 oracle's statistics from the inputs
    sh = (None, None) if g["sg"] is None else (host_f64(g["sg"]), host_f64(g["su"]))
    sel = rt["topk_idx"].cpu().numpy().astype(np.int64)
    ref = oracle.expert_activation_stats(host_f64(g["x"]), sel, LazyStack(g["wg"]),
                                         LazyStack(g["wu"]), *sh, E=E)
    act = ref[:, 0] > 0
    assert np.array_equal(st[:, 0], ref[:, 0])
    for c in (1, 2, 3):
        rel = np.abs(st[act, c] - ref[act, c]) / np.abs(ref[act, c])
        assert rel.max() < 5e-3, (c, rel.max())
    assert np.allclose(rat, oracle.norm_ratios(ref[:E]), rtol=5e-3)
    return rat


def test_expert_stats_small():
    _stats_case(_small(160, 90, 256, 24, 4, 128, 64), 4)
    _stats_case(_small(161, 40, 256, 64, 2, 64, 0), 2)    # idle experts, no shared


def test_expert_stats_blow_up_shows_in_ratio():
    """One expert's up projection scaled by 8: its mean norm grows 8x, and so
    does the max-to-median ratio."""
    g = _small(162, 256, 256, 8, 8, 64, 64)             # K = E: every expert sees every token
    base = _stats_case(g, 8)
    g["wu"] = g["wu"].clone()
    g["wu"][5] = (g["wu"][5].float() * 8).to(torch.bfloat16)
    big = _stats_case(g, 8)
    assert big[0] > 5 * base[0]


def test_expert_stats_flash_decode():
    g, _ = _flash("decode")
    _stats_case(g, 8)


# ---------------------------------------------------------------- per-kernel intermediates
@pytest.mark.parametrize("name", ["ragged_nb1_ksplit2", "nb2", "lds_block", "lds_I_ne_Is",
                                  "lds_wide_down"])
def test_gate_up_and_down_intermediates(name):
    """The two grouped GEMMs on their own: h (SwiGLU output, expert-contiguous
    rows, then the shared rows) and o (each row already times its routing
    weight) read from the workspace, against the oracle's per-row values for
    the GPU's own routing."""
    seed, T, H, E, K, I, Is = SMALL[name]
    g = _small(seed, T, H, E, K, I, Is)
    layer = B.MoELayer(g["Wr"], g["b"], g["wg"], g["wu"], g["wd"], g["sg"], g["su"], g["sd"], K=K)
    rt = B.alloc_routing(T, E, K, DEV)
    layer.forward(g["x"], routing=rt)
    torch.cuda.synchronize()
    lay = B.workspace_layout(T, H, E, K, I, Is)
    ws = layer.workspace()
    KT = T * K
    h = host_f64(ws[lay.h:lay.h + (KT * I + T * Is) * 2].view(torch.bfloat16))
    rows = KT + (T if Is else 0)
    o = host_f64(ws[lay.o:lay.o + rows * H * 2].view(torch.bfloat16)).reshape(rows, H)
    f = {k: (None if v is None else host_f64(v)) for k, v in g.items()}
    perm = rt["perm_token"].cpu().numpy()
    off = rt["offsets"].cpu().numpy()
    sel = rt["topk_idx"].cpu().numpy()
    w = rt["topk_w"].cpu().numpy().astype(np.float64)
    slot = rt["slot_pos"].cpu().numpy()
    h_ref = np.zeros((KT, I))
    o_ref = np.zeros((KT, H))
    for e in range(E):
        r = np.arange(off[e], off[e + 1])
        if r.size == 0:
            continue
        oe, he = oracle.swiglu_ffn(f["x"][perm[r]], f["wg"][e], f["wu"][e], f["wd"][e],
                                   return_hidden=True)
        h_ref[r], o_ref[r] = he, oe
    # weight of each routed row: the slot that points at it
    row_w = np.zeros(KT)
    row_w[slot.reshape(-1)] = w.reshape(-1)
    o_ref *= row_w[:, None]
    check_output(h[:KT * I].reshape(KT, I), h_ref, f"{name} h routed")
    check_output(o[:KT], o_ref, f"{name} o routed")
    if Is:
        os_, hs = oracle.swiglu_ffn(f["x"], f["sg"], f["su"], f["sd"], return_hidden=True)
        check_output(h[KT * I:].reshape(T, Is), hs, f"{name} h shared")
        check_output(o[KT:], os_, f"{name} o shared")
    assert np.array_equal(np.sort(perm[off[0]:off[E]]), np.sort(np.repeat(np.arange(T), K)))


# ---------------------------------------------------------------- HIP graph capture
@pytest.mark.parametrize("name", ["ragged_nb1_ksplit2", "lds_block"])
def test_hip_graph_capture_replays_bitwise(name):
    """The layer allocates, synchronises and clears nothing, so one call can be
    captured in a HIP graph.  Three replays, with eager calls on other data
    in between, each reproduce the eager result bit for bit (output and
    routing); the fused residual entry point is captured in the same graph."""
    seed, T, H, E, K, I, Is = SMALL[name]
    g = _small(seed, T, H, E, K, I, Is)
    layer = B.MoELayer(g["Wr"], g["b"], g["wg"], g["wu"], g["wd"], g["sg"], g["su"], g["sd"], K=K,
                       T_max=T)
    x = g["x"]
    y = torch.empty_like(x)
    rt = B.alloc_routing(T, E, K, DEV)
    r_in = (torch.randn(T, H, generator=torch.Generator().manual_seed(seed)) * 0.5).to(
        torch.bfloat16).to(DEV)
    r_out = torch.empty_like(r_in)
    xn = torch.empty_like(r_in)
    layer.forward(x, y, rt)
    layer.forward_residual(x, r_in, r_out, xn)
    torch.cuda.synchronize()
    want = (y.clone(), {k: v.clone() for k, v in rt.items()}, r_out.clone(), xn.clone())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.forward(x, y, rt)
        layer.forward_residual(x, r_in, r_out, xn)
    x_other = torch.randn(T, H, generator=torch.Generator().manual_seed(seed + 1)).to(
        torch.bfloat16).to(DEV)
    y_other = torch.empty_like(x)
    for rep in range(3):
        for t_ in (y, r_out, xn, *rt.values()):
            t_.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, want[0]), f"replay {rep}: y"
        for k in rt:
            assert torch.equal(rt[k], want[1][k]), f"replay {rep}: {k}"
        assert torch.equal(r_out, want[2]) and torch.equal(xn, want[3]), f"replay {rep}: residual"
        layer.forward(x_other, y_other)     # eager work between replays
        torch.cuda.synchronize()


def test_empty_batch_through_every_entry_point():
    """T = 0: moe_route and a routing output receive all-zero counts and
    offsets (over a garbage prefill); the layer, the fused residual path, the
    dense FFN and the residual norm write nothing and return MOE_OK."""
    print("case empty batch T=0", flush=True)
    g = _small(118, 4, 256, 16, 4, 64, 64)
    E, K, H = 16, 4, 256
    x0 = g["x"][:0]
    r = B.route(x0, g["Wr"], g["b"], K, I=64, Is=64)
    torch.cuda.synchronize()
    ref = oracle.route(host_f64(x0).reshape(0, H), host_f64(g["Wr"]), host_f64(g["b"]), K)
    assert r["topk_idx"].shape == ref["topk_idx"].shape == (0, K)
    assert np.array_equal(r["counts"].cpu().numpy(), ref["counts"])
    assert np.array_equal(r["offsets"].cpu().numpy(), ref["offsets"])
    out = B.alloc_routing(0, E, K, DEV)
    out["counts"].fill_(7)
    out["offsets"].fill_(-3)
    B.route(x0, g["Wr"], g["b"], K, I=64, Is=64, out=out)
    torch.cuda.synchronize()
    assert (out["counts"].cpu() == 0).all() and (out["offsets"].cpu() == 0).all()

    layer = B.MoELayer(g["Wr"], g["b"], g["wg"], g["wu"], g["wd"], g["sg"], g["su"], g["sd"], K=K)
    rt = B.alloc_routing(0, E, K, DEV)
    rt["counts"].fill_(5)
    rt["offsets"].fill_(5)
    y = layer.forward(x0, routing=rt)
    torch.cuda.synchronize()
    assert y.shape == (0, H)
    assert (rt["counts"].cpu() == 0).all() and (rt["offsets"].cpu() == 0).all()
    r_out = layer.forward_residual(x0, torch.empty((0, H), dtype=torch.bfloat16, device=DEV))
    assert r_out.shape == (0, H)
    # a non-empty call after the empty ones is unaffected
    _check_case(g, K)

    dense = B.DenseFFN(g["wg"][0], g["wu"][0], g["wd"][0], S=1)
    assert dense.forward(x0).shape == (0, H)
    ro, xo = B.residual_rmsnorm(torch.empty((0, H), dtype=torch.bfloat16, device=DEV),
                                torch.empty((0, H), dtype=torch.bfloat16, device=DEV))
    torch.cuda.synchronize()
    assert ro.shape == (0, H) and xo.shape == (0, H)


def test_read_probe_reads_without_writing():
    """The HBM read-ceiling probe runs both load kinds over a buffer and
    leaves its sink untouched (its write condition never holds)."""
    buf = torch.ones(64 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(16, dtype=torch.uint8, device="cuda")
    for nt in (False, True):
        B.read_probe(buf, sink, nt)
    torch.cuda.synchronize()
    assert int(sink.sum()) == 0


def test_mfma_probe_runs_on_every_cu():
    """The matrix-core ceiling probe: every CU's workgroup reports its loop's
    shader-clock and real-time counts, the clock they give lies in a
    physical range, and the sink is untouched."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    clocks = torch.zeros(2 * cus, dtype=torch.int64, device="cuda")
    sink = torch.zeros(4, dtype=torch.float32, device="cuda")
    B.mfma_probe(4096, clocks, sink)
    torch.cuda.synchronize()
    c = clocks.view(cus, 2).cpu().numpy().astype(np.float64)
    assert (c > 0).all(), c
    ghz = c[:, 0].sum() / c[:, 1].sum() * 0.1
    print(f"mfma probe: {cus} CUs, clock {ghz:.3f} GHz", flush=True)
    assert 0.3 < ghz < 3.5, ghz
    assert float(sink.abs().sum()) == 0.0
