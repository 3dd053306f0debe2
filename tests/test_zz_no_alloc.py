"""moe_forward_noalloc (the layer with the library's fixed scratch array
instead of a caller workspace) against moe_forward, through the C-ABI.

Two calls in a row on each shape, the second with fewer tokens: the fixed
array keeps the first call's contents, and the second call must not depend
on them.  Outputs and routing must be bit-identical to moe_forward's (the
same kernels and launch plan, another scratch address).
"""
import numpy as np
import pytest
import torch

from sparse_moe_transformer_fp32_amd import binding as B
from sparse_moe_transformer_fp32_amd.inputs import WORKLOADS, make_inputs, random_tiny

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _layer_small(seed, T, H, E, K, I, Is):
    inp = random_tiny(seed, T, H, E, K, I, Is, w_std=0.05)
    L = inp.layers[0]
    bf = lambda t: t.to(torch.bfloat16).to(DEV).contiguous()
    layer = B.MoELayer(inp.router_w.to(DEV), inp.router_b.to(DEV), bf(L.w_gate), bf(L.w_up),
                       bf(L.w_down), bf(L.ws_gate), bf(L.ws_up), bf(L.ws_down), K=K)
    return layer, bf(inp.x)


def _layer_flash(T):
    inp = make_inputs(WORKLOADS["decode"], device=DEV, T=T)
    L = inp.layers[0]
    layer = B.MoELayer(inp.router_w, inp.router_b, L.w_gate, L.w_up, L.w_down, L.ws_gate,
                       L.ws_up, L.ws_down, K=inp.wl.K)
    return layer, inp.x


def _compare(layer, x, T):
    xs = x[:T].contiguous()
    r_ref = B.alloc_routing(T, layer.E, layer.K, DEV)
    r_new = B.alloc_routing(T, layer.E, layer.K, DEV)
    y_ref = layer.forward(xs, routing=r_ref)
    y_new = torch.full_like(xs, 7.0)
    layer.forward_noalloc(xs, y_new, routing=r_new)
    torch.cuda.synchronize()
    assert torch.equal(y_new.view(torch.int16), y_ref.view(torch.int16)), "y differs"
    for k in r_ref:
        assert torch.equal(r_new[k], r_ref[k]), f"routing {k} differs"
    # and without a routing output (the routing then lives in the scratch)
    y_new2 = torch.full_like(xs, -3.0)
    layer.forward_noalloc(xs, y_new2)
    torch.cuda.synchronize()
    assert torch.equal(y_new2.view(torch.int16), y_ref.view(torch.int16)), "y differs (no routing)"


@pytest.mark.parametrize("case", [
    # LDS-pipelined GEMMs (192-row blocks), then a smaller register-kernel batch
    ("small", (131, 600, 256, 8, 2, 128, 128), 600, 40),
    # the Flash decode shape: 64 tokens, then the 16-token decode batch
    ("flash", None, 64, 16),
])
def test_noalloc_matches_moe_forward_two_calls(case):
    name, shape, T1, T2 = case
    print(f"noalloc case {name} T={T1} then T={T2}", flush=True)
    if name == "small":
        layer, x = _layer_small(*shape)
    else:
        layer, x = _layer_flash(T1)
    _compare(layer, x, T1)
    _compare(layer, x, T2)


def test_noalloc_refuses_layers_beyond_its_scratch():
    """Above the fixed size the call is refused on the host with
    MOE_ERR_WORKSPACE; a following call that fits still works."""
    layer, x = _layer_small(132, 64, 256, 8, 2, 128, 128)
    T = 1
    while B.workspace_bytes(T, 4096, 288, 8, 1280, 1280) <= B.NOALLOC_SCRATCH_BYTES:
        T += 1
    big = B.MoELayer.__new__(B.MoELayer)
    big.__dict__.update(layer.__dict__)
    big.H, big.E, big.K, big.I, big.Is = 4096, 288, 8, 1280, 1280
    xb = torch.zeros((T, 4096), dtype=torch.bfloat16, device=DEV)
    yb = torch.empty_like(xb)
    with pytest.raises(B.MoEError) as ei:
        big.forward_noalloc(xb, yb)
    assert ei.value.status == B.MOE_ERR_WORKSPACE
    assert "moe_forward" in str(ei.value)
    _compare(layer, x, 64)
