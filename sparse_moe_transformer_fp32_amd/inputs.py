"""Seeded synthetic inputs for the MoE FFN layer.

This module is shared by the CPU oracle's tests and by the HIP path (tests,
bench, smoke).  It only draws random numbers and shapes them into the
distributions the workloads call for; it holds none of the layer's own
arithmetic (no router, no selection, no expert FFN, no combine).

Workloads (sizes from the Step-3.5-Flash model card's raw config table:
hidden_size 4096, moe_num_experts 288, moe_top_k 8, moe_intermediate_size
1280, share_expert_dim 1280; torch_dtype bfloat16):

  tiny     T=64,    H=256,  E=16,  K=2, I=Is=64, fp32 draws, b ~ N(0, 0.1)
  decode   T=16,    Flash shape, b = 0, x rows scaled to unit RMS
  prefill  T=4096,  Flash shape, b = 0 (near-uniform routing)
  skew     T=8192,  Flash shape, b = +2.0 on 29 seeded experts
  skew_mild T=8192, Flash shape, b = +0.15 on the same 29 experts
  long     T=32768, Flash shape, 4 layers with their own weights

Draw order from one torch.Generator seeded once per workload:
x, Wr, b (when random), then per layer Wg, Wu, Wd (expert by expert), then
Wg_s, Wu_s, Wd_s.  Every tensor is drawn in float32, scaled, then cast once
(bf16 for x and the expert weights; the router weight and bias stay fp32).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    E: int
    K: int
    I: int
    Is: int
    seed: int
    w_std: float = 0.02          # expert and router weight std
    bias_std: float = 0.0        # > 0: b ~ N(0, bias_std)
    bias_boost: float = 0.0      # added to b on `n_boost` seeded experts
    n_boost: int = 0
    unit_rms_x: bool = True      # scale each x row to unit RMS
    layers: int = 1
    fp32_draws: bool = False     # tiny workload: fp32 x and expert weights
    route_scale: float = 3.0     # moe_router_scaling_factor
    norm_topk: bool = True       # norm_expert_weight

    @property
    def has_shared(self) -> bool:
        return self.Is > 0


FLASH = dict(H=4096, E=288, K=8, I=1280, Is=1280)

WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", T=64, H=256, E=16, K=2, I=64, Is=64, seed=1,
                     bias_std=0.1, unit_rms_x=False, fp32_draws=True),
    "decode": Workload("decode", T=16, seed=2, **FLASH),
    "prefill": Workload("prefill", T=4096, seed=3, **FLASH),
    "skew": Workload("skew", T=8192, seed=4, bias_boost=2.0, n_boost=29, **FLASH),
    "skew_mild": Workload("skew_mild", T=8192, seed=4, bias_boost=0.15, n_boost=29,
                          **FLASH),
    "long": Workload("long", T=32768, seed=5, layers=4, **FLASH),
}


def boosted_experts(wl: Workload) -> np.ndarray:
    """The seeded set of experts whose router bias is raised (skew workloads)."""
    if wl.n_boost == 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(np.random.default_rng(wl.seed).choice(wl.E, wl.n_boost, replace=False))


def _normal(gen: torch.Generator, shape, std: float, device) -> torch.Tensor:
    t = torch.randn(shape, generator=gen, dtype=torch.float32, device=device)
    if std != 1.0:
        t.mul_(std)
    return t


def _unit_rms_rows(z: torch.Tensor) -> torch.Tensor:
    # Input recipe only: "x ~ N(0,1), RMS-normalised" means each row of the
    # draw is divided by its root-mean-square (1e-6 floor) before the cast.
    return z / torch.sqrt(z.pow(2).mean(dim=1, keepdim=True) + 1e-6)


@dataclasses.dataclass
class LayerWeights:
    w_gate: torch.Tensor   # [E, I, H]
    w_up: torch.Tensor     # [E, I, H]
    w_down: torch.Tensor   # [E, H, I]
    ws_gate: Optional[torch.Tensor]  # [Is, H]
    ws_up: Optional[torch.Tensor]    # [Is, H]
    ws_down: Optional[torch.Tensor]  # [H, Is]


@dataclasses.dataclass
class Inputs:
    wl: Workload
    x: torch.Tensor               # [T, H]  bf16 (fp32 for fp32 draws)
    router_w: torch.Tensor        # [E, H]  fp32
    router_b: torch.Tensor        # [E]     fp32
    layers: List[LayerWeights]
    router_ws: List[torch.Tensor] = dataclasses.field(default_factory=list)
    router_bs: List[torch.Tensor] = dataclasses.field(default_factory=list)


def _expert_stack(gen, E, rows, cols, std, device, dtype) -> torch.Tensor:
    out = torch.empty((E, rows, cols), dtype=dtype, device=device)
    for e in range(E):
        out[e] = _normal(gen, (rows, cols), std, device).to(dtype)
    return out


def make_inputs(wl: Workload, device: str = "cpu", T: Optional[int] = None,
                layers: Optional[int] = None) -> Inputs:
    """Draw one workload's inputs.  `T` and `layers` override the sizes
    (used for reduced-size cases of the same recipe)."""
    T = wl.T if T is None else T
    L = wl.layers if layers is None else layers
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.seed)
    wdtype = torch.float32 if wl.fp32_draws else torch.bfloat16

    z = _normal(gen, (T, wl.H), 1.0, dev)
    if wl.unit_rms_x:
        z = _unit_rms_rows(z)
    x = z.to(wdtype)

    def router():
        w = _normal(gen, (wl.E, wl.H), wl.w_std, dev)
        if wl.bias_std > 0:
            b = _normal(gen, (wl.E,), wl.bias_std, dev)
        else:
            b = torch.zeros(wl.E, dtype=torch.float32, device=dev)
        if wl.n_boost:
            idx = torch.as_tensor(boosted_experts(wl), device=dev)
            b[idx] += wl.bias_boost
        return w, b

    rw, rb = router()
    router_ws, router_bs = [rw], [rb]
    layer_list = []
    for li in range(L):
        if li > 0:
            w, b = router()
            router_ws.append(w)
            router_bs.append(b)
        wg = _expert_stack(gen, wl.E, wl.I, wl.H, wl.w_std, dev, wdtype)
        wu = _expert_stack(gen, wl.E, wl.I, wl.H, wl.w_std, dev, wdtype)
        wd = _expert_stack(gen, wl.E, wl.H, wl.I, wl.w_std, dev, wdtype)
        if wl.has_shared:
            sg = _normal(gen, (wl.Is, wl.H), wl.w_std, dev).to(wdtype)
            su = _normal(gen, (wl.Is, wl.H), wl.w_std, dev).to(wdtype)
            sd = _normal(gen, (wl.H, wl.Is), wl.w_std, dev).to(wdtype)
        else:
            sg = su = sd = None
        layer_list.append(LayerWeights(wg, wu, wd, sg, su, sd))
    return Inputs(wl, x, rw, rb, layer_list, router_ws, router_bs)


@dataclasses.dataclass(frozen=True)
class DenseWorkload:
    """A dense gated FFN of the model's first layers (model card:
    intermediate_size 11264; 3 dense of 45 layers)."""
    name: str
    T: int
    H: int
    I: int
    seed: int
    w_std: float = 0.02
    slices: int = 8


DENSE_WORKLOADS: Dict[str, DenseWorkload] = {
    "dense_decode": DenseWorkload("dense_decode", T=16, H=4096, I=11264, seed=6),
    # 4 slices of 2816 at T = 4096 (1.15 ms against 1.19 ms with 8 slices);
    # 8 of 1408 at T = 16, where they give more workgroups
    "dense_prefill": DenseWorkload("dense_prefill", T=4096, H=4096, I=11264, seed=7, slices=4),
}


def make_dense_inputs(wl: DenseWorkload, device: str = "cpu", T: Optional[int] = None,
                      seed: Optional[int] = None):
    """x [T,H] bf16 (rows at unit RMS), Wg, Wu [I,H] and Wd [H,I] bf16 from
    one generator seeded once (with the workload's seed unless `seed` is
    given), drawn in that order."""
    T = wl.T if T is None else T
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.seed if seed is None else seed)
    x = _unit_rms_rows(_normal(gen, (T, wl.H), 1.0, dev)).to(torch.bfloat16)
    wg = _normal(gen, (wl.I, wl.H), wl.w_std, dev).to(torch.bfloat16)
    wu = _normal(gen, (wl.I, wl.H), wl.w_std, dev).to(torch.bfloat16)
    wd = _normal(gen, (wl.H, wl.I), wl.w_std, dev).to(torch.bfloat16)
    return x, wg, wu, wd


def random_tiny(seed: int, T: int, H: int, E: int, K: int, I: int, Is: int,
                bias_std: float = 0.1, w_std: float = 0.2) -> Inputs:
    """Small random fp32 case for property tests (CPU generator)."""
    wl = Workload(f"rand{seed}", T=T, H=H, E=E, K=K, I=I, Is=Is, seed=seed,
                  w_std=w_std, bias_std=bias_std, unit_rms_x=False, fp32_draws=True)
    return make_inputs(wl, "cpu")


def to_bf16(t: torch.Tensor) -> torch.Tensor:
    """Round-to-nearest-even cast (what the bf16 path receives)."""
    return t.to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """The raw uint16 bit patterns of a bf16 tensor, on the host."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
