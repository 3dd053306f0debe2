"""Helpers for comparing the HIP path with the CPU oracle.

Tolerances for the bf16 output: max|y - y_ref| <= 2e-2 max|y_ref| and
||y - y_ref||_2 / ||y_ref||_2 <= 5e-3 against the float64 oracle.
Routing: the discrete stage must match bit for bit on the GPU's own fp32 keys
(R1); against the float64 keys the selected sets must match wherever the gap
between the K-th and (K+1)-th key is >= DELTA (R2); closer tokens must pick a
set whose keys are within DELTA of the best (R3).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from sparse_moe_transformer_fp32_amd.inputs import bf16_bits

DELTA = 1e-5
MAX_REL = 2e-2
L2_REL = 5e-3
W_RTOL = 1e-6


def host_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a tensor's values on the host."""
    if t.dtype == torch.bfloat16:
        return oracle.bf16_bits_to_f64(bf16_bits(t)).reshape(tuple(t.shape))
    return t.detach().cpu().numpy().astype(np.float64)


class LazyStack:
    """Expert-indexed float64 view of a [E, r, c] bf16 device stack, copied
    to the host one expert at a time."""

    def __init__(self, t: torch.Tensor):
        self.t = t

    def __getitem__(self, e):
        return host_f64(self.t[int(e)])


def check_output(y_gpu: np.ndarray, y_ref: np.ndarray, what: str = "y"):
    err = np.abs(y_gpu - y_ref)
    ref_max = np.abs(y_ref).max()
    rel_max = err.max() / ref_max
    rel_l2 = np.linalg.norm(y_gpu - y_ref) / np.linalg.norm(y_ref)
    assert rel_max <= MAX_REL, f"{what}: max|err|/max|ref| = {rel_max:.3e} > {MAX_REL}"
    assert rel_l2 <= L2_REL, f"{what}: rel L2 = {rel_l2:.3e} > {L2_REL}"
    return rel_max, rel_l2


def gpu_routing_np(r: dict) -> dict:
    return {k: v.detach().cpu().numpy() for k, v in r.items()}


def check_routing(rg: dict, ref: dict, K: int, E: int, bias: np.ndarray, scale=3.0, norm=True,
                  biw=False, tokens=None):
    """rg: GPU routing (numpy, with keys and scores); ref: oracle.route output
    (float64) for the same tokens (or for `tokens` of them).  Returns the
    near-tie token indices."""
    sel_g = rg["topk_idx"].astype(np.int64)
    T = sel_g.shape[0]
    # R1: discrete stage on the GPU's own fp32 keys, every token
    sel_r1 = oracle.select_topk(rg["keys"], K)
    bad = np.nonzero((sel_r1 != sel_g).any(axis=1))[0]
    assert bad.size == 0, f"R1 selection differs on tokens {bad[:10]}"
    d = oracle.dispatch(sel_g, E)
    for name in ("counts", "offsets", "perm_token", "slot_pos"):
        got = rg[name].astype(np.int64).reshape(d[name].shape)
        assert np.array_equal(got, d[name]), f"R1 {name} differs"
    w_r1 = oracle.routing_weights(rg["scores"].astype(np.float64), sel_g, scale, norm, bias, biw)
    wd = np.abs(rg["topk_w"].astype(np.float64) - w_r1) / np.abs(w_r1)
    assert wd.max() <= W_RTOL, f"R1 topk_w rel err {wd.max():.3e}"
    if norm:
        assert np.allclose(rg["topk_w"].sum(axis=1), scale, rtol=0, atol=1e-5)
    # keys: fp32 vs float64
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    keys64 = ref["keys"]
    kerr = np.abs(rg["keys"][tok].astype(np.float64) - keys64).max()
    assert kerr < DELTA / 4, f"fp32 keys off by {kerr:.3e}"
    # R2 / R3 against the float64 keys
    near = []
    if K < E:
        srt = -np.sort(-keys64, axis=1)
        gap = srt[:, K - 1] - srt[:, K]
        sel64 = ref["topk_idx"]
        for i, t in enumerate(tok):
            if gap[i] >= DELTA:
                assert np.array_equal(sel_g[t], sel64[i]), f"R2: token {t} set differs"
            else:
                near.append(t)
                inset = np.zeros(E, bool)
                inset[sel_g[t]] = True
                assert keys64[i][inset].min() >= keys64[i][~inset].max() - DELTA, f"R3 token {t}"
    return near
