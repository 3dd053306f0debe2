"""Planted mistakes in the oracle must be caught by the pins (CPU only).

Each case monkeypatches one oracle function with a plausible bug (a dropped
term, a wrong sign or index, a transposed operand, a wrong reading) and checks
that the pin suite below no longer passes."""
import numpy as np
import pytest

import oracle
import oracle.moe_oracle as M
from tests import test_oracle_pins as P


def _pins_pass():
    checks = [
        P.test_p1_tiny_workload_matches_brute_force,
        lambda: [P.test_p1_random_tiny_matches_brute_force(s) for s in P.TINY_SHAPES],
        lambda: [P.test_p2_p3_weights_and_dispatch(s) for s in P.TINY_SHAPES],
        P.test_p5_identical_experts_closed_form,
        P.test_p6_k1_and_k_equals_e,
        P.test_p7_bias_forcing_and_reading,
        P.test_ties_go_to_lower_index,
        P.test_p8_routed_and_shared_halves,
        P.test_p9_single_row_textbook,
        P.test_rmsnorm_closed_forms,
        P.test_chain_closed_forms,
        P.test_swiglu_limit_closed_forms,
        P.test_dense_ffn_textbook,
        P.test_activation_stats_hand_computed,
        P.test_norm_ratios_hand_computed,
        lambda: [P.test_expert_stats_brute_force(s) for s in P.TINY_SHAPES],
        P.test_norm_ratios_closed_forms,
    ]
    for c in checks:
        try:
            c()
        except (AssertionError, ValueError, IndexError):
            return False
    return True


def test_unmutated_oracle_passes():
    assert _pins_pass()


def _silu_as_sigmoid(z):
    return 1.0 / (1.0 + np.exp(-np.asarray(z, np.float64)))


def _scores_wrong_sign(l):
    return 1.0 / (1.0 + np.exp(np.asarray(l, np.float64)))


def _keys_no_bias(s, b):
    return np.asarray(s, np.float64)


def _keys_bias_before_sigmoid_like(s, b):
    return np.asarray(s, np.float64) + 0.5 * np.asarray(b, np.float64)[None, :]


def _ties_to_higher(keys, K):
    keys = np.asarray(keys, np.float64)
    T, E = keys.shape
    out = np.empty((T, K), np.int64)
    for t in range(T):
        order = np.lexsort((-np.arange(E), -keys[t]))
        out[t] = np.sort(order[:K])
    return out


_orig_rw = M.routing_weights
_orig_ffn = M.swiglu_ffn
_orig_dispatch = M.dispatch
_orig_rms = M.rmsnorm
_orig_logits = M.router_logits


def _weights_scale1(s, sel, scale=3.0, norm=True, bias=None, bias_in_weights=False):
    return _orig_rw(s, sel, 1.0, norm, bias, bias_in_weights)


def _weights_unnormalised(s, sel, scale=3.0, norm=True, bias=None, bias_in_weights=False):
    return _orig_rw(s, sel, scale, False, bias, bias_in_weights)


def _weights_from_biased(s, sel, scale=3.0, norm=True, bias=None, bias_in_weights=False):
    return _orig_rw(s, sel, scale, norm, bias, True)


def _ffn_down_transposed(xr, Wg, Wu, Wd, return_hidden=False, **kw):
    Wd = np.asarray(Wd)
    if Wd.shape[0] == Wd.shape[1]:
        Wd = Wd.T
    else:
        raise ValueError("shape mismatch from the transposed operand")
    return _orig_ffn(xr, Wg, Wu, Wd, return_hidden, **kw)


def _ffn_gate_up_swapped(xr, Wg, Wu, Wd, return_hidden=False, **kw):
    return _orig_ffn(xr, Wu, Wg, Wd, return_hidden, **kw)


def _ffn_clamp_both_sides(xr, Wg, Wu, Wd, return_hidden=False, limit=0.0):
    if limit <= 0:
        return _orig_ffn(xr, Wg, Wu, Wd, return_hidden)
    xr = np.asarray(xr, np.float64)
    g = np.clip(xr @ np.asarray(Wg, np.float64).T, -limit, limit)
    u = np.clip(xr @ np.asarray(Wu, np.float64).T, -limit, limit)
    h = g / (1.0 + np.exp(-g)) * u
    o = h @ np.asarray(Wd, np.float64).T
    return (o, h) if return_hidden else o


def _dispatch_descending_rows(sel, E):
    d = _orig_dispatch(sel, E)
    off, perm = d["offsets"], d["perm_token"].copy()
    pos = d["slot_pos"].copy()
    for e in range(E):
        a, b = off[e], off[e + 1]
        perm[a:b] = perm[a:b][::-1]
    T, K = pos.shape
    for t in range(T):
        for j in range(K):
            r = pos[t, j]
            e = np.searchsorted(off, r, side="right") - 1
            pos[t, j] = off[e] + off[e + 1] - 1 - r
    return dict(d, perm_token=perm, slot_pos=pos)


def _rms_no_eps_mean_abs(v, eps=1e-6, gamma=None):
    v = np.asarray(v, np.float64)
    return v / np.mean(np.abs(v), axis=-1, keepdims=True)


def _rms_gain_not_centred(v, eps=1e-6, gamma=None):
    g = None if gamma is None else np.asarray(gamma) - 1.0
    return _orig_rms(v, eps, g)


def _logits_transposed_router(x, Wr):
    x = np.asarray(x, np.float64)
    Wr = np.asarray(Wr, np.float64)
    return x @ Wr[::-1].T


_orig_hidden = M.swiglu_hidden
_orig_stats = M.activation_stats


def _stats_mean_square_as_norm(h):
    h = np.asarray(h, np.float64)
    if h.shape[0] == 0:
        return np.zeros(4)
    n = np.mean(h * h, axis=1)
    return np.array([h.shape[0], n.sum(), np.sum(n * n), n.max()])


def _ratios_lower_median(stats):
    st = np.asarray(stats, np.float64)
    act = st[:, 0] > 0
    m = np.sort(st[act, 1] / st[act, 0])
    med = m[(len(m) - 1) // 2]
    return np.array([m.max() / med, m.min() / med])


def _ratios_include_empty(stats):
    st = np.asarray(stats, np.float64)
    m = st[:, 1] / np.maximum(st[:, 0], 1)
    med = np.median(m)
    return np.array([m.max() / med, m.min() / med])


def _hidden_gate_only(xr, Wg, Wu, limit=0.0):
    g = np.asarray(xr, np.float64) @ np.asarray(Wg, np.float64).T
    return g / (1.0 + np.exp(-g))


MUTATIONS = {
    "stats_mean_square_as_norm": ("activation_stats", _stats_mean_square_as_norm),
    "ratio_lower_median": ("norm_ratios", _ratios_lower_median),
    "ratio_counts_empty_experts": ("norm_ratios", _ratios_include_empty),
    "hidden_drops_up_branch": ("swiglu_hidden", _hidden_gate_only),
    "silu_is_sigmoid": ("silu", _silu_as_sigmoid),
    "sigmoid_wrong_sign": ("router_scores", _scores_wrong_sign),
    "bias_dropped": ("selection_keys", _keys_no_bias),
    "bias_halved": ("selection_keys", _keys_bias_before_sigmoid_like),
    "ties_to_higher_index": ("select_topk", _ties_to_higher),
    "scale_dropped": ("routing_weights", _weights_scale1),
    "normalisation_dropped": ("routing_weights", _weights_unnormalised),
    "weights_from_biased_keys": ("routing_weights", _weights_from_biased),
    "down_transposed": ("swiglu_ffn", _ffn_down_transposed),
    "gate_up_swapped": ("swiglu_ffn", _ffn_gate_up_swapped),
    "rows_descending": ("dispatch", _dispatch_descending_rows),
    "rmsnorm_wrong": ("rmsnorm", _rms_no_eps_mean_abs),
    "rmsnorm_gain_not_centred": ("rmsnorm", _rms_gain_not_centred),
    "router_rows_reversed": ("router_logits", _logits_transposed_router),
    "clamp_gate_both_sides": ("swiglu_ffn", _ffn_clamp_both_sides),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(M, attr, fn)
    if hasattr(oracle, attr):
        monkeypatch.setattr(oracle, attr, fn)
    assert not _pins_pass(), f"planted mistake {name!r} went unnoticed"
