"""Dense brute force of the MoE layer, written independently of the oracle.

Every expert runs on every token; a mask keeps the top-K.  It shares no code
with oracle/ and uses different formulations on purpose:
  * sigmoid via the identity sigma(z) = (1 + tanh(z/2)) / 2,
  * the top-K mask by counting, for each expert, how many experts beat it
    (larger key, or equal key and lower index), instead of sorting,
  * all expert products as dense einsums over the full expert stack.
"""
import numpy as np


def _sig(z):
    return 0.5 * (1.0 + np.tanh(0.5 * z))


def brute_mask(keys, K):
    keys = np.asarray(keys, dtype=np.float64)
    T, E = keys.shape
    idx = np.arange(E)
    kj = keys[:, None, :]            # competitor e'
    ke = keys[:, :, None]            # candidate e
    beats = (kj > ke) | ((kj == ke) & (idx[None, None, :] < idx[None, :, None]))
    rank = beats.sum(axis=2)
    return rank < K


def brute_moe(x, Wr, b, Wg, Wu, Wd, Wsg=None, Wsu=None, Wsd=None, K=8, scale=3.0,
              bias_in_weights=False, norm=True):
    x = np.asarray(x, np.float64)
    Wr = np.asarray(Wr, np.float64)
    b = np.asarray(b, np.float64)
    l = np.einsum("th,eh->te", x, Wr)
    s = _sig(l)
    keys = s + b[None, :]
    m = brute_mask(keys, K).astype(np.float64)
    g = s + b[None, :] if bias_in_weights else s
    if norm:
        w = scale * g * m / (g * m).sum(axis=1, keepdims=True)
    else:
        w = scale * g * m
    G = np.einsum("th,eih->tei", x, np.asarray(Wg, np.float64))
    U = np.einsum("th,eih->tei", x, np.asarray(Wu, np.float64))
    Hh = G * _sig(G) * U
    O = np.einsum("tei,ehi->teh", Hh, np.asarray(Wd, np.float64))
    y = np.einsum("te,teh->th", w, O)
    if Wsg is not None:
        gs = x @ np.asarray(Wsg, np.float64).T
        us = x @ np.asarray(Wsu, np.float64).T
        y = y + (gs * _sig(gs) * us) @ np.asarray(Wsd, np.float64).T
    return y, m.astype(bool), w


def textbook_swiglu_row(xv, Wg, Wu, Wd):
    """One token through one gated FFN with explicit scalar loops."""
    import math
    I, H = len(Wg), len(xv)
    h = []
    for i in range(I):
        gi = sum(float(Wg[i][k]) * float(xv[k]) for k in range(H))
        ui = sum(float(Wu[i][k]) * float(xv[k]) for k in range(H))
        h.append(gi / (1.0 + math.exp(-gi)) * ui)
    return [sum(float(Wd[n][i]) * h[i] for i in range(I)) for n in range(len(Wd))]
