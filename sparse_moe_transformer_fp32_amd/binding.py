"""Thin ctypes binding of the gfx950 C-ABI library `libsmoe_gfx950.so`.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  torch provides device memory and the stream (`tensor.data_ptr()`
and `torch.cuda.current_stream().cuda_stream`).  There is no fallback: if
the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsmoe_gfx950.so")
ABI_VERSION = 4

MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE = 0, -1, -2, -3
MOE_ERR_WORKSPACE, MOE_ERR_ALIGN, MOE_ERR_DEVICE, MOE_ERR_OPTION = -4, -5, -6, -7
STATUS_NAMES = {0: "MOE_OK", -1: "MOE_ERR_NULL", -2: "MOE_ERR_SHAPE", -3: "MOE_ERR_DTYPE",
                -4: "MOE_ERR_WORKSPACE", -5: "MOE_ERR_ALIGN", -6: "MOE_ERR_DEVICE",
                -7: "MOE_ERR_OPTION"}
# weight layouts a weight struct declares (only the packed one is read)
MOE_LAYOUT_ROW_MAJOR, MOE_LAYOUT_PACKED = 0, 1

EXPORTED = ["moe_abi_version", "moe_last_error", "moe_workspace_bytes", "moe_workspace_layout",
            "moe_route", "moe_forward", "moe_forward_residual", "moe_residual_rmsnorm",
            "moe_set_stage_events", "moe_pack_weights", "moe_pack_weights_strided",
            "moe_dense_workspace_bytes", "moe_dense_ffn", "moe_expert_stats", "moe_read_probe",
            "moe_mfma_probe", "moe_forward_noalloc"]
# bytes of the library's fixed scratch array (moe_forward_noalloc)
NOALLOC_SCRATCH_BYTES = 32 << 20
STAGES = ["route_logits", "route_topk", "dispatch", "gate_up", "down", "combine"]

_vp = ctypes.c_void_p


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("T", "H", "E", "K", "I", "Is")]


class Opts(ctypes.Structure):
    _fields_ = [("route_scale", ctypes.c_float), ("norm_topk", ctypes.c_int32),
                ("bias_in_weights", ctypes.c_int32), ("swiglu_limit", ctypes.c_float),
                ("swiglu_limit_shared", ctypes.c_float)]


class Router(ctypes.Structure):
    _fields_ = [("W", _vp), ("b", _vp)]


class Experts(ctypes.Structure):
    _fields_ = [("layout", ctypes.c_int32), ("w_gate", _vp), ("w_up", _vp), ("w_down", _vp)]


class Shared(ctypes.Structure):
    _fields_ = [("layout", ctypes.c_int32), ("w_gate", _vp), ("w_up", _vp), ("w_down", _vp)]


def packed_experts(w_gate, w_up, w_down) -> Experts:
    """moe_experts for packed weights (the output of moe_pack_weights)."""
    return Experts(MOE_LAYOUT_PACKED, _ptr(w_gate), _ptr(w_up), _ptr(w_down))


def packed_shared(w_gate, w_up, w_down) -> Shared:
    """moe_shared / moe_ffn for packed weights."""
    return Shared(MOE_LAYOUT_PACKED, _ptr(w_gate), _ptr(w_up), _ptr(w_down))


class Routing(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("topk_idx", "topk_w", "counts", "offsets", "perm_token",
                                   "slot_pos", "keys", "scores")]


class Residual(ctypes.Structure):
    _fields_ = [("r_in", _vp), ("r_out", _vp), ("x_next", _vp), ("gamma", _vp),
                ("eps", ctypes.c_float)]


class WsLayout(ctypes.Structure):
    _fields_ = [("h", ctypes.c_size_t), ("o", ctypes.c_size_t), ("total", ctypes.c_size_t)]


class MoEError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load the library once; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library {LIB_PATH} is not built; run "
                           "`python -m sparse_moe_transformer_fp32_amd.build` first")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    lib.moe_abi_version.restype = ctypes.c_int32
    lib.moe_abi_version.argtypes = []
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_last_error.argtypes = []
    lib.moe_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_workspace_bytes.argtypes = [P(Dims)]
    lib.moe_workspace_layout.restype = ctypes.c_int
    lib.moe_workspace_layout.argtypes = [P(Dims), P(WsLayout)]
    lib.moe_route.restype = ctypes.c_int
    lib.moe_route.argtypes = [P(Dims), P(Opts), _vp, P(Router), P(Routing), _vp, ctypes.c_size_t, _vp]
    lib.moe_forward.restype = ctypes.c_int
    lib.moe_forward.argtypes = [P(Dims), P(Opts), _vp, P(Router), P(Experts), P(Shared), _vp,
                                P(Routing), _vp, ctypes.c_size_t, _vp]
    lib.moe_forward_noalloc.restype = ctypes.c_int
    lib.moe_forward_noalloc.argtypes = [P(Dims), P(Opts), _vp, P(Router), P(Experts), P(Shared),
                                        _vp, P(Routing), _vp]
    lib.moe_forward_residual.restype = ctypes.c_int
    lib.moe_forward_residual.argtypes = [P(Dims), P(Opts), _vp, P(Router), P(Experts), P(Shared),
                                         P(Residual), P(Routing), _vp, ctypes.c_size_t, _vp]
    lib.moe_dense_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_dense_workspace_bytes.argtypes = [ctypes.c_int32] * 4
    lib.moe_dense_ffn.restype = ctypes.c_int
    lib.moe_dense_ffn.argtypes = [ctypes.c_int32] * 4 + [_vp, P(Shared), ctypes.c_float, _vp, _vp,
                                                         ctypes.c_size_t, _vp]
    lib.moe_expert_stats.restype = ctypes.c_int
    lib.moe_expert_stats.argtypes = [P(Dims), _vp, _vp, _vp, _vp, _vp]
    lib.moe_pack_weights_strided.restype = ctypes.c_int
    lib.moe_pack_weights_strided.argtypes = [_vp, _vp, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, _vp]
    lib.moe_residual_rmsnorm.restype = ctypes.c_int
    lib.moe_residual_rmsnorm.argtypes = [ctypes.c_int32, ctypes.c_int32, _vp, _vp, _vp,
                                         ctypes.c_float, _vp, _vp, _vp]
    lib.moe_pack_weights.restype = ctypes.c_int
    lib.moe_pack_weights.argtypes = [_vp, _vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _vp]
    lib.moe_set_stage_events.restype = ctypes.c_int
    lib.moe_set_stage_events.argtypes = [_vp, ctypes.c_int32]
    lib.moe_read_probe.restype = ctypes.c_int
    lib.moe_read_probe.argtypes = [_vp, ctypes.c_size_t, ctypes.c_int32, _vp, _vp]
    lib.moe_mfma_probe.restype = ctypes.c_int
    lib.moe_mfma_probe.argtypes = [ctypes.c_int32, _vp, ctypes.c_int32, _vp, _vp]
    v = lib.moe_abi_version()
    if v != ABI_VERSION:
        raise RuntimeError(f"{LIB_PATH}: ABI version {v}, binding expects {ABI_VERSION}")
    _lib = lib
    return lib


def last_error() -> str:
    return load().moe_last_error().decode()


def _check(status: int):
    if status != MOE_OK:
        raise MoEError(status, last_error())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def make_opts(route_scale=3.0, norm_topk=True, bias_in_weights=False, swiglu_limit=0.0,
              swiglu_limit_shared=0.0) -> Opts:
    return Opts(float(route_scale), int(bool(norm_topk)), int(bool(bias_in_weights)),
                float(swiglu_limit), float(swiglu_limit_shared))


def dims(T, H, E, K, I, Is) -> Dims:
    return Dims(int(T), int(H), int(E), int(K), int(I), int(Is))


def workspace_bytes(T, H, E, K, I, Is) -> int:
    d = dims(T, H, E, K, I, Is)
    n = load().moe_workspace_bytes(ctypes.byref(d))
    if n == 0:
        raise MoEError(MOE_ERR_SHAPE, last_error())
    return n


def workspace_layout(T, H, E, K, I, Is) -> WsLayout:
    d = dims(T, H, E, K, I, Is)
    out = WsLayout()
    _check(load().moe_workspace_layout(ctypes.byref(d), ctypes.byref(out)))
    return out


def alloc_workspace(T, H, E, K, I, Is, device="cuda") -> torch.Tensor:
    return torch.empty(workspace_bytes(T, H, E, K, I, Is), dtype=torch.uint8, device=device)


def alloc_routing(T, E, K, device="cuda", keys=False) -> Dict[str, torch.Tensor]:
    i32, f32 = torch.int32, torch.float32
    r = dict(topk_idx=torch.empty((T, K), dtype=i32, device=device),
             topk_w=torch.empty((T, K), dtype=f32, device=device),
             counts=torch.empty(E, dtype=i32, device=device),
             offsets=torch.empty(E + 1, dtype=i32, device=device),
             perm_token=torch.empty(T * K, dtype=i32, device=device),
             slot_pos=torch.empty((T, K), dtype=i32, device=device))
    if keys:
        r["keys"] = torch.empty((T, E), dtype=f32, device=device)
        r["scores"] = torch.empty((T, E), dtype=f32, device=device)
    return r


def _routing_struct(r: Dict[str, torch.Tensor]) -> Routing:
    return Routing(*[_ptr(r.get(n)) for n in ("topk_idx", "topk_w", "counts", "offsets",
                                               "perm_token", "slot_pos", "keys", "scores")])


def route(x: torch.Tensor, router_w: torch.Tensor, router_b: torch.Tensor, K: int, *,
          I: int = 64, Is: int = 0, keys: bool = False, ws: Optional[torch.Tensor] = None,
          out: Optional[Dict[str, torch.Tensor]] = None, **opts) -> Dict[str, torch.Tensor]:
    """Router and dispatch (moe_route).  I/Is only size the workspace."""
    lib = load()
    _dev(x, "x", torch.bfloat16)
    _dev(router_w, "router_w", torch.float32)
    _dev(router_b, "router_b", torch.float32)
    T, H = x.shape
    E = router_w.shape[0]
    d = dims(T, H, E, K, I, Is)
    if ws is None:
        ws = alloc_workspace(T, H, E, K, I, Is, x.device)
    r = out if out is not None else alloc_routing(T, E, K, x.device, keys)
    o = make_opts(**opts)
    rt = Router(_ptr(router_w), _ptr(router_b))
    rs = _routing_struct(r)
    _check(lib.moe_route(ctypes.byref(d), ctypes.byref(o), _ptr(x), ctypes.byref(rt),
                         ctypes.byref(rs), _ptr(ws), ws.numel(), _stream(x.device)))
    return r


def pack_weights(w: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Fragment-packed copy (moe_pack_weights) of a row-major bf16 matrix
    [R, C] or stack of matrices [n, R, C]."""
    lib = load()
    _dev(w, "w", torch.bfloat16)
    if w.dim() == 2:
        n, R, C = 1, w.shape[0], w.shape[1]
    elif w.dim() == 3:
        n, R, C = w.shape
    else:
        raise ValueError("pack_weights expects a 2-D or 3-D tensor")
    if out is None:
        out = torch.empty_like(w)
    _dev(out, "out", torch.bfloat16)
    _check(lib.moe_pack_weights(_ptr(w), _ptr(out), n, R, C, _stream(w.device)))
    return out


def pack_column_slices(w: torch.Tensor, S: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """S packed matrices [R, C/S] (moe_pack_weights_strided), matrix s being
    columns s*C/S .. (s+1)*C/S - 1 of the row-major bf16 matrix w [R, C]."""
    lib = load()
    _dev(w, "w", torch.bfloat16)
    R, C = w.shape
    if C % S:
        raise ValueError(f"{C} columns do not split into {S} slices")
    if out is None:
        out = torch.empty((S, R, C // S), dtype=w.dtype, device=w.device)
    _dev(out, "out", torch.bfloat16)
    _check(lib.moe_pack_weights_strided(_ptr(w), _ptr(out), S, R, C // S, C, C // S,
                                        _stream(w.device)))
    return out


class MoELayer:
    """One MoE FFN layer bound to device weights, with its workspace and
    output buffer allocated once (calls allocate nothing).  Expert weights
    are given row-major ([E,I,H], [E,I,H], [E,H,I]; shared [Is,H], [Is,H],
    [H,Is]) and packed once here, unless `packed=True` says they already are."""

    def __init__(self, router_w, router_b, w_gate, w_up, w_down, ws_gate=None, ws_up=None,
                 ws_down=None, K=8, T_max=None, packed=False, **opts):
        load()
        _dev(router_w, "router_w", torch.float32)
        _dev(router_b, "router_b", torch.float32)
        for n, t in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
            _dev(t, n, torch.bfloat16)
        self.E, self.H = router_w.shape
        self.I = w_gate.shape[1]
        self.K = int(K)
        self.Is = 0 if ws_gate is None else ws_gate.shape[0]
        if self.Is:
            for n, t in (("ws_gate", ws_gate), ("ws_up", ws_up), ("ws_down", ws_down)):
                _dev(t, n, torch.bfloat16)
        if not packed:
            w_gate, w_up, w_down = pack_weights(w_gate), pack_weights(w_up), pack_weights(w_down)
            if self.Is:
                ws_gate, ws_up, ws_down = (pack_weights(ws_gate), pack_weights(ws_up),
                                           pack_weights(ws_down))
        self.tensors = (router_w, router_b, w_gate, w_up, w_down, ws_gate, ws_up, ws_down)
        self.router = Router(_ptr(router_w), _ptr(router_b))
        self.experts = packed_experts(w_gate, w_up, w_down)
        self.shared = packed_shared(ws_gate, ws_up, ws_down) if self.Is else None
        self.opts = make_opts(**opts)
        self.device = router_w.device
        self._ws = None
        self._retired = []
        if T_max:
            self.reserve(T_max)

    def reserve(self, T: int) -> int:
        """Make the workspace hold a T-token call.  The size never falls as T
        grows, so one reserve for the largest batch serves every smaller one.
        A workspace that is outgrown is kept alive (HIP graphs captured on it
        may still replay), never handed back to the allocator."""
        need = workspace_bytes(T, self.H, self.E, self.K, self.I, self.Is)
        if self._ws is None or self._ws.numel() < need:
            if self._ws is not None:
                self._retired.append(self._ws)
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return need

    def workspace(self) -> torch.Tensor:
        return self._ws

    def forward(self, x: torch.Tensor, y: Optional[torch.Tensor] = None,
                routing: Optional[Dict[str, torch.Tensor]] = None) -> torch.Tensor:
        lib = load()
        _dev(x, "x", torch.bfloat16)
        T = x.shape[0]
        if x.shape[1] != self.H:
            raise ValueError(f"x has {x.shape[1]} columns, layer hidden size is {self.H}")
        ws_bytes = self.reserve(T)
        if y is None:
            y = torch.empty_like(x)
        _dev(y, "y", torch.bfloat16)
        d = dims(T, self.H, self.E, self.K, self.I, self.Is)
        rs = _routing_struct(routing) if routing is not None else None
        _check(lib.moe_forward(ctypes.byref(d), ctypes.byref(self.opts), _ptr(x),
                               ctypes.byref(self.router), ctypes.byref(self.experts),
                               ctypes.byref(self.shared) if self.shared is not None else None,
                               _ptr(y), ctypes.byref(rs) if rs is not None else None,
                               _ptr(self._ws), ws_bytes, _stream(x.device)))
        return y

    __call__ = forward

    def forward_noalloc(self, x: torch.Tensor, y: torch.Tensor,
                        routing: Optional[Dict[str, torch.Tensor]] = None) -> torch.Tensor:
        """moe_forward_noalloc: the layer with the library's fixed scratch
        array instead of a workspace; y (and routing) are the caller's."""
        lib = load()
        _dev(x, "x", torch.bfloat16)
        _dev(y, "y", torch.bfloat16)
        T = x.shape[0]
        d = dims(T, self.H, self.E, self.K, self.I, self.Is)
        rs = _routing_struct(routing) if routing is not None else None
        _check(lib.moe_forward_noalloc(ctypes.byref(d), ctypes.byref(self.opts), _ptr(x),
                                       ctypes.byref(self.router), ctypes.byref(self.experts),
                                       ctypes.byref(self.shared) if self.shared is not None
                                       else None, _ptr(y),
                                       ctypes.byref(rs) if rs is not None else None,
                                       _stream(x.device)))
        return y

    def forward_residual(self, x: torch.Tensor, r_in: torch.Tensor,
                         r_out: Optional[torch.Tensor] = None,
                         x_next: Optional[torch.Tensor] = None,
                         gamma: Optional[torch.Tensor] = None, eps: float = 1e-6,
                         routing: Optional[Dict[str, torch.Tensor]] = None) -> torch.Tensor:
        """r_out = r_in + layer(x); x_next (if given) = RMSNorm(r_out)
        (moe_forward_residual).  r_out may be r_in; x_next may be x."""
        lib = load()
        for n, t in (("x", x), ("r_in", r_in)):
            _dev(t, n, torch.bfloat16)
        T = x.shape[0]
        if r_out is None:
            r_out = torch.empty_like(r_in)
        _dev(r_out, "r_out", torch.bfloat16)
        if x_next is not None:
            _dev(x_next, "x_next", torch.bfloat16)
        if gamma is not None:
            _dev(gamma, "gamma", torch.float32)
        ws_bytes = self.reserve(T)
        d = dims(T, self.H, self.E, self.K, self.I, self.Is)
        res = Residual(_ptr(r_in), _ptr(r_out), _ptr(x_next), _ptr(gamma), float(eps))
        rs = _routing_struct(routing) if routing is not None else None
        _check(lib.moe_forward_residual(
            ctypes.byref(d), ctypes.byref(self.opts), _ptr(x), ctypes.byref(self.router),
            ctypes.byref(self.experts),
            ctypes.byref(self.shared) if self.shared is not None else None, ctypes.byref(res),
            ctypes.byref(rs) if rs is not None else None, _ptr(self._ws), ws_bytes,
            _stream(x.device)))
        return r_out

    def expert_stats(self, T: int, offsets: torch.Tensor, ratios: bool = True):
        """Per-expert activation statistics of the last call with T tokens
        (moe_expert_stats): stats [E (+1 shared), 4] = (rows, sum ||h||,
        sum ||h||^2, max ||h||) and ratios [2] = (max/median, min/median of
        the mean norms)."""
        lib = load()
        _dev(offsets, "offsets", torch.int32)
        lay = workspace_layout(T, self.H, self.E, self.K, self.I, self.Is)
        G = self.E + (1 if self.Is else 0)
        stats = torch.empty((G, 4), dtype=torch.float32, device=self.device)
        rat = torch.empty(2, dtype=torch.float32, device=self.device) if ratios else None
        d = dims(T, self.H, self.E, self.K, self.I, self.Is)
        h_ptr = ctypes.c_void_p(self._ws.data_ptr() + lay.h)
        _check(lib.moe_expert_stats(ctypes.byref(d), _ptr(offsets), h_ptr, _ptr(stats), _ptr(rat),
                                    _stream(self.device)))
        return (stats, rat) if ratios else stats


class DenseFFN:
    """A dense gated FFN y = Wd (silu(Wg x) * (Wu x)) run by moe_dense_ffn
    with its intermediate dimension cut into S slices.  Weights are given
    row-major (Wg, Wu [I,H]; Wd [H,I]) and packed once here."""

    def __init__(self, w_gate, w_up, w_down, S: int = 8, T_max=None, swiglu_limit: float = 0.0):
        load()
        for n, t in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
            _dev(t, n, torch.bfloat16)
        self.I, self.H = w_gate.shape
        self.S = int(S)
        self.tensors = (pack_weights(w_gate), pack_weights(w_up),
                        pack_column_slices(w_down, self.S))
        self.ffn = packed_shared(*self.tensors)
        self.limit = float(swiglu_limit)
        self.device = w_gate.device
        self._ws = None
        self._retired = []
        if T_max:
            self.reserve(T_max)

    def reserve(self, T: int) -> int:
        need = load().moe_dense_workspace_bytes(T, self.H, self.I, self.S)
        if need == 0:
            raise MoEError(MOE_ERR_SHAPE, last_error())
        if self._ws is None or self._ws.numel() < need:
            if self._ws is not None:   # kept alive, as in MoELayer.reserve
                self._retired.append(self._ws)
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return need

    def forward(self, x: torch.Tensor, y: Optional[torch.Tensor] = None) -> torch.Tensor:
        lib = load()
        _dev(x, "x", torch.bfloat16)
        T = x.shape[0]
        ws_bytes = self.reserve(T)
        if y is None:
            y = torch.empty_like(x)
        _dev(y, "y", torch.bfloat16)
        _check(lib.moe_dense_ffn(T, self.H, self.I, self.S, _ptr(x), ctypes.byref(self.ffn),
                                 self.limit, _ptr(y), _ptr(self._ws), ws_bytes, _stream(x.device)))
        return y

    __call__ = forward


def forward(x, router_w, router_b, w_gate, w_up, w_down, ws_gate=None, ws_up=None, ws_down=None,
            K=8, routing: bool = False, keys: bool = False, **opts):
    """One call of moe_forward with freshly allocated buffers.  With
    routing=True also returns the routing tensors."""
    layer = MoELayer(router_w, router_b, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, K=K, **opts)
    r = alloc_routing(x.shape[0], layer.E, K, x.device, keys) if routing else None
    y = layer.forward(x, routing=r)
    return (y, r, layer) if routing else y


def set_stage_events(events_array) -> None:
    """Install (or with None, remove) the per-stage timing events: a ctypes
    array of 2 * len(STAGES) hipEvent_t handles (see moe_set_stage_events)."""
    lib = load()
    if events_array is None:
        _check(lib.moe_set_stage_events(None, 0))
    else:
        _check(lib.moe_set_stage_events(ctypes.cast(events_array, _vp), len(events_array)))


def read_probe(buf: torch.Tensor, sink: torch.Tensor, nontemporal: bool) -> None:
    """One plain read of `buf` (device, 16-byte aligned, a multiple of 16384
    bytes) with ordinary or non-temporal 16-byte loads, on the current stream
    (moe_read_probe): the HBM read ceiling the weight streams are measured
    against.  `sink` is a 16-byte device tensor the kernel does not write."""
    lib = load()
    _check(lib.moe_read_probe(_vp(buf.data_ptr()), buf.numel() * buf.element_size(),
                              1 if nontemporal else 0, _vp(sink.data_ptr()), _stream(buf.device)))


def mfma_probe(iters: int, clocks: torch.Tensor, sink: torch.Tensor) -> None:
    """iters rounds of four bf16 32x32x16 MFMAs per wave, one 8-wave
    workgroup per CU, on the current stream (moe_mfma_probe): the matrix-core
    rate the chip sustains.  `clocks` is an int64 device tensor of at least
    2 x CU-count entries that receives each workgroup's (shader clock ticks,
    100 MHz ticks) over its loop; `sink` a 16-byte device tensor."""
    lib = load()
    _check(lib.moe_mfma_probe(iters, _vp(clocks.data_ptr()), clocks.numel(), _vp(sink.data_ptr()),
                              _stream(clocks.device)))


def residual_rmsnorm(r_in: torch.Tensor, y_add: Optional[torch.Tensor] = None,
                     gamma: Optional[torch.Tensor] = None, eps: float = 1e-6,
                     r_out: Optional[torch.Tensor] = None, x_out: Optional[torch.Tensor] = None,
                     want_r: bool = True, want_x: bool = True):
    """r = r_in + y_add (bf16), x = RMSNorm(r) (bf16), via moe_residual_rmsnorm."""
    lib = load()
    _dev(r_in, "r_in", torch.bfloat16)
    T, H = r_in.shape
    if y_add is not None:
        _dev(y_add, "y_add", torch.bfloat16)
        if r_out is None and want_r:
            r_out = torch.empty_like(r_in)
    if gamma is not None:
        _dev(gamma, "gamma", torch.float32)
    if x_out is None and want_x:
        x_out = torch.empty_like(r_in)
    _check(lib.moe_residual_rmsnorm(T, H, _ptr(r_in), _ptr(y_add), _ptr(gamma), float(eps),
                                    _ptr(r_out), _ptr(x_out), _stream(r_in.device)))
    return r_out, x_out


class MoEChain:
    """Pre-norm residual stream through chained MoE layers:
        x_0 = RMSNorm(r_0);  r_{l+1} = r_l + MoE_l(x_l);  x_{l+1} = RMSNorm(r_{l+1})
    One moe_residual_rmsnorm call makes x_0; then each layer is one
    moe_forward_residual call, whose last kernel adds the layer output to
    the stream and, for all but the last layer, writes the next layer's
    input.  Returns the last residual stream.  Buffers are allocated once per
    batch size."""

    def __init__(self, layers, eps: float = 1e-6, gamma: Optional[torch.Tensor] = None):
        self.layers = list(layers)
        self.eps = float(eps)
        self.gamma = gamma
        self._bufs = None

    def _buffers(self, x):
        if self._bufs is None or self._bufs[0].shape != x.shape:
            self._bufs = tuple(torch.empty_like(x) for _ in range(3))
        return self._bufs

    def forward(self, r0: torch.Tensor, capture: bool = False,
                routing_last: Optional[Dict[str, torch.Tensor]] = None):
        """capture=True also returns, per layer, (r_l, x_l, routing_l)
        copies (routing with keys and scores) for checking.  routing_last
        receives the last layer's routing."""
        xn, ra, rb = self._buffers(r0)
        trace = []
        residual_rmsnorm(r0, None, self.gamma, self.eps, None, xn, want_r=False)
        r = r0
        for li, lay in enumerate(self.layers):
            last = li == len(self.layers) - 1
            rt = alloc_routing(r0.shape[0], lay.E, lay.K, r0.device, keys=True) if capture else None
            if rt is None and last:
                rt = routing_last
            if capture:
                trace.append((r.clone(), xn.clone(), rt))
            r_next = ra if li % 2 == 0 else rb
            lay.forward_residual(xn, r, r_next, None if last else xn, self.gamma, self.eps, rt)
            r = r_next
        return (r, trace) if capture else r

    __call__ = forward
