"""C-ABI checks that need no GPU: the library loads, exports every function
include/moe_mi355x.h declares, sizes workspaces, and rejects bad arguments
with the documented status before any HIP call."""
import ctypes
import os
import re

import pytest

from sparse_moe_transformer_fp32_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mi355x.h")

FLASH = (16, 4096, 288, 8, 1280, 1280)


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(moe_[a-z_]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    lib = B.load()
    declared = _declared_functions()
    assert set(declared) == set(B.EXPORTED), declared
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.moe_abi_version() == B.ABI_VERSION


def test_workspace_sizes():
    small = B.workspace_bytes(*FLASH)
    big = B.workspace_bytes(4096, 4096, 288, 8, 1280, 1280)
    assert 0 < small < big
    lay = B.workspace_layout(*FLASH)
    T, H, E, K, I, Is = FLASH
    assert lay.total == small
    assert lay.h % 256 == 0 and lay.o % 256 == 0
    assert lay.o - lay.h >= (T * K * I + T * Is) * 2
    assert lay.total - lay.o >= (T * K + T) * H * 2
    # no shared expert: smaller h and o
    assert B.workspace_bytes(16, 4096, 288, 8, 1280, 0) < small


@pytest.mark.parametrize("dims,frag", [
    ((0, 4096, 288, 8, 1280, 1280), "T=0"),
    ((16, 4000, 288, 8, 1280, 1280), "H=4000"),
    ((16, 4096, 0, 8, 1280, 1280), "E=0"),
    ((16, 4096, 2000, 8, 1280, 1280), "E=2000"),
    ((16, 4096, 4, 8, 1280, 1280), "K=8"),
    ((16, 4096, 288, 17, 1280, 1280), "K=17"),
    ((16, 4096, 288, 8, 1000, 1280), "I=1000"),
    ((16, 4096, 288, 8, 1280, 100), "Is=100"),
])
def test_bad_shapes_rejected(dims, frag):
    with pytest.raises(B.MoEError) as ei:
        B.workspace_bytes(*dims)
    assert ei.value.status == B.MOE_ERR_SHAPE
    assert frag in str(ei.value)


# Fake, 16-byte aligned device addresses: every call below fails its checks
# before touching them.
A = 0x10000


def _vp(v):
    return ctypes.c_void_p(v)


def _forward(dims=FLASH, opts=None, x=A, W=A, b=A, wg=A, wu=A, wd=A, shared=(A, A, A), y=2 * A,
             ws=A, ws_bytes=None, routing=None):
    lib = B.load()
    d = B.dims(*dims)
    o = opts if opts is not None else B.make_opts()
    r = B.Router(_vp(W), _vp(b))
    e = B.Experts(_vp(wg), _vp(wu), _vp(wd))
    sh = None if shared is None else B.Shared(*[_vp(v) for v in shared])
    if ws_bytes is None:
        ws_bytes = B.workspace_bytes(*dims) if dims[0] >= 1 and dims[1] % 128 == 0 else 1 << 40
    return lib.moe_forward(ctypes.byref(d), ctypes.byref(o), _vp(x), ctypes.byref(r),
                           ctypes.byref(e), ctypes.byref(sh) if sh is not None else None,
                           _vp(y), ctypes.byref(routing) if routing is not None else None,
                           _vp(ws), ws_bytes, None)


def test_forward_null_checks():
    assert _forward(x=0) == B.MOE_ERR_NULL
    assert "NULL" in B.last_error()
    assert _forward(W=0) == B.MOE_ERR_NULL
    assert _forward(wd=0) == B.MOE_ERR_NULL
    assert _forward(y=0) == B.MOE_ERR_NULL
    assert _forward(ws=0) == B.MOE_ERR_NULL
    assert _forward(shared=None) == B.MOE_ERR_NULL          # Is > 0 needs shared
    assert _forward(shared=(A, 0, A)) == B.MOE_ERR_NULL
    bad_r = B.Routing(_vp(A), _vp(A), None, _vp(A), _vp(A), _vp(A), None, None)
    assert _forward(routing=bad_r) == B.MOE_ERR_NULL


def test_forward_check_order():
    # null is reported before shape, shape before options, options before alignment
    bad_opts = B.make_opts(route_scale=-1.0)
    assert _forward(dims=(0,) + FLASH[1:], x=0, ws_bytes=1) == B.MOE_ERR_NULL
    assert _forward(dims=(0,) + FLASH[1:], opts=bad_opts, ws_bytes=1) == B.MOE_ERR_SHAPE
    assert _forward(opts=bad_opts, x=A + 2) == B.MOE_ERR_OPTION
    assert _forward(x=A + 2, ws_bytes=1) == B.MOE_ERR_ALIGN


def test_forward_option_checks():
    for kw in (dict(route_scale=0.0), dict(route_scale=float("nan")), dict(swiglu_limit=-1.0),
               dict(swiglu_limit_shared=float("inf"))):
        assert _forward(opts=B.make_opts(**kw)) == B.MOE_ERR_OPTION, kw
    o = B.make_opts()
    o.norm_topk = 2
    assert _forward(opts=o) == B.MOE_ERR_OPTION
    assert _forward(x=A, y=A) == B.MOE_ERR_OPTION          # aliasing x and y


def test_forward_alignment_and_workspace():
    assert _forward(x=A + 8) == B.MOE_ERR_ALIGN
    assert _forward(wu=A + 4) == B.MOE_ERR_ALIGN
    assert _forward(shared=(A, A, A + 2)) == B.MOE_ERR_ALIGN
    need = B.workspace_bytes(*FLASH)
    assert _forward(ws_bytes=need - 1) == B.MOE_ERR_WORKSPACE
    assert "workspace" in B.last_error()


def test_route_checks():
    lib = B.load()
    d = B.dims(*FLASH)
    r = B.Router(_vp(A), _vp(A))
    full = B.Routing(*([_vp(A)] * 6 + [None, None]))
    need = B.workspace_bytes(*FLASH)

    def call(x=A, out=full, ws=A, ws_bytes=need, dims=d, router=r):
        return lib.moe_route(ctypes.byref(dims), None, _vp(x), ctypes.byref(router),
                             ctypes.byref(out), _vp(ws), ws_bytes, None)

    assert call(x=0) == B.MOE_ERR_NULL
    assert call(out=B.Routing(*([_vp(A)] * 5 + [None, None, None]))) == B.MOE_ERR_NULL
    assert call(router=B.Router(_vp(A), None)) == B.MOE_ERR_NULL
    assert call(dims=B.dims(16, 4096, 8, 9, 1280, 1280)) == B.MOE_ERR_SHAPE
    assert call(x=A + 2) == B.MOE_ERR_ALIGN
    assert call(out=B.Routing(*([_vp(A)] * 6 + [_vp(A + 4), None]))) == B.MOE_ERR_ALIGN
    assert call(ws_bytes=10) == B.MOE_ERR_WORKSPACE


def test_residual_rmsnorm_checks():
    lib = B.load()
    f = lib.moe_residual_rmsnorm
    assert f(16, 4096, None, None, None, 1e-6, None, _vp(A), None) == B.MOE_ERR_NULL
    assert f(16, 4096, _vp(A), None, None, 1e-6, None, None, None) == B.MOE_ERR_NULL
    assert f(0, 4096, _vp(A), None, None, 1e-6, None, _vp(A), None) == B.MOE_ERR_SHAPE
    assert f(16, 100, _vp(A), None, None, 1e-6, None, _vp(A), None) == B.MOE_ERR_SHAPE
    assert f(16, 4096, _vp(A), None, None, -1.0, None, _vp(A), None) == B.MOE_ERR_OPTION
    assert f(16, 4096, _vp(A + 2), None, None, 1e-6, None, _vp(A), None) == B.MOE_ERR_ALIGN


def test_error_string_clears_on_success():
    _forward(x=0)
    assert B.last_error() != ""
    B.workspace_bytes(*FLASH)
    assert B.last_error() == ""


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros((16, 4096), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        B.route(x, torch.zeros((288, 4096)), torch.zeros(288), 8)


def test_pack_weights_checks():
    lib = B.load()
    f = lib.moe_pack_weights
    assert f(None, _vp(A), 1, 16, 32, None) == B.MOE_ERR_NULL
    assert f(_vp(A), _vp(1 << 30), 1, 8, 32, None) == B.MOE_ERR_SHAPE
    assert f(_vp(A), _vp(1 << 30), 1, 16, 48, None) == B.MOE_ERR_SHAPE
    assert f(_vp(A), _vp(1 << 30), 0, 16, 32, None) == B.MOE_ERR_SHAPE
    assert f(_vp(A + 2), _vp(1 << 30), 1, 16, 32, None) == B.MOE_ERR_ALIGN
    assert f(_vp(A), _vp(A + 512), 1, 16, 32, None) == B.MOE_ERR_OPTION   # overlap
