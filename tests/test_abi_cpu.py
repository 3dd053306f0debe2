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
    ((-1, 4096, 288, 8, 1280, 1280), "T=-1"),
    (((1 << 20) + 1, 4096, 288, 8, 1280, 1280), "T=1048577"),
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
             ws=A, ws_bytes=None, routing=None, layout=None, shared_layout=None):
    lib = B.load()
    d = B.dims(*dims)
    o = opts if opts is not None else B.make_opts()
    r = B.Router(_vp(W), _vp(b))
    lay = B.MOE_LAYOUT_PACKED if layout is None else layout
    e = B.Experts(lay, _vp(wg), _vp(wu), _vp(wd))
    slay = B.MOE_LAYOUT_PACKED if shared_layout is None else shared_layout
    sh = None if shared is None else B.Shared(slay, *[_vp(v) for v in shared])
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
    # null is reported before layout, layout before shape, shape before
    # options, options before alignment
    bad_opts = B.make_opts(route_scale=-1.0)
    assert _forward(dims=(16, 4000) + FLASH[2:], x=0, ws_bytes=1) == B.MOE_ERR_NULL
    assert _forward(dims=(16, 4000) + FLASH[2:], x=0, layout=0, ws_bytes=1) == B.MOE_ERR_NULL
    assert _forward(dims=(16, 4000) + FLASH[2:], layout=0, ws_bytes=1) == B.MOE_ERR_DTYPE
    assert _forward(dims=(16, 4000) + FLASH[2:], opts=bad_opts, ws_bytes=1) == B.MOE_ERR_SHAPE
    assert _forward(opts=bad_opts, x=A + 2) == B.MOE_ERR_OPTION
    assert _forward(x=A + 2, ws_bytes=1) == B.MOE_ERR_ALIGN


def test_row_major_weights_are_refused():
    """A weight struct filled as the plain [E,I,H] / [E,H,I] row-major layout
    (layout field left at 0, as a zero-initialised C struct has it) is refused
    with MOE_ERR_DTYPE before any HIP call, instead of being read as packed
    tiles; so is an unknown layout tag.  Only MOE_LAYOUT_PACKED passes."""
    assert _forward(layout=B.MOE_LAYOUT_ROW_MAJOR) == B.MOE_ERR_DTYPE
    assert "MOE_LAYOUT_ROW_MAJOR" in B.last_error() and "moe_pack_weights" in B.last_error()
    assert _forward(shared_layout=B.MOE_LAYOUT_ROW_MAJOR) == B.MOE_ERR_DTYPE
    assert "shared" in B.last_error()
    assert _forward(layout=7) == B.MOE_ERR_DTYPE
    assert "unknown layout 7" in B.last_error()
    # no shared expert (Is = 0): the shared struct is not read at all
    assert _forward(dims=FLASH[:5] + (0,), shared=None, ws_bytes=1) == B.MOE_ERR_WORKSPACE
    R = B.Residual(_vp(3 * A), _vp(4 * A), _vp(5 * A), None, 1e-6)
    lib = B.load()
    d, o, r = B.dims(*FLASH), B.make_opts(), B.Router(_vp(A), _vp(A))
    e = B.Experts(B.MOE_LAYOUT_ROW_MAJOR, _vp(A), _vp(A), _vp(A))
    sh = B.Shared(B.MOE_LAYOUT_PACKED, _vp(A), _vp(A), _vp(A))
    assert lib.moe_forward_residual(ctypes.byref(d), ctypes.byref(o), _vp(A), ctypes.byref(r),
                                    ctypes.byref(e), ctypes.byref(sh), ctypes.byref(R), None,
                                    _vp(6 * A), 1 << 40, None) == B.MOE_ERR_DTYPE


def test_workspace_never_shrinks_as_T_grows():
    """One workspace sized for the largest batch serves every smaller one:
    moe_workspace_bytes is non-decreasing in T (Flash shape over
    T = 0..4096, and small shapes where the router's H split and the GEMM
    row-block height change most often)."""
    for shape in (FLASH[1:], (128, 1024, 1, 64, 0), (256, 16, 2, 64, 64), (1024, 30, 3, 64, 64)):
        prev = 0
        for T in range(0, 4097):
            n = B.workspace_bytes(T, *shape)
            assert n >= prev, (shape, T, n, prev)
            prev = n
    lib = B.load()
    prev = 0
    for T in range(0, 2049):
        n = lib.moe_dense_workspace_bytes(T, 4096, 11264, 8)
        assert n >= prev, (T, n, prev)
        prev = n


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
    assert f(-1, 4096, _vp(A), None, None, 1e-6, None, _vp(A), None) == B.MOE_ERR_SHAPE
    # an empty batch is a no-op (returns before any HIP call), pointers unused
    assert f(0, 4096, None, None, None, 1e-6, None, None, None) == B.MOE_OK
    assert f(0, 100, None, None, None, 1e-6, None, None, None) == B.MOE_ERR_SHAPE
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


def _forward_res(res=None, x=A, ws_bytes=None, dims=FLASH):
    lib = B.load()
    d = B.dims(*dims)
    o = B.make_opts()
    r = B.Router(_vp(A), _vp(A))
    e = B.Experts(B.MOE_LAYOUT_PACKED, _vp(A), _vp(A), _vp(A))
    sh = B.Shared(B.MOE_LAYOUT_PACKED, _vp(A), _vp(A), _vp(A))
    if res is None:
        res = B.Residual(_vp(3 * A), _vp(4 * A), _vp(5 * A), None, 1e-6)
    if ws_bytes is None:
        ws_bytes = B.workspace_bytes(*dims)
    return lib.moe_forward_residual(ctypes.byref(d), ctypes.byref(o), _vp(x), ctypes.byref(r),
                                    ctypes.byref(e), ctypes.byref(sh),
                                    ctypes.byref(res) if res is not False else None, None,
                                    _vp(6 * A), ws_bytes, None)


def test_forward_residual_checks():
    R = B.Residual
    assert _forward_res(res=False) == B.MOE_ERR_NULL
    assert _forward_res(res=R(None, _vp(4 * A), None, None, 1e-6)) == B.MOE_ERR_NULL
    assert _forward_res(res=R(_vp(3 * A), None, None, None, 1e-6)) == B.MOE_ERR_NULL
    assert _forward_res(x=0) == B.MOE_ERR_NULL
    assert _forward_res(res=R(_vp(3 * A), _vp(4 * A), None, None, -1.0)) == B.MOE_ERR_OPTION
    assert _forward_res(res=R(_vp(3 * A), _vp(4 * A), _vp(4 * A), None, 1e-6)) == B.MOE_ERR_OPTION
    assert _forward_res(res=R(_vp(3 * A), _vp(4 * A), _vp(3 * A), None, 1e-6)) == B.MOE_ERR_OPTION
    assert _forward_res(x=3 * A) == B.MOE_ERR_OPTION               # x aliases r_in
    assert _forward_res(res=R(_vp(3 * A + 2), _vp(4 * A), None, None, 1e-6)) == B.MOE_ERR_ALIGN
    assert _forward_res(res=R(_vp(3 * A), _vp(4 * A), None, _vp(A + 4), 1e-6)) == B.MOE_ERR_ALIGN
    assert _forward_res(ws_bytes=100) == B.MOE_ERR_WORKSPACE
    # r_out may alias r_in and x_next may alias x: only the workspace fails here
    ok = R(_vp(3 * A), _vp(3 * A), _vp(A), None, 1e-6)
    assert _forward_res(res=ok, ws_bytes=100) == B.MOE_ERR_WORKSPACE


def test_dense_checks():
    lib = B.load()
    assert lib.moe_dense_workspace_bytes(16, 4096, 11264, 8) > 0
    assert lib.moe_dense_workspace_bytes(16, 4096, 11264, 7) == 0       # 11264 % 7
    assert lib.moe_dense_workspace_bytes(16, 4096, 11264, 32) == 0      # S > 16
    assert lib.moe_dense_workspace_bytes(16, 4096, 11264 + 32, 8) == 0  # slices not % 64
    assert lib.moe_dense_workspace_bytes(-1, 4096, 11264, 8) == 0
    need = lib.moe_dense_workspace_bytes(16, 4096, 11264, 8)
    f = B.Shared(B.MOE_LAYOUT_PACKED, _vp(A), _vp(A), _vp(A))

    def call(T=16, H=4096, I=11264, S=8, x=A, ffn=f, lim=0.0, y=2 * A, ws=3 * A, n=need):
        return lib.moe_dense_ffn(T, H, I, S, _vp(x), ctypes.byref(ffn) if ffn else None, lim,
                                 _vp(y), _vp(ws), n, None)

    assert call(x=0) == B.MOE_ERR_NULL
    assert call(ffn=B.Shared(B.MOE_LAYOUT_PACKED, _vp(A), None, _vp(A))) == B.MOE_ERR_NULL
    # row-major weights (layout left at 0) are refused, not read as packed
    assert call(ffn=B.Shared(B.MOE_LAYOUT_ROW_MAJOR, _vp(A), _vp(A), _vp(A))) == B.MOE_ERR_DTYPE
    assert call(I=1000) == B.MOE_ERR_SHAPE
    assert call(H=4000) == B.MOE_ERR_SHAPE
    assert call(lim=-1.0) == B.MOE_ERR_OPTION
    assert call(y=A) == B.MOE_ERR_OPTION
    assert call(x=A + 2) == B.MOE_ERR_ALIGN
    assert call(n=need - 1) == B.MOE_ERR_WORKSPACE


def test_expert_stats_checks():
    lib = B.load()
    d = B.dims(*FLASH)
    f = lib.moe_expert_stats
    assert f(ctypes.byref(d), None, _vp(A), _vp(A), None, None) == B.MOE_ERR_NULL
    assert f(ctypes.byref(d), _vp(A), _vp(A), None, None, None) == B.MOE_ERR_NULL
    bad = B.dims(16, 4096, 288, 9, 1280, 1280)
    bad.K = 17
    assert f(ctypes.byref(bad), _vp(A), _vp(A), _vp(A), None, None) == B.MOE_ERR_SHAPE
    assert f(ctypes.byref(d), _vp(A), _vp(A), _vp(A), _vp(A + 4), None) == B.MOE_ERR_ALIGN


def test_pack_weights_strided_checks():
    lib = B.load()
    f = lib.moe_pack_weights_strided
    assert f(_vp(A), _vp(1 << 30), 2, 16, 32, 16, 32, None) == B.MOE_ERR_SHAPE    # ld < cols
    assert f(_vp(A), _vp(1 << 30), 2, 16, 32, 68, 32, None) == B.MOE_ERR_SHAPE    # ld % 8
    assert f(_vp(A), _vp(1 << 30), 2, 16, 32, 64, -8, None) == B.MOE_ERR_SHAPE
    # the source spans (n-1)*stride + (rows-1)*ld + cols elements: overlap found
    assert f(_vp(A), _vp(A + 2 * (15 * 64 + 64) - 16), 2, 16, 32, 64, 32, None) == B.MOE_ERR_OPTION


def test_empty_batch_host_paths():
    """T = 0: workspace sizes stay positive, NULL T-sized pointers are
    accepted, and calls that need no device work return MOE_OK before any
    HIP call (the fake addresses are never touched)."""
    assert B.workspace_bytes(0, *FLASH[1:]) > 0
    lib = B.load()
    assert lib.moe_dense_workspace_bytes(0, 4096, 11264, 8) > 0
    empty = (0,) + FLASH[1:]
    assert _forward(dims=empty, x=0, y=0) == B.MOE_OK
    assert B.last_error() == ""
    assert _forward(dims=empty, x=0, y=0, W=0) == B.MOE_ERR_NULL      # router still required
    assert _forward(dims=empty, x=0, y=0, ws_bytes=10) == B.MOE_ERR_WORKSPACE
    # a routing output for T = 0 needs only counts and offsets (which the
    # call would zero on the device, so it is exercised on the GPU)
    bad = B.Routing(None, None, None, _vp(A), None, None, None, None)
    assert _forward(dims=empty, x=0, y=0, routing=bad) == B.MOE_ERR_NULL
    ffn = B.Shared(B.MOE_LAYOUT_PACKED, _vp(A), _vp(A), _vp(A))
    need = lib.moe_dense_workspace_bytes(0, 4096, 11264, 8)
    assert lib.moe_dense_ffn(0, 4096, 11264, 8, None, ctypes.byref(ffn), 0.0, None, _vp(A), need,
                             None) == B.MOE_OK
    d = B.dims(*empty)
    assert lib.moe_expert_stats(ctypes.byref(d), _vp(A), _vp(A), _vp(A), None,
                                None) == B.MOE_ERR_SHAPE


def test_mfma_probe_checks():
    """moe_mfma_probe rejects bad arguments on the host, before any HIP call."""
    lib = B.load()
    assert lib.moe_mfma_probe(16, None, 512, _vp(A), None) == B.MOE_ERR_NULL
    assert lib.moe_mfma_probe(16, _vp(A), 512, None, None) == B.MOE_ERR_NULL
    assert lib.moe_mfma_probe(16, _vp(A + 8), 512, _vp(A), None) == B.MOE_ERR_ALIGN
    assert lib.moe_mfma_probe(16, _vp(A), 512, _vp(A + 4), None) == B.MOE_ERR_ALIGN
    assert lib.moe_mfma_probe(0, _vp(A), 512, _vp(A), None) == B.MOE_ERR_SHAPE
    assert lib.moe_mfma_probe((1 << 24) + 1, _vp(A), 512, _vp(A), None) == B.MOE_ERR_SHAPE
    assert "iters" in B.last_error()


def test_read_probe_checks():
    """moe_read_probe rejects bad arguments on the host, before any HIP call."""
    lib = B.load()
    assert lib.moe_read_probe(None, 16384, 1, _vp(A), None) == B.MOE_ERR_NULL
    assert lib.moe_read_probe(_vp(A), 16384, 1, None, None) == B.MOE_ERR_NULL
    assert lib.moe_read_probe(_vp(A + 8), 16384, 1, _vp(A), None) == B.MOE_ERR_ALIGN
    assert lib.moe_read_probe(_vp(A), 16384, 1, _vp(A + 4), None) == B.MOE_ERR_ALIGN
    assert lib.moe_read_probe(_vp(A), 0, 1, _vp(A), None) == B.MOE_ERR_SHAPE
    assert lib.moe_read_probe(_vp(A), 16384 + 16, 0, _vp(A), None) == B.MOE_ERR_SHAPE
    assert "multiple of 16384" in B.last_error()
    assert lib.moe_read_probe(_vp(A), 16384, 2, _vp(A), None) == B.MOE_ERR_OPTION


def test_noalloc_host_checks():
    """moe_forward_noalloc checks its arguments as moe_forward does, and
    refuses a layer whose scratch need exceeds the fixed array, all on the
    host before any HIP call."""
    lib = B.load()
    r = B.Router(_vp(A), _vp(A))
    e = B.Experts(B.MOE_LAYOUT_PACKED, _vp(A), _vp(A), _vp(A))
    sh = B.Shared(B.MOE_LAYOUT_PACKED, _vp(A), _vp(A), _vp(A))
    o = B.make_opts()

    def call(dims=FLASH, x=A, y=2 * A, experts=e, opts=o):
        d = B.dims(*dims)
        return lib.moe_forward_noalloc(ctypes.byref(d), ctypes.byref(opts), _vp(x),
                                       ctypes.byref(r), ctypes.byref(experts), ctypes.byref(sh),
                                       _vp(y), None, None)

    assert call(x=0) == B.MOE_ERR_NULL
    assert call(experts=B.Experts(B.MOE_LAYOUT_ROW_MAJOR, _vp(A), _vp(A), _vp(A))) == B.MOE_ERR_DTYPE
    assert call(dims=(16, 4000) + FLASH[2:]) == B.MOE_ERR_SHAPE
    assert call(opts=B.make_opts(route_scale=-1.0)) == B.MOE_ERR_OPTION
    assert call(y=2 * A + 2) == B.MOE_ERR_ALIGN
    assert call(x=A, y=A) == B.MOE_ERR_OPTION
    T_max = 1
    while B.workspace_bytes(T_max + 1, *FLASH[1:]) <= B.NOALLOC_SCRATCH_BYTES:
        T_max += 1
    assert T_max == 290          # the Flash shape fits up to 290 tokens
    assert call(dims=(T_max + 1,) + FLASH[1:]) == B.MOE_ERR_WORKSPACE
    assert "moe_forward with a workspace" in B.last_error()
