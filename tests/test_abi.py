"""The C ABI without a GPU: the library loads, exports every function
include/gs.h declares, answers its size queries, and rejects invalid arguments
before any HIP call."""

import ctypes
import os
import re

import pytest

from gaussian_splatting_differentiable_ewa_amd import _lib as L
from gaussian_splatting_differentiable_ewa_amd import scenes as S

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "gs.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from gaussian_splatting_differentiable_ewa_amd import build
        build.build()
    return L.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gs_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_function_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 17
    for name in names:
        assert hasattr(lib, name), name
    assert sorted(L.EXPORTS) == names


def test_queries(lib):
    assert L.abi_version() == L.ABI_VERSION == 2
    assert [L.param_rows(d) for d in range(4)] == [S.param_rows(d) for d in range(4)]
    assert L.param_rows(4) == -1
    assert lib.gs_tiles_x(1920) == 120 and lib.gs_tiles_y(1080) == 68 and lib.gs_tiles_x(1) == 1
    # 32 depth bits + bits for view * tiles ids
    assert L.sort_end_bit(4, 8160) == 32 + 15
    assert L.sort_end_bit(1, 256) == 40
    assert L.sort_end_bit(1, 1) == 32
    assert L.preprocess_workspace_bytes(10, 1) > 0
    assert L.sort_workspace_bytes(7_000_000) >= 4 * 256 * (7_000_000 // 2048)
    for s in range(5):
        assert L.status_string(s)


def _cam(**kw):
    c = S.CONFIGS[0].cameras()[0]
    return S.Camera(**{**c.__dict__, **kw})


def _call(f, names, defaults, **kw):
    """Call f with its arguments given by name over a set of valid defaults."""
    unknown = set(kw) - set(names)
    assert not unknown, unknown
    return f(*[kw.get(n, defaults[n]) for n in names])


def test_invalid_arguments_rejected_on_host(lib):
    INV = L.GS_ERR_INVALID_ARGUMENT
    cams = L.cameras(S.CONFIGS[0].cameras())
    fake = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    ws = ctypes.c_size_t(1 << 20)
    # gs_preprocess
    pre_names = ["params", "n", "sh", "cams", "V", "rec", "rect", "depth", "grad2d", "offsets", "total", "ws",
                 "ws_bytes", "stream"]
    pre_ok = dict(params=fake, n=10, sh=0, cams=cams, V=1, rec=fake, rect=fake, depth=None, grad2d=None, offsets=fake,
                  total=fake, ws=fake, ws_bytes=ws, stream=None)

    def pre(**kw):
        return _call(lib.gs_preprocess, pre_names, pre_ok, **kw)

    assert pre(n=-1) == INV
    assert pre(sh=4) == INV
    assert pre(V=0) == INV
    assert pre(V=17) == INV
    assert pre(total=None) == INV
    assert pre(offsets=None, total=None) == INV
    assert pre(offsets=None, ws_bytes=ctypes.c_size_t(3)) == INV  # the wave sums of 10 Gaussians: 4 bytes
    assert pre(ws_bytes=0) == INV
    assert pre(cams=L.cameras([_cam(), _cam(width=128)]), V=2) == INV
    assert pre(cams=L.cameras([_cam(fx=0.0)])) == INV
    assert pre(cams=L.cameras([_cam(width=16 * 70000)])) == INV
    # gs_emit_intersections
    assert lib.gs_emit_intersections(fake, fake, fake, -1, 1, 256, 256, fake, fake, 10, fake, None) == INV
    assert lib.gs_emit_intersections(fake, fake, fake, 10, 1, 0, 256, fake, fake, 10, fake, None) == INV
    assert lib.gs_emit_intersections(fake, fake, fake, 10, 1, 256, 256, fake, fake, 10, None, None) == INV
    assert lib.gs_emit_intersections(fake, fake, fake, 10, 1, 256, 256, None, fake, 10, fake, None) == INV
    # gs_sort_keys
    alt = ctypes.c_int32(7)
    assert lib.gs_sort_keys(fake, fake, fake, fake, 100, 0, fake, ws, ctypes.byref(alt), None) == INV
    assert lib.gs_sort_keys(fake, fake, fake, fake, 100, 65, fake, ws, ctypes.byref(alt), None) == INV
    assert lib.gs_sort_keys(fake, fake, fake, fake, 1 << 32, 40, fake, ws, ctypes.byref(alt), None) == INV
    assert lib.gs_sort_keys(fake, fake, fake, fake, 100, 40, fake, 8, ctypes.byref(alt), None) == INV
    assert lib.gs_sort_keys(fake, fake, fake, fake, 100, 40, fake, ws, None, None) == INV
    assert lib.gs_sort_keys(None, None, None, None, 0, 40, None, 0, ctypes.byref(alt), None) == L.GS_OK
    assert alt.value == 0
    # gs_tile_lists
    big = ctypes.c_size_t(1 << 40)
    tl_names = ["rec", "rect", "depth", "gauss", "gauss_off", "set_max", "n", "V", "W", "H", "row0", "rows", "vals",
                "masks",
                "capacity", "ranges", "overflow", "sticky", "ws", "ws_bytes", "stream"]
    tl_ok = dict(rec=fake, rect=fake, depth=None, gauss=None, gauss_off=None, set_max=0, n=10, V=1, W=256, H=256, row0=0,
                 rows=16, vals=fake, masks=None, capacity=10, ranges=fake, overflow=fake, sticky=None, ws=fake,
                 ws_bytes=big, stream=None)

    def tl(**kw):
        return _call(lib.gs_tile_lists, tl_names, tl_ok, **kw)

    assert tl(n=-1) == INV
    assert tl(V=0) == INV
    assert tl(H=0) == INV
    assert tl(ranges=None) == INV
    assert tl(overflow=None) == INV
    assert tl(vals=None) == INV
    assert tl(capacity=1 << 32) == INV
    assert tl(row0=12, rows=5) == INV
    need = L.tile_lists_workspace_bytes(10, 1, 256, 256, 10)
    assert need > 0 and L.tile_lists_workspace_bytes(10, 0, 256, 256, 10) == 0
    assert L.tile_lists_workspace_bytes(10, 1, 16 * 8193, 256, 10) == 0
    assert tl(ws_bytes=need - 1) == INV
    assert tl(gauss=fake) == INV  # a set without its offsets
    assert tl(set_max=5) == INV  # a set size without a set
    assert tl(gauss=fake, gauss_off=fake, set_max=-1) == INV
    # gs_window_gaussians
    wws = L.window_gaussians_workspace_bytes(1000, 2)
    assert wws > 0 and L.window_gaussians_workspace_bytes(-1, 2) == 0
    wg = lib.gs_window_gaussians
    assert wg(fake, 1000, 2, 256, 12, 5, fake, fake, fake, wws, None) == INV  # window past the 16 tile rows
    assert wg(fake, 1000, 2, 256, 0, 16, fake, None, fake, wws, None) == INV
    assert wg(fake, 1000, 2, 256, 0, 16, fake, fake, fake, wws - 4, None) == INV
    assert wg(fake, -1, 2, 256, 0, 16, fake, fake, fake, wws, None) == INV
    assert wg(fake, 1000, 0, 256, 0, 16, fake, fake, fake, wws, None) == INV
    # gs_seen_gaussians
    sws = L.seen_gaussians_workspace_bytes(1000)
    assert sws > 0 and L.seen_gaussians_workspace_bytes(-1) == 0
    sg = lib.gs_seen_gaussians
    assert sg(fake, 1000, 2, fake, fake, fake, sws - 4, None) == INV
    assert sg(fake, 1000, 2, fake, None, fake, sws, None) == INV
    assert sg(fake, 1000, 2, None, fake, fake, sws, None) == INV
    assert sg(fake, -1, 2, fake, fake, fake, sws, None) == INV
    assert sg(fake, 1000, 17, fake, fake, fake, sws, None) == INV
    assert sg(fake, (1 << 31) + 1, 1, fake, fake, fake, 1 << 40, None) == INV
    # gs_tile_ranges
    assert lib.gs_tile_ranges(fake, 10, -1, fake, None) == INV
    assert lib.gs_tile_ranges(None, 10, 4, fake, None) == INV
    # raster: every call takes the list capacity, < 2^32, and needs vals and
    # masks when it is non-zero
    bg = (ctypes.c_float * 3)(0, 0, 0)
    qws = L.rasterize_fwd_l1_workspace_bytes(1, 256, 256)
    assert qws == 16 * 16 * 4 * 8 + 258 * 8 and L.rasterize_fwd_l1_workspace_bytes(0, 256, 256) == 0
    head = ["rec", "n", "ranges", "vals", "masks", "capacity", "cams", "V", "row0", "rows", "bg"]
    head_ok = dict(rec=fake, n=10, ranges=fake, vals=fake, masks=fake, capacity=100, cams=cams, V=1, row0=0, rows=16,
                   bg=bg)

    def common_cases(f):
        assert f(n=-5) == INV
        assert f(masks=None) == INV
        assert f(vals=None) == INV
        assert f(capacity=1 << 32) == INV
        assert f(bg=None) == INV
        assert f(V=0) == INV
        assert f(row0=8, rows=9) == INV  # a window outside the 16 tile rows of a 256-pixel image
        assert f(row0=-1, rows=4) == INV
        assert f(rows=0) == INV

    fwd_names = head + ["image", "T_final", "n_contrib", "stream"]
    fwd_ok = dict(head_ok, image=fake, T_final=fake, n_contrib=fake, stream=None)

    def fwd(**kw):
        return _call(lib.gs_rasterize_fwd, fwd_names, fwd_ok, **kw)

    common_cases(fwd)
    assert fwd(image=None) == INV
    assert fwd(n_contrib=None) == INV

    l1_names = head + ["target", "scale", "image", "T_final", "n_contrib", "dL", "loss", "accumulate", "ws",
                       "ws_bytes", "stream"]
    l1_ok = dict(head_ok, target=fake, scale=1.0, image=None, T_final=fake, n_contrib=fake, dL=fake, loss=fake,
                 accumulate=0, ws=fake, ws_bytes=qws, stream=None)

    def l1(**kw):
        return _call(lib.gs_rasterize_fwd_l1, l1_names, l1_ok, **kw)

    common_cases(l1)
    assert l1(target=None) == INV
    assert l1(dL=None) == INV
    assert l1(loss=None) == INV
    assert l1(ws=None) == INV
    assert l1(ws_bytes=qws - 8) == INV

    bwd_names = head + ["T_final", "n_contrib", "dL", "grad2d", "accumulate", "stream"]
    bwd_ok = dict(head_ok, T_final=fake, n_contrib=fake, dL=fake, grad2d=fake, accumulate=0, stream=None)

    def bwd(**kw):
        return _call(lib.gs_rasterize_bwd, bwd_names, bwd_ok, **kw)

    common_cases(bwd)
    assert bwd(dL=None) == INV
    assert bwd(grad2d=None) == INV

    fws = L.rasterize_fwd_bwd_l1_workspace_bytes(1, 256, 256)
    assert fws == 16 * 16 * (4 * 8 + 4) + 258 * 8 + 8 * 4 and L.rasterize_fwd_bwd_l1_workspace_bytes(1, 0, 256) == 0
    fb_names = head + ["target", "scale", "image", "T_final", "n_contrib", "dL", "loss", "grad2d", "accumulate", "ws",
                       "ws_bytes", "stream"]
    fb_ok = dict(head_ok, target=fake, scale=1.0, image=None, T_final=None, n_contrib=None, dL=None, loss=fake,
                 grad2d=fake, accumulate=0, ws=fake, ws_bytes=fws, stream=None)

    def fb(**kw):
        return _call(lib.gs_rasterize_fwd_bwd_l1, fb_names, fb_ok, **kw)

    common_cases(fb)
    assert fb(target=None) == INV
    assert fb(loss=None) == INV
    assert fb(grad2d=None) == INV
    assert fb(ws=None) == INV
    assert fb(ws_bytes=fws - 4) == INV
    assert fb(accumulate=4) == INV  # only GS_ACCUMULATE_LOSS | GS_ACCUMULATE_GRAD2D
    assert fb(accumulate=-1) == INV
    # the allocation-free form: the same checks, and windows whose workspace
    # exceeds the fixed array are refused before any HIP call
    na_names = [n_ for n_ in fb_names if n_ not in ("ws", "ws_bytes")]
    na_ok = {k: v for k, v in fb_ok.items() if k not in ("ws", "ws_bytes")}

    def na(**kw):
        return _call(lib.gs_rasterize_fwd_bwd_l1_noalloc, na_names, na_ok, **kw)

    common_cases(na)
    assert na(target=None) == INV and na(loss=None) == INV and na(grad2d=None) == INV
    assert na(accumulate=4) == INV
    assert lib.gs_rasterize_fwd_bwd_l1_noalloc_max_bytes() == 8 << 20
    big4k = L.cameras([_cam(width=3840, height=2160)] * 8)  # 8 x 32400 tiles: 9.3 MB of workspace
    assert na(cams=big4k, V=8, rows=135) == L.GS_ERR_CAPACITY
    # the diagnostic exp path and the plain copy
    assert lib.gs_raster_exp(None, fake, 10, None) == INV
    assert lib.gs_raster_exp(fake, fake, -1, None) == INV
    assert lib.gs_raster_exp(None, None, 0, None) == L.GS_OK
    assert lib.gs_stream_copy(fake, fake, 24, None) == INV  # not a multiple of 16
    assert lib.gs_stream_copy(ctypes.c_void_p(24), fake, 32, None) == INV  # misaligned
    assert lib.gs_stream_copy(None, fake, 32, None) == INV
    assert lib.gs_stream_copy(None, None, 0, None) == L.GS_OK
    # tile masks
    mws = L.tile_masks_workspace_bytes(100)
    assert mws == 400
    assert lib.gs_tile_masks(fake, 10, fake, fake, 100, cams, 1, None, fake, mws, None) == INV
    assert lib.gs_tile_masks(fake, 10, None, fake, 100, cams, 1, fake, fake, mws, None) == INV
    assert lib.gs_tile_masks(fake, -1, fake, fake, 100, cams, 1, fake, fake, mws, None) == INV
    assert lib.gs_tile_masks(fake, 10, fake, fake, 100, cams, 0, fake, fake, mws, None) == INV
    assert lib.gs_tile_masks(fake, 10, fake, fake, 100, cams, 1, fake, fake, mws - 4, None) == INV
    assert lib.gs_tile_masks(fake, 10, fake, fake, 1 << 32, cams, 1, fake, fake, 1 << 40, None) == INV
    # loss, preprocess_bwd, adam
    assert lib.gs_loss_l1(fake, fake, -1, 1.0, fake, fake, 0, None) == INV
    assert lib.gs_loss_l1(fake, fake, 10, 1.0, fake, None, 0, None) == INV
    assert lib.gs_loss_l1(ctypes.c_void_p(20), fake, 10, 1.0, fake, fake, 0, None) == INV  # misaligned
    assert lib.gs_preprocess_bwd(fake, 10, 5, cams, 1, fake, fake, fake, None, None) == INV
    assert lib.gs_preprocess_bwd(fake, 10, 3, cams, 1, None, fake, fake, None, None) == INV
    # the compact backward: a list, its count, a stride >= 1 and the overflow flag
    pc = lib.gs_preprocess_bwd_compact
    assert pc(fake, 10, 3, cams, 1, fake, fake, fake, fake, 0, fake, fake, None) == INV
    assert pc(fake, 10, 3, cams, 1, fake, fake, None, fake, 4, fake, fake, None) == INV
    assert pc(fake, 10, 3, cams, 1, fake, fake, fake, None, 4, fake, fake, None) == INV
    assert pc(fake, 10, 3, cams, 1, fake, fake, fake, fake, 4, None, fake, None) == INV
    assert pc(fake, 10, 3, cams, 1, fake, fake, fake, fake, 4, fake, None, None) == INV
    assert pc(fake, 10, 4, cams, 1, fake, fake, fake, fake, 4, fake, fake, None) == INV
    assert pc(fake, 10, 3, cams, 0, fake, fake, fake, fake, 4, fake, fake, None) == INV
    assert pc(fake, 10, 3, cams, 1, None, fake, fake, fake, 4, fake, fake, None) == INV
    assert pc(fake, -1, 3, cams, 1, fake, fake, fake, fake, 4, fake, fake, None) == INV
    ac = lib.gs_adam_step_compact
    ac_names = ["params", "grad", "stride", "list", "count", "m", "v", "n", "rows", "rect", "V", "state", "lr", "b1",
                "b2", "eps", "step", "skip", "stream"]
    ac_ok = dict(params=fake, grad=fake, stride=4, list=fake, count=fake, m=fake, v=fake, n=10, rows=59, rect=fake,
                 V=1, state=None, lr=1e-3, b1=0.9, b2=0.999, eps=1e-15, step=1, skip=None, stream=None)

    def acc(**kw):
        return _call(ac, ac_names, ac_ok, **kw)

    assert acc(stride=0) == INV
    assert acc(list=None) == INV
    assert acc(count=None) == INV
    assert acc(grad=None) == INV
    assert acc(rect=None) == INV
    assert acc(m=None) == INV
    assert acc(rows=0) == INV
    assert acc(rows=262141) == INV
    assert acc(n=-1) == INV
    assert acc(V=17) == INV
    assert acc(step=0) == INV
    assert acc(b2=1.0) == INV
    assert acc(eps=-1.0) == INV
    assert acc(state=fake, eps=0.0) == INV
    assert acc(n=(1 << 31) + 1) == INV
    av = lib.gs_adam_step_visible
    assert av(fake, fake, fake, fake, 10, 59, None, None, 1e-3, 0.9, 0.999, 1e-15, 1, None, None) == INV  # flags
    assert av(fake, fake, fake, fake, 10, 0, fake, None, 1e-3, 0.9, 0.999, 1e-15, 1, None, None) == INV
    assert av(fake, fake, fake, fake, -1, 59, fake, None, 1e-3, 0.9, 0.999, 1e-15, 1, None, None) == INV
    assert av(fake, fake, fake, fake, 10, 59, fake, None, 1e-3, 0.9, 0.999, 1e-15, 0, None, None) == INV
    assert av(fake, fake, fake, fake, 10, 59, fake, fake, 1e-3, 0.9, 0.999, 0.0, 1, None, None) == INV  # state, eps 0
    assert av(fake, None, fake, fake, 10, 59, fake, None, 1e-3, 0.9, 0.999, 1e-15, 1, None, None) == INV
    assert lib.gs_adam_step(fake, fake, fake, fake, 10, 1e-3, 0.9, 0.999, 1e-15, 0, None) == INV
    assert lib.gs_adam_step(fake, fake, fake, fake, 10, 1e-3, 1.0, 0.999, 1e-15, 1, None) == INV
    assert lib.gs_adam_step(fake, fake, fake, fake, -1, 1e-3, 0.9, 0.999, 1e-15, 1, None) == INV
    assert lib.gs_adam_step(fake, fake, fake, fake, 10, 1e-3, 0.9, 0.999, -1.0, 1, None) == INV
    assert lib.gs_adam_step(None, fake, fake, fake, 10, 1e-3, 0.9, 0.999, 1e-15, 1, None) == INV
    # the fused preprocess backward + Adam: both checks apply
    assert lib.gs_preprocess_bwd_adam(fake, 10, 3, cams, 1, fake, fake, None, fake, 1e-3, 0.9, 0.999, 1e-15, 1,
                                      None, None, None, None) == INV
    assert lib.gs_preprocess_bwd_adam(fake, 10, 3, cams, 1, fake, fake, fake, fake, 1e-3, 0.9, 0.999, 1e-15, 0,
                                      None, None, None, None) == INV
    assert lib.gs_preprocess_bwd_adam(fake, 10, 3, cams, 1, fake, fake, fake, fake, 1e-3, 1.5, 0.999, 1e-15, 1,
                                      None, None, None, None) == INV
    assert lib.gs_preprocess_bwd_adam(fake, 10, 4, cams, 1, fake, fake, fake, fake, 1e-3, 0.9, 0.999, 1e-15, 1,
                                      None, None, None, None) == INV
    # the guarded variant needs its flag, and checks the same arguments
    assert lib.gs_adam_step_unless(fake, fake, fake, fake, 10, 1e-3, 0.9, 0.999, 1e-15, 1, None, None) == INV
    assert lib.gs_adam_step_unless(fake, fake, fake, fake, 10, 1e-3, 0.9, 0.999, 1e-15, 0, fake, None) == INV
    assert lib.gs_adam_step_unless(None, fake, fake, fake, 10, 1e-3, 0.9, 0.999, 1e-15, 1, fake, None) == INV


def test_product_path_does_not_reach_the_oracle():
    """The package never imports the oracle (it is test infrastructure)."""
    import subprocess
    import sys
    root = os.path.dirname(HEADER).rsplit(os.sep, 1)[0]
    code = ("import sys; import gaussian_splatting_differentiable_ewa_amd.step, "
            "gaussian_splatting_differentiable_ewa_amd._lib; "
            "assert not any(m == 'oracle' or m.startswith('oracle.') for m in sys.modules), 'oracle imported'")
    subprocess.run([sys.executable, "-c", code], cwd=root, check=True)
    pkg = os.path.join(root, "gaussian_splatting_differentiable_ewa_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in src and "from oracle" not in src, f
                assert "liboracle" not in src, f
