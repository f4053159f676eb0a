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
    assert L.abi_version() == 1
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


def test_invalid_arguments_rejected_on_host(lib):
    INV = L.GS_ERR_INVALID_ARGUMENT
    cams = L.cameras(S.CONFIGS[0].cameras())
    fake = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    ws = ctypes.c_size_t(1 << 20)
    # gs_preprocess
    assert lib.gs_preprocess(fake, -1, 0, cams, 1, fake, fake, None, fake, fake, fake, ws, None) == INV
    assert lib.gs_preprocess(fake, 10, 4, cams, 1, fake, fake, None, fake, fake, fake, ws, None) == INV
    assert lib.gs_preprocess(fake, 10, 0, cams, 0, fake, fake, None, fake, fake, fake, ws, None) == INV
    assert lib.gs_preprocess(fake, 10, 0, cams, 17, fake, fake, None, fake, fake, fake, ws, None) == INV
    assert lib.gs_preprocess(fake, 10, 0, cams, 1, fake, fake, None, None, fake, fake, ws, None) == INV
    assert lib.gs_preprocess(fake, 10, 0, cams, 1, fake, fake, None, fake, fake, fake, 0, None) == INV
    two = L.cameras([_cam(), _cam(width=128)])
    assert lib.gs_preprocess(fake, 10, 0, two, 2, fake, fake, None, fake, fake, fake, ws, None) == INV
    bad_f = L.cameras([_cam(fx=0.0)])
    assert lib.gs_preprocess(fake, 10, 0, bad_f, 1, fake, fake, None, fake, fake, fake, ws, None) == INV
    huge = L.cameras([_cam(width=16 * 70000)])
    assert lib.gs_preprocess(fake, 10, 0, huge, 1, fake, fake, None, fake, fake, fake, ws, None) == INV
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
    assert lib.gs_tile_lists(fake, fake, None, -1, 1, 256, 256, 0, 16, fake, None, 10, fake, fake, fake, big, None) == INV
    assert lib.gs_tile_lists(fake, fake, None, 10, 0, 256, 256, 0, 16, fake, None, 10, fake, fake, fake, big, None) == INV
    assert lib.gs_tile_lists(fake, fake, None, 10, 1, 256, 0, 0, 16, fake, None, 10, fake, fake, fake, big, None) == INV
    assert lib.gs_tile_lists(fake, fake, None, 10, 1, 256, 256, 0, 16, fake, None, 10, None, fake, fake, big, None) == INV
    assert lib.gs_tile_lists(fake, fake, None, 10, 1, 256, 256, 0, 16, fake, None, 10, fake, None, fake, big, None) == INV
    assert lib.gs_tile_lists(fake, fake, None, 10, 1, 256, 256, 0, 16, None, None, 10, fake, fake, fake, big, None) == INV
    assert lib.gs_tile_lists(fake, fake, None, 10, 1, 256, 256, 0, 16, fake, None, 1 << 32, fake, fake, fake, big, None) == INV
    need = L.tile_lists_workspace_bytes(10, 1, 256, 256, 10)
    assert need > 0 and L.tile_lists_workspace_bytes(10, 0, 256, 256, 10) == 0
    assert L.tile_lists_workspace_bytes(10, 1, 16 * 8193, 256, 10) == 0
    assert lib.gs_tile_lists(fake, fake, None, 10, 1, 256, 256, 0, 16, fake, None, 10, fake, fake, fake, need - 1, None) == INV
    # gs_tile_ranges
    assert lib.gs_tile_ranges(fake, 10, -1, fake, None) == INV
    assert lib.gs_tile_ranges(None, 10, 4, fake, None) == INV
    # raster
    bg = (ctypes.c_float * 3)(0, 0, 0)
    qws = L.rasterize_fwd_l1_workspace_bytes(1, 256, 256)
    assert qws == 16 * 16 * 4 * 8 and L.rasterize_fwd_l1_workspace_bytes(0, 256, 256) == 0
    f1 = lib.gs_rasterize_fwd_l1
    assert f1(fake, 10, fake, fake, fake, cams, 1, 0, 16, bg, None, 1.0, None, fake, fake, fake, fake, 0, fake, qws, None) == INV
    assert f1(fake, 10, fake, fake, fake, cams, 1, 0, 16, bg, fake, 1.0, None, fake, fake, None, fake, 0, fake, qws, None) == INV
    assert f1(fake, 10, fake, fake, fake, cams, 1, 0, 16, bg, fake, 1.0, None, fake, fake, fake, None, 0, fake, qws, None) == INV
    assert f1(fake, 10, fake, fake, fake, cams, 1, 0, 16, bg, fake, 1.0, None, fake, fake, fake, fake, 0, fake,
              qws - 8, None) == INV
    # windows of tile rows outside the 16 rows of a 256-pixel image
    assert f1(fake, 10, fake, fake, fake, cams, 1, 8, 9, bg, fake, 1.0, None, fake, fake, fake, fake, 0, fake, qws,
              None) == INV
    assert lib.gs_rasterize_fwd(fake, 10, fake, fake, fake, cams, 1, 0, 0, bg, fake, fake, fake, None) == INV
    assert lib.gs_rasterize_bwd(fake, 10, fake, fake, fake, cams, 1, -1, 4, bg, fake, fake, fake, fake, 0, None) == INV
    assert lib.gs_tile_lists(fake, fake, None, 10, 1, 256, 256, 12, 5, fake, None, 10, fake, fake, fake, big, None) == INV
    assert f1(fake, 10, fake, fake, fake, cams, 1, 0, 16, bg, fake, 1.0, None, fake, fake, fake, fake, 0, None, qws, None) == INV
    assert f1(fake, 10, fake, fake, None, cams, 1, 0, 16, bg, fake, 1.0, None, fake, fake, fake, fake, 0, fake, qws, None) == INV
    assert lib.gs_rasterize_fwd(fake, 10, fake, fake, fake, cams, 1, 0, 16, None, fake, fake, fake, None) == INV
    assert lib.gs_rasterize_fwd(fake, 10, fake, fake, fake, cams, 1, 0, 16, bg, None, fake, fake, None) == INV
    assert lib.gs_rasterize_fwd(fake, -5, fake, fake, fake, cams, 1, 0, 16, bg, fake, fake, fake, None) == INV
    assert lib.gs_rasterize_fwd(fake, 10, fake, fake, None, cams, 1, 0, 16, bg, fake, fake, fake, None) == INV  # no masks
    assert lib.gs_rasterize_bwd(fake, 10, fake, fake, fake, cams, 1, 0, 16, bg, fake, fake, None, fake, 0, None) == INV
    assert lib.gs_rasterize_bwd(fake, 10, fake, fake, fake, cams, 0, 0, 16, bg, fake, fake, fake, fake, 0, None) == INV
    assert lib.gs_rasterize_bwd(fake, 10, fake, fake, None, cams, 1, 0, 16, bg, fake, fake, fake, fake, 0, None) == INV
    f2 = lib.gs_rasterize_fwd_bwd_l1
    fws = L.rasterize_fwd_bwd_l1_workspace_bytes(1, 256, 256)
    assert fws == 16 * 16 * (4 * 8 + 4) + 8 * 4 and L.rasterize_fwd_bwd_l1_workspace_bytes(1, 0, 256) == 0
    ok = (fake, 10, fake, fake, fake, cams, 1, 0, 16, bg, fake, 1.0, None, None, None, None, fake, fake, 0, fake, fws,
          None)

    def fb(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f2(*a)

    assert fb(a10=None) == INV  # target
    assert fb(a16=None) == INV  # loss
    assert fb(a17=None) == INV  # grad2d
    assert fb(a19=None) == INV  # workspace
    assert fb(a20=fws - 4) == INV
    assert fb(a4=None) == INV  # masks
    assert fb(a7=8, a8=9) == INV  # window outside the image
    assert fb(a6=0) == INV  # no views
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
    assert lib.gs_preprocess_bwd(fake, 10, 5, cams, 1, fake, fake, fake, None) == INV
    assert lib.gs_preprocess_bwd(fake, 10, 3, cams, 1, None, fake, fake, None) == INV
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
