"""Thin ctypes binding of the C ABI in ``include/gs.h`` (same names).

Argument marshalling only: tensors become device pointers, cameras become
``gs_camera`` structs, the current HIP stream is passed through. Every step of
the computation runs in the HIP library; if that library is not built, every
call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgs_hip.so")

GS_OK, GS_ERR_INVALID_ARGUMENT, GS_ERR_CAPACITY, GS_ERR_HIP, GS_ERR_UNSUPPORTED = range(5)
GS_TILE = 16
GS_MAX_VIEWS = 16
GS_REC_FLOATS = 12
GS_GRAD2D_ROWS = 9
GS_ACCUMULATE_LOSS, GS_ACCUMULATE_GRAD2D = 1, 2
ABI_VERSION = 2
(REC_U, REC_V, REC_A, REC_B, REC_C, REC_OPACITY, REC_R, REC_G, REC_BLUE,
 REC_EXT_X, REC_EXT_Y, REC_DEPTH) = range(12)

# every function the header declares, for the export check
EXPORTS = (
    "gs_abi_version", "gs_status_string", "gs_param_rows", "gs_tiles_x", "gs_tiles_y",
    "gs_sort_end_bit", "gs_preprocess_workspace_bytes", "gs_sort_workspace_bytes",
    "gs_tile_lists_workspace_bytes", "gs_rasterize_fwd_l1_workspace_bytes", "gs_rasterize_fwd_bwd_l1_workspace_bytes",
    "gs_preprocess", "gs_emit_intersections", "gs_sort_keys", "gs_tile_lists", "gs_tile_ranges", "gs_tile_masks",
    "gs_tile_masks_workspace_bytes",
    "gs_rasterize_fwd", "gs_rasterize_fwd_l1", "gs_loss_l1", "gs_rasterize_bwd", "gs_rasterize_fwd_bwd_l1",
    "gs_preprocess_bwd", "gs_adam_step", "gs_adam_step_unless", "gs_preprocess_bwd_adam",
    "gs_raster_exp", "gs_stream_copy",
    "gs_rasterize_fwd_bwd_l1_noalloc", "gs_rasterize_fwd_bwd_l1_noalloc_max_bytes",
    "gs_window_gaussians", "gs_window_gaussians_workspace_bytes", "gs_adam_step_visible",
    "gs_seen_gaussians", "gs_seen_gaussians_workspace_bytes", "gs_preprocess_bwd_compact", "gs_adam_step_compact",
)


class GsError(RuntimeError):
    pass


class GsCamera(ctypes.Structure):
    _fields_ = [
        ("width", ctypes.c_int32), ("height", ctypes.c_int32),
        ("fx", ctypes.c_float), ("fy", ctypes.c_float),
        ("cx", ctypes.c_float), ("cy", ctypes.c_float),
        ("R", ctypes.c_float * 9), ("t", ctypes.c_float * 3),
        ("near_plane", ctypes.c_float), ("far_plane", ctypes.c_float),
    ]


_P = ctypes.c_void_p
_I32, _I64, _U64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
_F32, _F64, _SZ = ctypes.c_float, ctypes.c_double, ctypes.c_size_t
_LIB = None


def lib():
    """Load the HIP library (raises when it is not built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise GsError(f"HIP library {LIB_PATH} is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "gs_abi_version": ([], ctypes.c_int),
            "gs_status_string": ([ctypes.c_int], ctypes.c_char_p),
            "gs_param_rows": ([_I32], ctypes.c_int),
            "gs_tiles_x": ([_I32], _I32),
            "gs_tiles_y": ([_I32], _I32),
            "gs_sort_end_bit": ([_I32, _I64], _I32),
            "gs_preprocess_workspace_bytes": ([_I64, _I32], _SZ),
            "gs_sort_workspace_bytes": ([_U64], _SZ),
            "gs_tile_lists_workspace_bytes": ([_I64, _I32, _I32, _I32, _U64], _SZ),
            "gs_rasterize_fwd_l1_workspace_bytes": ([_I32, _I32, _I32], _SZ),
            "gs_rasterize_fwd_bwd_l1_workspace_bytes": ([_I32, _I32, _I32], _SZ),
            "gs_preprocess": ([_P, _I64, _I32, _P, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
            "gs_emit_intersections": ([_P, _P, _P, _I64, _I32, _I32, _I32, _P, _P, _U64, _P, _P], ctypes.c_int),
            "gs_sort_keys": ([_P, _P, _P, _P, _U64, _I32, _P, _SZ, _P, _P], ctypes.c_int),
            "gs_tile_ranges": ([_P, _U64, _I64, _P, _P], ctypes.c_int),
            "gs_tile_lists": ([_P, _P, _P, _P, _P, _I64, _I64, _I32, _I32, _I32, _I32, _I32, _P, _P, _U64, _P, _P, _P,
                               _P, _SZ, _P], ctypes.c_int),
            "gs_window_gaussians_workspace_bytes": ([_I64, _I32], _SZ),
            "gs_window_gaussians": ([_P, _I64, _I32, _I32, _I32, _I32, _P, _P, _P, _SZ, _P], ctypes.c_int),
            "gs_tile_masks_workspace_bytes": ([_U64], _SZ),
            "gs_tile_masks": ([_P, _I64, _P, _P, _U64, _P, _I32, _P, _P, _SZ, _P], ctypes.c_int),
            "gs_rasterize_fwd": ([_P, _I64, _P, _P, _P, _U64, _P, _I32, _I32, _I32, _P, _P, _P, _P, _P],
                                 ctypes.c_int),
            "gs_rasterize_fwd_l1": ([_P, _I64, _P, _P, _P, _U64, _P, _I32, _I32, _I32, _P, _P, _F32, _P, _P, _P, _P,
                                     _P, _I32, _P, _SZ, _P], ctypes.c_int),
            "gs_loss_l1": ([_P, _P, _I64, _F32, _P, _P, _I32, _P], ctypes.c_int),
            "gs_rasterize_fwd_bwd_l1": ([_P, _I64, _P, _P, _P, _U64, _P, _I32, _I32, _I32, _P, _P, _F32, _P, _P,
                                         _P, _P, _P, _P, _I32, _P, _SZ, _P], ctypes.c_int),
            "gs_rasterize_bwd": ([_P, _I64, _P, _P, _P, _U64, _P, _I32, _I32, _I32, _P, _P, _P, _P, _P, _I32, _P],
                                 ctypes.c_int),
            "gs_preprocess_bwd": ([_P, _I64, _I32, _P, _I32, _P, _P, _P, _P, _P], ctypes.c_int),
            "gs_adam_step_visible": ([_P, _P, _P, _P, _I64, _I32, _P, _P, _F64, _F64, _F64, _F64, _I64, _P, _P],
                                     ctypes.c_int),
            "gs_seen_gaussians_workspace_bytes": ([_I64], _SZ),
            "gs_seen_gaussians": ([_P, _I64, _I32, _P, _P, _P, _SZ, _P], ctypes.c_int),
            "gs_preprocess_bwd_compact": ([_P, _I64, _I32, _P, _I32, _P, _P, _P, _P, _I64, _P, _P, _P], ctypes.c_int),
            "gs_adam_step_compact": ([_P, _P, _I64, _P, _P, _P, _P, _I64, _I32, _P, _I32, _P, _F64, _F64, _F64, _F64,
                                      _I64, _P, _P], ctypes.c_int),
            "gs_adam_step": ([_P, _P, _P, _P, _I64, _F64, _F64, _F64, _F64, _I64, _P], ctypes.c_int),
            "gs_adam_step_unless": ([_P, _P, _P, _P, _I64, _F64, _F64, _F64, _F64, _I64, _P, _P], ctypes.c_int),
            "gs_preprocess_bwd_adam": ([_P, _I64, _I32, _P, _I32, _P, _P, _P, _P, _F64, _F64, _F64, _F64, _I64, _P,
                                        _P, _P, _P], ctypes.c_int),
            "gs_rasterize_fwd_bwd_l1_noalloc": ([_P, _I64, _P, _P, _P, _U64, _P, _I32, _I32, _I32, _P, _P, _F32, _P,
                                                 _P, _P, _P, _P, _P, _I32, _P], ctypes.c_int),
            "gs_rasterize_fwd_bwd_l1_noalloc_max_bytes": ([], _SZ),
            "gs_raster_exp": ([_P, _P, _I64, _P], ctypes.c_int),
            "gs_stream_copy": ([_P, _P, _U64, _P], ctypes.c_int),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _LIB = L
    return _LIB


def status_string(status: int) -> str:
    return lib().gs_status_string(status).decode()


def _check(status: int, name: str):
    if status != GS_OK:
        raise GsError(f"{name} failed: {status_string(status)} ({status})")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def cameras(cams: Sequence):
    arr = (GsCamera * len(cams))()
    for k, c in enumerate(cams):
        o = arr[k]
        o.width, o.height = int(c.width), int(c.height)
        o.fx, o.fy, o.cx, o.cy = c.fx, c.fy, c.cx, c.cy
        for i in range(9):
            o.R[i] = c.R[i]
        for i in range(3):
            o.t[i] = c.t[i]
        o.near_plane, o.far_plane = c.near, c.far
    return arr


# ---- queries (host only) ----------------------------------------------------
def abi_version() -> int:
    return lib().gs_abi_version()


def param_rows(sh_degree: int) -> int:
    return lib().gs_param_rows(sh_degree)


def sort_end_bit(n_views: int, tiles_per_view: int) -> int:
    return lib().gs_sort_end_bit(n_views, tiles_per_view)


def preprocess_workspace_bytes(n: int, n_views: int) -> int:
    return lib().gs_preprocess_workspace_bytes(n, n_views)


def sort_workspace_bytes(n_keys: int) -> int:
    return lib().gs_sort_workspace_bytes(n_keys)


def rasterize_fwd_l1_workspace_bytes(n_views: int, width: int, height: int) -> int:
    return lib().gs_rasterize_fwd_l1_workspace_bytes(n_views, width, height)


def rasterize_fwd_bwd_l1_workspace_bytes(n_views: int, width: int, height: int) -> int:
    return lib().gs_rasterize_fwd_bwd_l1_workspace_bytes(n_views, width, height)


def tile_lists_workspace_bytes(n: int, n_views: int, width: int, height: int, capacity: int) -> int:
    return lib().gs_tile_lists_workspace_bytes(n, n_views, width, height, capacity)


# ---- the step ----------------------------------------------------------------
def gs_preprocess(params, n, sh_degree, cams, rec, rect, offsets, total, ws, stream=None, depth=None, grad2d=None):
    """depth (optional): the compact depth copy; grad2d (optional): 2D-gradient
    records zeroed for every visible (view, Gaussian)."""
    cc = cameras(cams)
    _check(lib().gs_preprocess(_ptr(params), n, sh_degree, cc, len(cams), _ptr(rec), _ptr(rect), _ptr(depth),
                               _ptr(grad2d), _ptr(offsets), _ptr(total), _ptr(ws), ws.numel() * ws.element_size(),
                               _stream(stream)), "gs_preprocess")


def gs_emit_intersections(rec, rect, offsets, n, n_views, width, height, keys, vals, capacity,
                          overflow, stream=None):
    _check(lib().gs_emit_intersections(_ptr(rec), _ptr(rect), _ptr(offsets), n, n_views, width, height,
                                       _ptr(keys), _ptr(vals), capacity, _ptr(overflow),
                                       _stream(stream)), "gs_emit_intersections")


def tiles_y(height: int) -> int:
    return int(lib().gs_tiles_y(height))


def _window(height, rows):
    return tiles_y(height) if rows is None else rows


def gs_tile_lists(rec, rect, n, n_views, width, height, vals, capacity, ranges, overflow, ws, masks=None,
                  row0=0, rows=None, stream=None, depth=None, sticky=None, gauss=None, gauss_off=None, set_max=0):
    """masks (optional): the entries' sub-block masks, as gs_tile_masks;
    row0, rows: the window of tile rows (the whole image by default);
    depth (optional): gs_preprocess's compact depths; sticky (optional): a
    device flag set with the overflow and never cleared; gauss, gauss_off
    (optional): gs_window_gaussians' per-view sets to bin; set_max: the
    largest set expected (sizes the binning grid; 0 for all n)."""
    _check(lib().gs_tile_lists(_ptr(rec), _ptr(rect), _ptr(depth), _ptr(gauss), _ptr(gauss_off), set_max, n,
                               n_views, width,
                               height, row0, _window(height, rows),
                               _ptr(vals), _ptr(masks), capacity,
                               _ptr(ranges), _ptr(overflow), _ptr(sticky), _ptr(ws), ws.numel() * ws.element_size(),
                               _stream(stream)), "gs_tile_lists")


def window_gaussians_workspace_bytes(n: int, n_views: int) -> int:
    return lib().gs_window_gaussians_workspace_bytes(n, n_views)


def gs_window_gaussians(rect, n, n_views, height, row0, rows, gauss, gauss_off, ws, stream=None):
    _check(lib().gs_window_gaussians(_ptr(rect), n, n_views, height, row0, rows, _ptr(gauss), _ptr(gauss_off),
                                     _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "gs_window_gaussians")


def gs_sort_keys(keys, vals, keys_alt, vals_alt, n_keys, end_bit, ws, stream=None) -> bool:
    """Returns True when the sorted data ended in the alt pair."""
    alt = ctypes.c_int32(0)
    _check(lib().gs_sort_keys(_ptr(keys), _ptr(vals), _ptr(keys_alt), _ptr(vals_alt), n_keys, end_bit,
                              _ptr(ws), ws.numel() * ws.element_size(), ctypes.byref(alt),
                              _stream(stream)), "gs_sort_keys")
    return bool(alt.value)


def gs_tile_ranges(keys, n_keys, n_tiles_total, ranges, stream=None):
    _check(lib().gs_tile_ranges(_ptr(keys), n_keys, n_tiles_total, _ptr(ranges), _stream(stream)),
           "gs_tile_ranges")


def tile_masks_workspace_bytes(capacity: int) -> int:
    return lib().gs_tile_masks_workspace_bytes(capacity)


def gs_tile_masks(rec, n, ranges, vals, capacity, cams, masks, ws, stream=None):
    _check(lib().gs_tile_masks(_ptr(rec), n, _ptr(ranges), _ptr(vals), capacity, cameras(cams), len(cams),
                               _ptr(masks), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "gs_tile_masks")


def _capacity(vals, masks, capacity):
    """List slots the raster calls may read: the given capacity, else the
    smaller of the two list buffers."""
    if capacity is not None:
        return int(capacity)
    return min(vals.numel(), masks.numel()) if vals is not None and masks is not None else 0


def gs_rasterize_fwd(rec, n, ranges, vals, masks, cams, bg, image, T_final, n_contrib, row0=0, rows=None, stream=None,
                     capacity=None):
    bgv = (ctypes.c_float * 3)(*bg)
    _check(lib().gs_rasterize_fwd(_ptr(rec), n, _ptr(ranges), _ptr(vals), _ptr(masks), _capacity(vals, masks, capacity),
                                  cameras(cams), len(cams), row0,
                                  _window(cams[0].height, rows), bgv,
                                  _ptr(image), _ptr(T_final), _ptr(n_contrib), _stream(stream)),
           "gs_rasterize_fwd")


def gs_rasterize_fwd_l1(rec, n, ranges, vals, masks, cams, bg, target, scale, image, T_final, n_contrib, dL_dimage, loss,
                        ws, accumulate=False, row0=0, rows=None, stream=None, capacity=None):
    """image may be None (not written)."""
    bgv = (ctypes.c_float * 3)(*bg)
    _check(lib().gs_rasterize_fwd_l1(_ptr(rec), n, _ptr(ranges), _ptr(vals), _ptr(masks),
                                     _capacity(vals, masks, capacity), cameras(cams), len(cams),
                                     row0, _window(cams[0].height, rows), bgv,
                                     _ptr(target), scale, _ptr(image), _ptr(T_final), _ptr(n_contrib),
                                     _ptr(dL_dimage), _ptr(loss), int(bool(accumulate)), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)), "gs_rasterize_fwd_l1")


def gs_loss_l1(image, target, count, scale, dL_dimage, loss, accumulate=False, stream=None):
    _check(lib().gs_loss_l1(_ptr(image), _ptr(target), count, scale, _ptr(dL_dimage), _ptr(loss),
                            int(bool(accumulate)), _stream(stream)), "gs_loss_l1")


def gs_rasterize_bwd(rec, n, ranges, vals, masks, cams, bg, T_final, n_contrib, dL_dimage, grad2d,
                     accumulate=False, row0=0, rows=None, stream=None, capacity=None):
    bgv = (ctypes.c_float * 3)(*bg)
    _check(lib().gs_rasterize_bwd(_ptr(rec), n, _ptr(ranges), _ptr(vals), _ptr(masks), _capacity(vals, masks, capacity),
                                  cameras(cams), len(cams), row0,
                                  _window(cams[0].height, rows), bgv,
                                  _ptr(T_final), _ptr(n_contrib), _ptr(dL_dimage), _ptr(grad2d),
                                  int(bool(accumulate)), _stream(stream)), "gs_rasterize_bwd")


def gs_rasterize_fwd_bwd_l1(rec, n, ranges, vals, masks, cams, bg, target, scale, loss, grad2d, ws, image=None,
                            T_final=None, n_contrib=None, dL_dimage=None, accumulate=False, row0=0, rows=None,
                            stream=None, capacity=None, accumulate_grad2d=None):
    """image, T_final, n_contrib and dL_dimage are optional outputs.
    `accumulate` adds to the loss and the 2D gradients; `accumulate_grad2d`,
    when given, decides for the 2D gradients alone (e.g. records zeroed by
    gs_preprocess, with the loss overwritten)."""
    bgv = (ctypes.c_float * 3)(*bg)
    acc_g = accumulate if accumulate_grad2d is None else accumulate_grad2d
    flags = (GS_ACCUMULATE_LOSS if accumulate else 0) | (GS_ACCUMULATE_GRAD2D if acc_g else 0)
    _check(lib().gs_rasterize_fwd_bwd_l1(_ptr(rec), n, _ptr(ranges), _ptr(vals), _ptr(masks),
                                         _capacity(vals, masks, capacity), cameras(cams),
                                         len(cams), row0, _window(cams[0].height, rows), bgv, _ptr(target), scale,
                                         _ptr(image), _ptr(T_final), _ptr(n_contrib), _ptr(dL_dimage), _ptr(loss),
                                         _ptr(grad2d), flags, _ptr(ws),
                                         ws.numel() * ws.element_size(), _stream(stream)), "gs_rasterize_fwd_bwd_l1")


def gs_rasterize_fwd_bwd_l1_noalloc(rec, n, ranges, vals, masks, cams, bg, target, scale, loss, grad2d, image=None,
                                    T_final=None, n_contrib=None, dL_dimage=None, accumulate=False, row0=0, rows=None,
                                    stream=None, capacity=None, accumulate_grad2d=None):
    """gs_rasterize_fwd_bwd_l1 with the library's fixed per-device workspace
    (no workspace argument, nothing allocated)."""
    bgv = (ctypes.c_float * 3)(*bg)
    acc_g = accumulate if accumulate_grad2d is None else accumulate_grad2d
    flags = (GS_ACCUMULATE_LOSS if accumulate else 0) | (GS_ACCUMULATE_GRAD2D if acc_g else 0)
    _check(lib().gs_rasterize_fwd_bwd_l1_noalloc(_ptr(rec), n, _ptr(ranges), _ptr(vals), _ptr(masks),
                                                 _capacity(vals, masks, capacity), cameras(cams), len(cams), row0,
                                                 _window(cams[0].height, rows), bgv, _ptr(target), scale, _ptr(image),
                                                 _ptr(T_final), _ptr(n_contrib), _ptr(dL_dimage), _ptr(loss),
                                                 _ptr(grad2d), flags, _stream(stream)),
           "gs_rasterize_fwd_bwd_l1_noalloc")


def gs_preprocess_bwd(params, n, sh_degree, cams, rect, grad2d, grad_params, stream=None, visible=None):
    """visible (optional, uint8 [n]): sparse output, rows written only for
    Gaussians visible in some view (see the header)."""
    _check(lib().gs_preprocess_bwd(_ptr(params), n, sh_degree, cameras(cams), len(cams), _ptr(rect),
                                   _ptr(grad2d), _ptr(grad_params), _ptr(visible), _stream(stream)),
           "gs_preprocess_bwd")


def gs_adam_step_visible(params, grad, m, v, n, rows, visible, lr, beta1, beta2, eps, step, state=None, skip=None,
                         stream=None):
    _check(lib().gs_adam_step_visible(_ptr(params), _ptr(grad), _ptr(m), _ptr(v), n, rows, _ptr(visible),
                                      _ptr(state), lr, beta1, beta2, eps, step, _ptr(skip), _stream(stream)),
           "gs_adam_step_visible")


def seen_gaussians_workspace_bytes(n: int) -> int:
    return lib().gs_seen_gaussians_workspace_bytes(n)


def gs_seen_gaussians(rect, n, n_views, gauss, count, ws, stream=None):
    _check(lib().gs_seen_gaussians(_ptr(rect), n, n_views, _ptr(gauss), _ptr(count), _ptr(ws),
                                   ws.numel() * ws.element_size(), _stream(stream)), "gs_seen_gaussians")


def gs_preprocess_bwd_compact(params, n, sh_degree, cams, rect, grad2d, gauss, count, stride, grad_compact, overflow,
                              stream=None):
    _check(lib().gs_preprocess_bwd_compact(_ptr(params), n, sh_degree, cameras(cams), len(cams), _ptr(rect),
                                           _ptr(grad2d), _ptr(gauss), _ptr(count), stride, _ptr(grad_compact),
                                           _ptr(overflow), _stream(stream)), "gs_preprocess_bwd_compact")


def gs_adam_step_compact(params, grad_compact, stride, gauss, count, m, v, n, rows, rect, n_views, lr, beta1, beta2,
                         eps, step, state=None, skip=None, stream=None):
    _check(lib().gs_adam_step_compact(_ptr(params), _ptr(grad_compact), stride, _ptr(gauss), _ptr(count), _ptr(m),
                                      _ptr(v), n, rows, _ptr(rect), n_views, _ptr(state), lr, beta1, beta2, eps, step,
                                      _ptr(skip), _stream(stream)), "gs_adam_step_compact")


def gs_adam_step(params, grad, m, v, count, lr, beta1, beta2, eps, step, stream=None):
    _check(lib().gs_adam_step(_ptr(params), _ptr(grad), _ptr(m), _ptr(v), count, lr, beta1, beta2, eps,
                              step, _stream(stream)), "gs_adam_step")


def gs_preprocess_bwd_adam(params, n, sh_degree, cams, rect, grad2d, m, v, lr, beta1, beta2, eps, step, skip=None,
                           grad_params=None, state=None, stream=None):
    """state (optional): uint8 [n], 0 where the Gaussian's moments are zero
    (see the header); never-seen Gaussians are then skipped."""
    _check(lib().gs_preprocess_bwd_adam(_ptr(params), n, sh_degree, cameras(cams), len(cams), _ptr(rect), _ptr(grad2d),
                                        _ptr(m), _ptr(v), lr, beta1, beta2, eps, step, _ptr(skip), _ptr(state),
                                        _ptr(grad_params), _stream(stream)), "gs_preprocess_bwd_adam")


def gs_adam_step_unless(params, grad, m, v, count, lr, beta1, beta2, eps, step, skip, stream=None):
    _check(lib().gs_adam_step_unless(_ptr(params), _ptr(grad), _ptr(m), _ptr(v), count, lr, beta1, beta2, eps,
                                     step, _ptr(skip), _stream(stream)), "gs_adam_step_unless")


def gs_raster_exp(x, y, stream=None):
    """y = the raster passes' exp of x (device fp32 tensors)."""
    _check(lib().gs_raster_exp(_ptr(x), _ptr(y), x.numel(), _stream(stream)), "gs_raster_exp")


def gs_stream_copy(dst, src, nbytes=None, stream=None):
    """Plain device copy of nbytes (default: all of src) from src to dst."""
    nb = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    _check(lib().gs_stream_copy(_ptr(dst), _ptr(src), nb, _stream(stream)), "gs_stream_copy")
