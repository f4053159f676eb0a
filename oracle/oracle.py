"""TEST INFRASTRUCTURE ONLY: Python front of the CPU oracle (ctypes over
liboracle.so). Only tests, the smoke check and the benchmark's CPU-baseline leg
import this module; the product path never does.

Every function takes numpy arrays and returns numpy arrays. ``precision``
selects the fp32 parity build (decisions in fp32 in the pinned order, gradients
accumulated in fp64) or the fp64 build (finite differences).
"""

from __future__ import annotations

import ctypes
import os
from typing import Dict, Sequence

import numpy as np

from . import build as _build

REC_U, REC_V, REC_Z, REC_A2, REC_B2, REC_C2, REC_CA, REC_CB, REC_CC, REC_O = range(10)
REC_RGB = slice(10, 13)
INT_VIS, INT_RAD, INT_X0, INT_Y0, INT_X1, INT_Y1, INT_COUNT, INT_FLAGS = range(8)


class OrCamera(ctypes.Structure):
    _fields_ = [
        ("width", ctypes.c_int32), ("height", ctypes.c_int32),
        ("fx", ctypes.c_float), ("fy", ctypes.c_float),
        ("cx", ctypes.c_float), ("cy", ctypes.c_float),
        ("R", ctypes.c_float * 9), ("t", ctypes.c_float * 3),
        ("near_plane", ctypes.c_float), ("far_plane", ctypes.c_float),
    ]


_LIB = None


def lib():
    global _LIB
    if _LIB is None:
        path = _build.LIB
        if not os.path.exists(path):
            _build.build()
        _LIB = ctypes.CDLL(path)
        _declare(_LIB)
    return _LIB


P = ctypes.c_void_p
I64 = ctypes.c_int64
I32 = ctypes.c_int


def _declare(L):
    for sfx in ("f32", "f64"):
        getattr(L, "or_preprocess_" + sfx).argtypes = [P, I64, I32, P, I32, P, P]
        getattr(L, "or_render_fwd_" + sfx).argtypes = [P, P, I64, P, I32, P, P, P, P, P, P]
        getattr(L, "or_loss_l1_" + sfx).argtypes = [P, P, I64, I32, P]
        getattr(L, "or_loss_l1_" + sfx).restype = ctypes.c_double
        getattr(L, "or_render_bwd_" + sfx).argtypes = [P, P, I64, P, I32, P, P, P, P]
        getattr(L, "or_preprocess_bwd_" + sfx).argtypes = [P, I64, I32, P, I32, P, P]
    L.or_emit_sorted.argtypes = [P, P, P, I64, I32, I32, I32, P, P, I64]
    L.or_emit_sorted.restype = I64
    L.or_tile_ranges.argtypes = [P, I64, I64, P]
    L.or_exclusive_scan.argtypes = [P, I64, P]
    L.or_adam.argtypes = [P, P, P, P, I64, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                          ctypes.c_double, I64]
    L.or_set_threads.argtypes = [I32]
    L.or_exp_band.argtypes = [ctypes.c_float]
    L.or_exp_band.restype = ctypes.c_double
    L.or_alpha_band.argtypes = [ctypes.c_float]
    L.or_alpha_band.restype = ctypes.c_double
    L.or_exp_libm_rel.restype = ctypes.c_double
    L.or_exp_hw_ulp.restype = ctypes.c_double
    L.or_set_band_scale.argtypes = [ctypes.c_double]
    L.or_set_exp_perturb.argtypes = [I32]
    L.or_expf_batch.argtypes = [P, P, I64]
    L.or_exp_band_batch.argtypes = [P, P, I64]
    assert L.or_camera_bytes() == ctypes.sizeof(OrCamera)


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "arrays passed to the oracle must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _dtype(precision):
    return {"f32": np.float32, "f64": np.float64}[precision]


def cameras(cams: Sequence) -> ctypes.Array:
    arr = (OrCamera * len(cams))()
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


def preprocess(params: np.ndarray, sh_degree: int, cams: Sequence, precision: str = "f32") -> Dict:
    """Project all Gaussians into all views. Returns ``rec`` [V][N][16] and
    ``iv`` [V][N][8] (see gs_oracle_body.h for the fields)."""
    L = lib()
    dt = _dtype(precision)
    params = np.ascontiguousarray(params, dtype=dt)
    n = params.shape[1]
    V = len(cams)
    rec = np.zeros((V, n, L.or_rec_stride()), dtype=dt)
    iv = np.zeros((V, n, L.or_int_stride()), dtype=np.int32)
    cc = cameras(cams)
    getattr(L, "or_preprocess_" + precision)(_ptr(params), n, sh_degree, cc, V, _ptr(rec), _ptr(iv))
    return {"rec": rec, "iv": iv, "n": n, "V": V}


def render_fwd(proj: Dict, cams: Sequence, bg=(0.0, 0.0, 0.0), precision: str = "f32") -> Dict:
    L = lib()
    dt = _dtype(precision)
    V, n = proj["V"], proj["n"]
    H, W = cams[0].height, cams[0].width
    image = np.zeros((V, 3, H, W), dtype=dt)
    T = np.zeros((V, H, W), dtype=dt)
    nc = np.zeros((V, H, W), dtype=np.int32)
    amb = np.zeros((V, H, W), dtype=np.uint8)
    sig = np.zeros((V, H, W), dtype=np.uint64)
    bgv = np.asarray(bg, dtype=np.float32)
    getattr(L, "or_render_fwd_" + precision)(
        _ptr(proj["rec"]), _ptr(proj["iv"]), n, cameras(cams), V, _ptr(bgv),
        _ptr(image), _ptr(T), _ptr(nc), _ptr(amb), _ptr(sig))
    return {"image": image, "T_final": T, "n_contrib": nc, "amb": amb, "sig": sig}


def loss_l1(image: np.ndarray, target: np.ndarray, precision: str = "f32"):
    L = lib()
    dt = _dtype(precision)
    image = np.ascontiguousarray(image, dtype=dt)
    target = np.ascontiguousarray(target, dtype=dt)
    V = image.shape[0]
    per_view = image[0].size
    dL = np.zeros_like(image)
    loss = getattr(L, "or_loss_l1_" + precision)(_ptr(image), _ptr(target), per_view, V, _ptr(dL))
    return loss, dL


def render_bwd(proj: Dict, cams: Sequence, dL_dimage: np.ndarray, bg=(0.0, 0.0, 0.0),
               precision: str = "f32", with_abs: bool = False):
    """Gradients w.r.t. the 2D quantities, ``[V][N][9]`` fp64:
    du dv dA dB dC dopacity dr dg db."""
    L = lib()
    dt = _dtype(precision)
    V, n = proj["V"], proj["n"]
    dL = np.ascontiguousarray(dL_dimage, dtype=dt)
    g2 = np.zeros((V, n, 9), dtype=np.float64)
    gabs = np.zeros((V, n, 9), dtype=np.float64) if with_abs else None
    bgv = np.asarray(bg, dtype=np.float32)
    getattr(L, "or_render_bwd_" + precision)(
        _ptr(proj["rec"]), _ptr(proj["iv"]), n, cameras(cams), V, _ptr(bgv), _ptr(dL), _ptr(g2),
        _ptr(gabs) if gabs is not None else None)
    return (g2, gabs) if with_abs else g2


def preprocess_bwd(params: np.ndarray, sh_degree: int, cams: Sequence, grad2d: np.ndarray,
                   precision: str = "f32") -> np.ndarray:
    """Parameter gradients ``[P][N]`` fp64, summed over views."""
    L = lib()
    dt = _dtype(precision)
    params = np.ascontiguousarray(params, dtype=dt)
    n = params.shape[1]
    g2 = np.ascontiguousarray(grad2d, dtype=np.float64)
    out = np.zeros((params.shape[0], n), dtype=np.float64)
    getattr(L, "or_preprocess_bwd_" + precision)(_ptr(params), n, sh_degree, cameras(cams),
                                                 len(cams), _ptr(g2), _ptr(out))
    return out


def rects(proj: Dict):
    """rect [V][N][4] int32 (x0 y0 x1 y1), visible [V][N] uint8, z [V][N] fp32."""
    iv = proj["iv"]
    rect = np.ascontiguousarray(iv[..., INT_X0:INT_Y1 + 1])
    vis = np.ascontiguousarray(iv[..., INT_VIS].astype(np.uint8))
    z = np.ascontiguousarray(proj["rec"][..., REC_Z].astype(np.float32))
    return rect, vis, z


def emit_sorted(rect: np.ndarray, visible: np.ndarray, z: np.ndarray, tiles_x: int, tiles_y: int):
    """All intersection keys in sorted order and their Gaussian ids."""
    L = lib()
    rect = np.ascontiguousarray(rect, dtype=np.int32)
    visible = np.ascontiguousarray(visible, dtype=np.uint8)
    z = np.ascontiguousarray(z, dtype=np.float32)
    V, n = visible.shape
    K = L.or_emit_sorted(_ptr(rect), _ptr(visible), _ptr(z), n, V, tiles_x, tiles_y, None, None, 0)
    keys = np.zeros(max(K, 1), dtype=np.uint64)
    vals = np.zeros(max(K, 1), dtype=np.uint32)
    K2 = L.or_emit_sorted(_ptr(rect), _ptr(visible), _ptr(z), n, V, tiles_x, tiles_y,
                          _ptr(keys), _ptr(vals), K)
    assert K2 == K
    return keys[:K], vals[:K]


def tile_ranges(keys: np.ndarray, n_tiles_total: int) -> np.ndarray:
    L = lib()
    keys = np.ascontiguousarray(keys, dtype=np.uint64)
    out = np.zeros((n_tiles_total, 2), dtype=np.uint32)
    L.or_tile_ranges(_ptr(keys) if keys.size else None, keys.size, n_tiles_total, _ptr(out))
    return out


def exclusive_scan(counts: np.ndarray) -> np.ndarray:
    L = lib()
    counts = np.ascontiguousarray(counts, dtype=np.uint32).reshape(-1)
    out = np.zeros(counts.size + 1, dtype=np.uint64)
    L.or_exclusive_scan(_ptr(counts), counts.size, _ptr(out))
    return out


def adam(theta, g, m, v, lr, b1, b2, eps, step):
    """Returns updated copies (theta, m, v), fp32."""
    L = lib()
    th = np.array(theta, dtype=np.float32, copy=True, order="C")
    mm = np.array(m, dtype=np.float32, copy=True, order="C")
    vv = np.array(v, dtype=np.float32, copy=True, order="C")
    gg = np.ascontiguousarray(g, dtype=np.float32)
    L.or_adam(_ptr(th), _ptr(gg), _ptr(mm), _ptr(vv), th.size, lr, b1, b2, eps, step)
    return th, mm, vv


def max_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().or_max_threads())


def set_threads(n: int):
    lib().or_set_threads(int(n))


def expf(p: np.ndarray) -> np.ndarray:
    """The oracle's fp32 exp (the C library's expf), element-wise."""
    p = np.ascontiguousarray(p, dtype=np.float32)
    out = np.empty_like(p)
    lib().or_expf_batch(_ptr(p), _ptr(out), p.size)
    return out


def exp_band(p: np.ndarray) -> np.ndarray:
    """rG(p): the largest relative difference between a GPU's exp of the fp32
    power p and the oracle's (see gs_oracle.c), element-wise, fp64."""
    p = np.ascontiguousarray(p, dtype=np.float32)
    out = np.empty(p.shape, dtype=np.float64)
    lib().or_exp_band_batch(_ptr(p), _ptr(out), p.size)
    return out


class exp_perturbed:
    """Context: every exp of the fp32 oracle's compositing moved to an edge of
    its band (mode +1, -1, or 2 = the edge picked per power), as a GPU's exp
    could be; the flags of the render are then those of the moved values."""

    def __init__(self, mode: int):
        self.mode = mode

    def __enter__(self):
        lib().or_set_exp_perturb(self.mode)
        return self

    def __exit__(self, *a):
        lib().or_set_exp_perturb(0)


class band_scaled:
    """Context: the flags' bands multiplied by `scale` (a narrowed band is the
    mistake the band tests must catch)."""

    def __init__(self, scale: float):
        self.scale = scale

    def __enter__(self):
        lib().or_set_band_scale(self.scale)
        return self

    def __exit__(self, *a):
        lib().or_set_band_scale(1.0)


def train_step(params, sh_degree, cams, target, lr, b1, b2, eps, step, m=None, v=None,
               bg=(0.0, 0.0, 0.0)):
    """One full oracle step (fp32 parity build). Returns a dict of every
    intermediate."""
    proj = preprocess(params, sh_degree, cams)
    fwd = render_fwd(proj, cams, bg)
    loss, dL = loss_l1(fwd["image"], target)
    g2 = render_bwd(proj, cams, dL, bg)
    grad = preprocess_bwd(params, sh_degree, cams, g2)
    if m is None:
        m = np.zeros_like(params)
        v = np.zeros_like(params)
    th, m2, v2 = adam(params, grad.astype(np.float32), m, v, lr, b1, b2, eps, step)
    return {"proj": proj, "fwd": fwd, "loss": loss, "dL": dL, "grad2d": g2, "grad": grad,
            "params": th, "m": m2, "v": v2}
