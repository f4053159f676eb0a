"""Helpers for hand-built scenes in tests (no rasterizer arithmetic here)."""

import math

import numpy as np

from gaussian_splatting_differentiable_ewa_amd.scenes import Camera, param_rows


def block(means, log_scales, quats, opacity_logits, sh, dtype=np.float32):
    """Assemble a ``[P][N]`` parameter block from per-Gaussian arrays.
    ``sh`` is ``[N][K][3]`` (K = (d+1)^2)."""
    means = np.asarray(means, np.float64).reshape(-1, 3)
    n = means.shape[0]
    sh = np.asarray(sh, np.float64).reshape(n, -1, 3)
    K = sh.shape[1]
    deg = int(round(math.sqrt(K))) - 1
    P = param_rows(deg)
    out = np.zeros((P, n), dtype=np.float64)
    out[0:3] = means.T
    out[3:6] = np.asarray(log_scales, np.float64).reshape(n, 3).T
    out[6:10] = np.asarray(quats, np.float64).reshape(n, 4).T
    out[10] = np.asarray(opacity_logits, np.float64).reshape(n)
    out[11:] = sh.reshape(n, K * 3).T
    return out.astype(dtype), deg


def pinhole(width, height, f, R=None, t=(0.0, 0.0, 0.0), near=0.01, far=math.inf, cx=None, cy=None,
            fy=None):
    R = np.eye(3) if R is None else np.asarray(R, np.float64)
    return Camera(width=width, height=height, fx=float(f), fy=float(f if fy is None else fy),
                  cx=width / 2.0 if cx is None else float(cx),
                  cy=height / 2.0 if cy is None else float(cy),
                  R=tuple(float(np.float32(v)) for v in R.reshape(-1)),
                  t=tuple(float(np.float32(v)) for v in t), near=near, far=far)


def logit(p):
    return math.log(p / (1.0 - p))


def sh0_for_rgb(rgb):
    """DC coefficient giving colour ``rgb`` (before the +0.5 offset is added):
    the degree-0 basis function is the constant 1/(2 sqrt(pi))."""
    return (np.asarray(rgb, np.float64) - 0.5) * (2.0 * math.sqrt(math.pi))
