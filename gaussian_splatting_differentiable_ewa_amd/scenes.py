"""Seeded synthetic scenes and cameras: the only code shared by the HIP path and
the CPU oracle's tests.

This module draws random numbers and builds camera poses. It holds none of the
rasterizer's arithmetic (no projection, colour, compositing or gradients), so
both sides can take their inputs from it without sharing any of the method.

The pages measure on public datasets (city blocks, Mip-NeRF 360 scenes and
others named in "On Scaling Up 3D Gaussian Splatting Training" and the ByteSplat
abstract); none is available here, so the five scenes below stand in for them.
Each has the shapes and value distributions of a training step: N Gaussians with
59 fp32 parameters at SH degree 3 ("On Scaling Up 3D Gaussian Splatting
Training", answer on the storage requirement), cameras at 720p to 4K.

Parameter block layout, ``[P][N]`` float32, structure-of-arrays:

    rows 0-2   mean x, y, z (world)
    rows 3-5   log-scale per axis (natural log)
    rows 6-9   rotation quaternion w, x, y, z
    row  10    opacity logit
    rows 11..  SH coefficient k, colour channel c at row 11 + 3k + c,
               k = 0 .. (d+1)^2 - 1

so P = 11 + 3(d+1)^2: 59 at degree 3, 14 at degree 0.

Draw recipe (``numpy.random.default_rng(seed)``, float32 normals via
``standard_normal(dtype=float32)``), in this order: cluster centres (uniform in
the box), cluster assignments (uniform integers), offsets ``N(0, sigma)`` per
axis with points outside the box redrawn until none is left, then log-scales
``[3][N]``, quaternions ``[4][N]`` (normalised), opacity logits ``[N]``, DC
colour ``[3][N]``, higher SH bands ``[3((d+1)^2-1)][N]``.  Boxes without
clusters draw means uniformly.  The world uses camera-style axes (x right,
y down, z forward), so a ground plane at height h sits at y = -h.
"""

from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

TILE = 16


def param_rows(sh_degree: int) -> int:
    """Rows of the parameter block at SH degree ``sh_degree``."""
    if sh_degree not in (0, 1, 2, 3):
        raise ValueError(f"sh_degree must be 0..3, got {sh_degree}")
    return 11 + 3 * (sh_degree + 1) ** 2


@dataclasses.dataclass(frozen=True)
class Camera:
    """Pinhole camera. ``R`` (3x3) and ``t`` map world to camera: p_c = R p + t.

    Camera axes: x right, y down, z forward. Pixel (i, j) covers
    [i, i+1) x [j, j+1); its centre is (i + 0.5, j + 0.5).
    """

    width: int
    height: int
    fx: float
    fy: float
    cx: float
    cy: float
    R: Tuple[float, ...]  # 9 floats, row-major
    t: Tuple[float, float, float]
    near: float = 0.01
    far: float = math.inf

    @property
    def tiles_x(self) -> int:
        return (self.width + TILE - 1) // TILE

    @property
    def tiles_y(self) -> int:
        return (self.height + TILE - 1) // TILE

    @property
    def n_tiles(self) -> int:
        return self.tiles_x * self.tiles_y

    @property
    def n_pixels(self) -> int:
        return self.width * self.height


def look_camera(width, height, f, position, yaw_deg=0.0, near=0.01, far=math.inf) -> Camera:
    """Camera at ``position`` whose forward axis is +z turned by ``yaw_deg``
    about the world y axis (no pitch or roll); principal point at the image
    centre."""
    th = math.radians(yaw_deg)
    c, s = math.cos(th), math.sin(th)
    # camera-to-world rotation: columns are the camera's right, down, forward.
    c2w = np.array([[c, 0.0, s], [0.0, 1.0, 0.0], [-s, 0.0, c]], dtype=np.float64)
    w2c = c2w.T
    pos = np.asarray(position, dtype=np.float64)
    t = -w2c @ pos
    return Camera(
        width=int(width), height=int(height), fx=float(f), fy=float(f),
        cx=width / 2.0, cy=height / 2.0,
        R=tuple(float(np.float32(v)) for v in w2c.reshape(-1)),
        t=tuple(float(np.float32(v)) for v in t),
        near=float(near), far=float(far),
    )


@dataclasses.dataclass(frozen=True)
class SceneConfig:
    name: str
    seed: int
    target_seed: int
    n: int
    sh_degree: int
    box_lo: Tuple[float, float, float]
    box_hi: Tuple[float, float, float]
    n_clusters: int  # 0 = uniform in the box
    cluster_sigma: float
    log_scale_mean: float
    log_scale_std: float
    width: int
    height: int
    focal: float
    yaws: Tuple[float, ...] = (0.0,)
    orbit_centre: Optional[Tuple[float, float, float]] = None
    camera_pos: Tuple[float, float, float] = (0.0, 0.0, 0.0)
    far: float = math.inf
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-15

    @property
    def P(self) -> int:
        return param_rows(self.sh_degree)

    @property
    def n_views(self) -> int:
        return len(self.yaws)

    def cameras(self) -> List[Camera]:
        cams = []
        for yaw in self.yaws:
            if self.orbit_centre is not None:
                ctr = np.asarray(self.orbit_centre, dtype=np.float64)
                radius = float(ctr[2] - self.camera_pos[2])
                th = math.radians(yaw)
                pos = ctr + radius * np.array([-math.sin(th), 0.0, -math.cos(th)])
            else:
                pos = np.asarray(self.camera_pos, dtype=np.float64)
            cams.append(look_camera(self.width, self.height, self.focal, pos, yaw,
                                    far=self.far))
        return cams


CONFIGS = {
    0: SceneConfig("tiny-10k-sh0-256", 0, 1, 10_000, 0,
                   (-1.0, -1.0, 2.0), (1.0, 1.0, 6.0), 0, 0.0, -3.5, 0.3,
                   256, 256, 256.0),
    1: SceneConfig("object-200k-sh3-720p", 2, 3, 200_000, 3,
                   (-3.0, -3.0, 3.0), (3.0, 3.0, 12.0), 32, 0.3, -4.0, 0.5,
                   1280, 720, 1000.0),
    2: SceneConfig("headline-1M-sh3-4x1080p", 4, 5, 1_000_000, 3,
                   (-10.0, -10.0, 4.0), (10.0, 10.0, 40.0), 128, 0.3, -4.5, 0.6,
                   1920, 1080, 1400.0, yaws=(0.0, 5.0, 10.0, 15.0),
                   orbit_centre=(0.0, 0.0, 22.0)),
    3: SceneConfig("stress-5M-sh3-4k", 6, 7, 5_000_000, 3,
                   (-20.0, -20.0, 4.0), (20.0, 20.0, 80.0), 512, 0.3, -4.0, 0.7,
                   3840, 2160, 2800.0),
    4: SceneConfig("city-40M-sh3-1080p", 8, 9, 40_000_000, 3,
                   (-200.0, -30.0, -200.0), (200.0, 0.0, 200.0), 0, 0.0, -3.0, 0.8,
                   1920, 1080, 1400.0, camera_pos=(0.0, -1.7, 0.0), far=120.0),
}


# A parity-test scene beside the five workloads: the object-scale recipe
# (config 1's distributions) seen by two views of 250x190 pixels, so that
# neither image side is a multiple of the 16-pixel tile (the last tile column
# is 10 pixels wide, the last tile row 14 pixels tall).
RAGGED = SceneConfig("ragged-200k-sh3-2x250x190", 10, 11, 200_000, 3,
                     (-3.0, -3.0, 3.0), (3.0, 3.0, 12.0), 32, 0.3, -4.0, 0.5,
                     250, 190, 195.3125, yaws=(0.0, 6.0), orbit_centre=(0.0, 0.0, 7.5))


def _normal(rng, shape_or_out, mean, std):
    out = shape_or_out
    rng.standard_normal(dtype=np.float32, out=out)
    if std != 1.0:
        out *= np.float32(std)
    if mean != 0.0:
        out += np.float32(mean)
    return out


def make_params(cfg: SceneConfig, seed: Optional[int] = None, n: Optional[int] = None) -> np.ndarray:
    """Draw the ``[P][N]`` float32 parameter block of ``cfg`` (see module doc)."""
    seed = cfg.seed if seed is None else seed
    N = cfg.n if n is None else int(n)
    rng = np.random.default_rng(seed)
    P = cfg.P
    out = np.empty((P, N), dtype=np.float32)
    lo = np.asarray(cfg.box_lo, dtype=np.float32)
    hi = np.asarray(cfg.box_hi, dtype=np.float32)
    means = out[0:3]
    if cfg.n_clusters > 0:
        centres = rng.uniform(lo, hi, size=(cfg.n_clusters, 3)).astype(np.float32)
        assign = rng.integers(0, cfg.n_clusters, size=N)
        for a in range(3):
            means[a] = centres[assign, a]
        offs = np.empty((3, N), dtype=np.float32)
        _normal(rng, offs, 0.0, cfg.cluster_sigma)
        means += offs
        del offs
        while True:
            bad = np.nonzero(((means < lo[:, None]) | (means > hi[:, None])).any(axis=0))[0]
            if bad.size == 0:
                break
            redo = np.empty((3, bad.size), dtype=np.float32)
            _normal(rng, redo, 0.0, cfg.cluster_sigma)
            for a in range(3):
                means[a, bad] = centres[assign[bad], a] + redo[a]
    else:
        for a in range(3):
            means[a] = rng.uniform(lo[a], hi[a], size=N).astype(np.float32)
    _normal(rng, out[3:6], cfg.log_scale_mean, cfg.log_scale_std)
    q = out[6:10]
    _normal(rng, q, 0.0, 1.0)
    q /= np.sqrt((q.astype(np.float64) ** 2).sum(axis=0)).astype(np.float32)
    _normal(rng, out[10], 0.0, 1.0)
    _normal(rng, out[11:14], 0.0, 0.5)
    if P > 14:
        _normal(rng, out[14:], 0.0, 0.05)
    return out


def make_target_params(cfg: SceneConfig, n: Optional[int] = None) -> np.ndarray:
    """The scene whose render is the L1 target (drawn from ``cfg.target_seed``)."""
    return make_params(cfg, seed=cfg.target_seed, n=n)


def random_image(seed: int, n_views: int, height: int, width: int) -> np.ndarray:
    """A seeded uniform [0, 1) image stack ``[V][3][H][W]`` float32, used as the
    L1 target where a rendered target would have to come from the code under
    test."""
    rng = np.random.default_rng(seed)
    return rng.random((n_views, 3, height, width), dtype=np.float32)


def adam_state(P: int, N: int, seed: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Adam moments: zeros (the start of training), or seeded non-trivial
    moments when ``seed`` is given (to exercise later steps)."""
    if seed is None:
        return np.zeros((P, N), np.float32), np.zeros((P, N), np.float32)
    rng = np.random.default_rng(seed)
    m = (rng.standard_normal((P, N), dtype=np.float32) * np.float32(1e-3))
    v = (rng.random((P, N), dtype=np.float32) * np.float32(1e-6))
    return m, v


def cameras_equal_size(cams: Sequence[Camera]) -> bool:
    return all(c.width == cams[0].width and c.height == cams[0].height for c in cams)
