"""Pins of the oracle's backward pass: central finite differences of its fp64
forward (preprocess -> composite -> L1 loss) on tiny scenes, for every one of
the 59 (or 14) parameters of every Gaussian. A coordinate whose +-h runs change
any decision (culling, guard-band clamp, colour clamp, tile rectangle, alpha
skip / 0.99 clamp / stop, sign of the L1 residual) is skipped: the loss is not
differentiable there."""

import math

import numpy as np
import pytest
from scipy.spatial.transform import Rotation

from oracle import oracle as O
from tests.util import pinhole


def tiny_scene(seed, n, deg, n_views=2, W=32, H=32, f=36.0):
    rng = np.random.default_rng(seed)
    P = 11 + 3 * (deg + 1) ** 2
    p = np.zeros((P, n))
    p[0] = rng.uniform(-0.35, 0.35, n)
    p[1] = rng.uniform(-0.35, 0.35, n)
    p[2] = rng.uniform(2.5, 4.0, n)
    p[3:6] = rng.uniform(-2.1, -1.5, (3, n))
    p[6:10] = rng.normal(size=(4, n))
    p[10] = rng.normal(0.5, 1.5, n)
    p[10, 0] = 6.0  # one nearly opaque Gaussian: exercises the 0.99 clamp
    p[11:14] = rng.normal(0, 0.6, (3, n))
    if P > 14:
        p[14:] = rng.normal(0, 0.15, (P - 14, n))
    cams = []
    for v in range(n_views):
        R = Rotation.from_euler("xy", [2.0 * v, -4.0 * v], degrees=True).as_matrix()
        cams.append(pinhole(W, H, f, R=R, t=(0.05 * v, -0.03 * v, 0.1 * v), fy=0.9 * f))
    target = rng.random((n_views, 3, H, W))
    return p, cams, target


def forward(p, deg, cams, target, bg):
    pr = O.preprocess(p, deg, cams, "f64")
    out = O.render_fwd(pr, cams, bg, "f64")
    loss, dL = O.loss_l1(out["image"], target, "f64")
    decisions = (pr["iv"].tobytes(), out["sig"].tobytes(), np.sign(dL).tobytes())
    return loss, dL, pr, decisions


def analytic(p, deg, cams, target, bg):
    loss, dL, pr, _ = forward(p, deg, cams, target, bg)
    g2 = O.render_bwd(pr, cams, dL, bg, "f64")
    return O.preprocess_bwd(p, deg, cams, g2, "f64")


def fd_check(p, deg, cams, target, bg, rel=2e-5):
    g = analytic(p, deg, cams, target, bg)
    _, _, _, base = forward(p, deg, cams, target, bg)
    scale = np.abs(g).max()
    checked = skipped = 0
    worst = 0.0
    for r in range(p.shape[0]):
        for k in range(p.shape[1]):
            h = 1e-6 * max(1.0, abs(p[r, k]))
            pp, pm = p.copy(), p.copy()
            pp[r, k] += h
            pm[r, k] -= h
            lp, _, _, dp = forward(pp, deg, cams, target, bg)
            lm, _, _, dm = forward(pm, deg, cams, target, bg)
            if dp != base or dm != base:
                skipped += 1
                continue
            fd = (lp - lm) / (2 * h)
            err = abs(fd - g[r, k])
            worst = max(worst, err / (abs(g[r, k]) + 1e-6 * scale))
            assert err <= rel * abs(g[r, k]) + 1e-6 * scale, (r, k, fd, g[r, k])
            checked += 1
    return checked, skipped, worst


@pytest.mark.parametrize("seed,n,deg", [(0, 1, 3), (1, 4, 3), (2, 8, 3), (3, 6, 0), (4, 5, 1), (5, 5, 2)])
def test_finite_differences(seed, n, deg):
    p, cams, target = tiny_scene(seed, n, deg)
    checked, skipped, worst = fd_check(p, deg, cams, target, (0.0, 0.0, 0.0))
    assert checked >= 0.8 * p.size, (checked, skipped)
    # every parameter row is non-trivially exercised somewhere
    g = analytic(p, deg, cams, target, (0.0, 0.0, 0.0))
    assert np.all(np.abs(g).max(axis=1) > 0)


def test_finite_differences_background():
    p, cams, target = tiny_scene(7, 5, 3)
    checked, skipped, _ = fd_check(p, 3, cams, target, (0.3, 0.6, 0.1))
    assert checked >= 0.8 * p.size


def test_finite_differences_guard_band():
    """A large Gaussian beyond the 1.3 x half-fov guard band: the clamped
    Jacobian's depth dependence is part of the gradient."""
    p, cams, target = tiny_scene(8, 3, 3, n_views=1)
    p[0, 0], p[2, 0] = 2.4, 3.0  # x/z = 0.8 > 1.3 * 16/36
    p[3:6, 0] = -0.4
    pr = O.preprocess(p, 3, cams, "f64")
    assert pr["iv"][0, 0, O.INT_VIS] == 1 and pr["iv"][0, 0, O.INT_FLAGS] & 1
    checked, skipped, _ = fd_check(p, 3, cams, target, (0.0, 0.0, 0.0))
    assert checked >= 0.8 * p.size


def test_stop_rule_exercised():
    """Dense opaque stack: some pixels reach T < 1e-4, and FD still agrees."""
    rng = np.random.default_rng(10)
    n = 20
    p, cams, target = tiny_scene(10, n, 0, n_views=1)
    p[0] = rng.uniform(-0.05, 0.05, n)
    p[1] = rng.uniform(-0.05, 0.05, n)
    p[10] = rng.uniform(5.0, 7.0, n)
    p[3:6] = -0.8
    pr = O.preprocess(p, 0, cams, "f64")
    out = O.render_fwd(pr, cams, (0, 0, 0), "f64")
    assert (out["T_final"] < 1.01e-4).sum() > 0
    checked, skipped, _ = fd_check(p, 0, cams, target, (0.0, 0.0, 0.0))
    assert checked >= 0.6 * p.size


def test_f32_oracle_gradient_close_to_f64():
    """The fp32 parity build (fp32 decisions, fp64 accumulation) gives the fp64
    gradient to fp32 accuracy on a scene without near-threshold pixels."""
    p, cams, target = tiny_scene(11, 8, 3)
    g64 = analytic(p, 3, cams, target, (0, 0, 0))
    p32 = p.astype(np.float32)
    pr = O.preprocess(p32, 3, cams, "f32")
    out = O.render_fwd(pr, cams)
    assert out["amb"].sum() == 0
    _, dL = O.loss_l1(out["image"], target.astype(np.float32))
    g2 = O.render_bwd(pr, cams, dL)
    g32 = O.preprocess_bwd(p32, 3, cams, g2)
    np.testing.assert_allclose(g32, g64, rtol=2e-3, atol=2e-5 * np.abs(g64).max())
