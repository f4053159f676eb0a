"""Pins of the oracle's view-dependent colour (real spherical harmonics up to
degree 3, Condon-Shortley sign, k = l^2 + l + m) against scipy's complex
harmonics, the addition theorem and orthonormality by exact quadrature."""

import math

import numpy as np
import pytest
import scipy.special as sp
from scipy.spatial.transform import Rotation

from oracle import oracle as O
from tests.util import block, logit, pinhole


def _camera_looking(d, pos):
    """Camera at ``pos`` whose forward (+z) axis points along unit ``d``."""
    rot, _ = Rotation.align_vectors([d], [[0.0, 0.0, 1.0]])
    c2w = rot.as_matrix()
    w2c = c2w.T
    return pinhole(64, 64, 60.0, R=w2c, t=-w2c @ np.asarray(pos))


def oracle_basis(d, deg=3, precision="f64", coef=0.1):
    """Read Y_k(d) back from the colour of Gaussians carrying one unit-ish SH
    coefficient each (channel 0): rgb = coef * Y_k + 0.5."""
    d = np.asarray(d, np.float64)
    d = d / np.linalg.norm(d)
    pos = np.array([0.3, -0.2, 0.1])
    nb = (deg + 1) ** 2
    cam = _camera_looking(d, pos)
    # camera R, t are stored in fp32: recover the exact centre the oracle sees
    R = np.asarray(cam.R, np.float64).reshape(3, 3)
    centre = -R.T @ np.asarray(cam.t, np.float64)
    fwd = R[2]
    mean = centre + 5.0 * fwd
    sh = np.zeros((nb, nb, 3))
    for k in range(nb):
        sh[k, k, 0] = coef
    p, _ = block([mean] * nb, [[-1, -1, -1]] * nb, [[1, 0, 0, 0]] * nb, [logit(0.5)] * nb, sh,
                 dtype=np.float64 if precision == "f64" else np.float32)
    pr = O.preprocess(p, deg, [cam], precision)
    assert np.all(pr["iv"][0, :, O.INT_VIS] == 1)
    e = mean - centre
    return (pr["rec"][0, :, 10] - 0.5) / coef, e / np.linalg.norm(e)


def scipy_real_cs(l, m, d):
    """Real harmonic with the Condon-Shortley phase kept, from scipy's complex
    Y_l^m (which includes it): sqrt(2) Re Y_l^m (m > 0), Y_l^0, sqrt(2) Im Y_l^|m|
    (m < 0)."""
    x, y, z = d
    theta = math.acos(max(-1.0, min(1.0, z)))
    phi = math.atan2(y, x) % (2 * math.pi)
    Y = complex(sp.sph_harm_y(l, abs(m), theta, phi))
    if m > 0:
        return math.sqrt(2) * Y.real
    if m < 0:
        return math.sqrt(2) * Y.imag
    return Y.real


def test_basis_matches_scipy():
    rng = np.random.default_rng(7)
    for _ in range(12):
        d = rng.normal(size=3)
        Y, du = oracle_basis(d)
        for l in range(4):
            for m in range(-l, l + 1):
                k = l * l + l + m
                assert Y[k] == pytest.approx(scipy_real_cs(l, m, du), abs=1e-10), (l, m)


def test_addition_theorem():
    rng = np.random.default_rng(8)
    for _ in range(10):
        Y, _ = oracle_basis(rng.normal(size=3))
        for l in range(4):
            s = sum(Y[l * l + l + m] ** 2 for m in range(-l, l + 1))
            assert s == pytest.approx((2 * l + 1) / (4 * math.pi), rel=1e-10)


def test_orthonormal_by_quadrature():
    """Gauss-Legendre in cos(theta) (8 nodes) x 16 uniform azimuths integrates
    products of degree <= 3 harmonics exactly."""
    xs, ws = np.polynomial.legendre.leggauss(8)
    G = np.zeros((16, 16))
    nphi = 16
    for ct, w in zip(xs, ws):
        st = math.sqrt(1 - ct * ct)
        for j in range(nphi):
            phi = 2 * math.pi * (j + 0.25) / nphi
            Y, _ = oracle_basis([st * math.cos(phi), st * math.sin(phi), ct])
            G += np.outer(Y, Y) * w * (2 * math.pi / nphi)
    # camera poses are stored in fp32, so the probed directions sit ~1e-8 off
    # the quadrature nodes
    np.testing.assert_allclose(G, np.eye(16), atol=1e-7)


def test_degree0_colour_and_clamp():
    cam = pinhole(64, 64, 60.0)
    dc = np.array([[0.7, -0.2, -2.0]])
    p, deg = block([[0, 0, 4.0]], [[-1, -1, -1]], [[1, 0, 0, 0]], [0.0], dc.reshape(1, 1, 3))
    pr = O.preprocess(p, deg, [cam], "f32")
    rgb = pr["rec"][0, 0, 10:13].astype(np.float64)
    y00 = scipy_real_cs(0, 0, (0, 0, 1))
    expect = dc[0] * y00 + 0.5
    np.testing.assert_allclose(rgb[:2], expect[:2], rtol=1e-6)
    assert expect[2] < 0 and rgb[2] == 0.0
    assert pr["iv"][0, 0, O.INT_FLAGS] >> 2 == 0b100


def test_f32_basis_close_to_f64():
    rng = np.random.default_rng(9)
    for _ in range(4):
        d = rng.normal(size=3)
        Y64, _ = oracle_basis(d, precision="f64")
        Y32, _ = oracle_basis(d, precision="f32", coef=0.25)
        np.testing.assert_allclose(Y32, Y64, atol=2e-5)
