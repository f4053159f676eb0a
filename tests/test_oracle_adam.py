"""Pins of the oracle's Adam step (Kingma & Ba, reference [12] of "A Scalable
PyTorch Abstraction for Multi-GPU Gaussian Splatting"): the first-step closed
form, zero gradients, and two steps worked by hand."""

import numpy as np
import pytest

from oracle import oracle as O


def test_first_step_closed_form():
    """From zero moments, step 1 gives m_hat = g and v_hat = g^2, so the
    update is lr * g / (|g| + eps)."""
    rng = np.random.default_rng(0)
    n = 10_000
    th = rng.normal(size=n).astype(np.float32)
    g = (rng.normal(size=n) * 10.0 ** rng.uniform(-8, 2, n)).astype(np.float32)
    z = np.zeros(n, np.float32)
    lr, eps = 1e-3, 1e-15
    t1, m1, v1 = O.adam(th, g, z, z, lr, 0.9, 0.999, eps, 1)
    g64 = g.astype(np.float64)
    expect = th.astype(np.float64) - lr * g64 / (np.abs(g64) + eps)
    np.testing.assert_allclose(t1, expect, rtol=1e-6, atol=1e-9)
    np.testing.assert_allclose(m1, 0.1 * g64, rtol=1e-6)
    np.testing.assert_allclose(v1, 0.001 * g64 * g64, rtol=1e-6)


def test_zero_gradient_leaves_parameters():
    th = np.linspace(-2, 2, 101, dtype=np.float32)
    z = np.zeros_like(th)
    t1, m1, v1 = O.adam(th, z, z, z, 1e-3, 0.9, 0.999, 1e-15, 1)
    np.testing.assert_array_equal(t1, th)
    assert not m1.any() and not v1.any()


def test_two_steps_by_hand():
    """theta0 = 0.5, g1 = 0.2, g2 = -0.1, lr 1e-3, betas 0.9 / 0.999, eps 1e-15.
    Step 1: m1 = 0.02, v1 = 4e-5, m_hat = 0.2, v_hat = 0.04 -> theta1 = 0.499.
    Step 2: m2 = 0.018 - 0.01 = 0.008, v2 = 3.996e-5 + 1e-5 = 4.996e-5,
    bias corrections 1 - 0.81 = 0.19 and 1 - 0.998001 = 0.001999,
    m_hat = 0.0421052631578947..., v_hat = 0.0249924962481240...,
    sqrt(v_hat) = 0.158090152280665..., theta2 = 0.498733662960339..."""
    th = np.array([0.5], np.float32)
    z = np.zeros(1, np.float32)
    t1, m1, v1 = O.adam(th, np.array([0.2], np.float32), z, z, 1e-3, 0.9, 0.999, 1e-15, 1)
    assert t1[0] == pytest.approx(0.499, rel=1e-7)
    assert m1[0] == pytest.approx(0.02, rel=1e-7) and v1[0] == pytest.approx(4e-5, rel=1e-6)
    t2, m2, v2 = O.adam(t1, np.array([-0.1], np.float32), m1, v1, 1e-3, 0.9, 0.999, 1e-15, 2)
    assert m2[0] == pytest.approx(0.008, rel=1e-6)
    assert v2[0] == pytest.approx(4.996e-5, rel=1e-6)
    assert t2[0] == pytest.approx(0.498733662960339, rel=1e-7)
