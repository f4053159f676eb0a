"""The storage order of the Gaussians (host code): a permutation that lists
the means in Morton (Z-order) order."""

import numpy as np

from gaussian_splatting_differentiable_ewa_amd.step import spatial_order


def test_cube_corners_in_z_order():
    # the corners of a cube, listed with x varying fastest, then y, then z,
    # are in Z-order (bit interleave x, y, z from the lowest bit)
    corners = np.array([[x, y, z] for z in (0, 1) for y in (0, 1) for x in (0, 1)], dtype=np.float32).T
    shuffle = np.random.default_rng(0).permutation(8)
    perm = spatial_order(corners[:, shuffle])
    assert np.array_equal(corners[:, shuffle][:, perm], corners)


def test_two_levels_of_octants():
    # 4 x 4 x 4 grid: every block of 8 consecutive entries is one octant of
    # side 2, and the blocks visit the octants in Z-order too
    g = np.array([[x, y, z] for z in range(4) for y in range(4) for x in range(4)], dtype=np.float32).T
    perm = spatial_order(g)
    p = g[:, perm].astype(int)
    assert np.array_equal(np.sort(perm), np.arange(64))
    for b in range(8):
        blk = p[:, 8 * b:8 * b + 8]
        oct_ = blk // 2
        assert (oct_ == oct_[:, :1]).all()
        assert np.array_equal(oct_[:, 0], [b & 1, (b >> 1) & 1, (b >> 2) & 1])


def test_random_means_permutation_and_locality():
    rng = np.random.default_rng(1)
    m = rng.uniform(-5, 5, size=(3, 20000)).astype(np.float32)
    perm = spatial_order(m)
    assert np.array_equal(np.sort(perm), np.arange(m.shape[1]))
    o = m[:, perm]
    step = np.linalg.norm(np.diff(o, axis=1), axis=0).mean()
    rand = np.linalg.norm(np.diff(m, axis=1), axis=0).mean()
    assert step < 0.1 * rand
