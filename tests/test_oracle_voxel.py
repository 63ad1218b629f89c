"""Pins of the oracle's voxel-grid down-sampling (CUDA-KDTree ICP article,
§4.3: voxel filter before the tree is built).  CPU only."""

import math

import numpy as np
import pytest

import oracle


def test_hand_voxels():
    P = [[0.5, 0.5, 0.5], [0.25, 0.75, 0.5],   # voxel (0, 0, 0): mean (0.375, 0.625, 0.5)
         [1.0, 0.0, 0.0],                      # on a boundary: voxel (1, 0, 0)
         [-0.5, 0.0, 0.0]]                     # negative: voxel (-1, 0, 0)
    c, n = oracle.voxel_downsample(P, 1.0)
    assert c.tolist() == [[-0.5, 0.0, 0.0], [0.375, 0.625, 0.5], [1.0, 0.0, 0.0]]
    assert n.tolist() == [1, 2, 1]


def test_order_is_x_fastest_then_y_then_z():
    P = [[0.5, 0.5, 1.5], [0.5, 1.5, 0.5], [1.5, 0.5, 0.5], [0.5, 0.5, 0.5]]
    c, _ = oracle.voxel_downsample(P, 1.0)
    # keys over the 2x2x2 grid: (0,0,0) -> 0, (1,0,0) -> 1, (0,1,0) -> 2, (0,0,1) -> 4
    assert c.tolist() == [[0.5, 0.5, 0.5], [1.5, 0.5, 0.5], [0.5, 1.5, 0.5], [0.5, 0.5, 1.5]]


def test_non_finite_points_are_dropped():
    P = [[0.1, 0.1, 0.1], [np.nan, 0, 0], [0, np.inf, 0], [0.3, 0.3, 0.3]]
    c, n = oracle.voxel_downsample(P, 1.0)
    assert n.tolist() == [2]
    assert c[0].tolist() == [np.float32(0.2)] * 3
    c, n = oracle.voxel_downsample([[np.nan, 0, 0]], 1.0)
    assert len(c) == 0 and len(n) == 0


def test_quotient_is_float64():
    """x = fl32(0.7) = 0.699999988079071: x / 0.1 in float64 is 6.99999988...,
    voxel 6; the float32 quotient fl32(x) / fl32(0.1) would round to 7.0."""
    x = np.float32(0.7)
    assert math.floor(float(x / np.float32(0.1))) == 7
    c, _ = oracle.voxel_downsample([[x, 0, 0], [0.65, 0, 0]], 0.1)
    assert len(c) == 1                        # both in voxel 6
    c, _ = oracle.voxel_downsample([[x, 0, 0], [0.71, 0, 0]], 0.1)
    assert len(c) == 2                        # 0.71 is in voxel 7


def _by_dict(P, leaf):
    """Independent grouping: Python dict of integer voxel tuples, Python-float
    running sums in index order, sorted by (z, y, x)."""
    groups = {}
    for i, p in enumerate(np.asarray(P, np.float32)):
        if not np.all(np.isfinite(p)):
            continue
        key = tuple(math.floor(float(x) / leaf) for x in p)
        s = groups.setdefault(key, [0.0, 0.0, 0.0, 0])
        for a in range(3):
            s[a] += float(p[a])
        s[3] += 1
    keys = sorted(groups, key=lambda k: (k[2], k[1], k[0]))
    c = np.array([[np.float32(groups[k][a] / groups[k][3]) for a in range(3)] for k in keys],
                 np.float32).reshape(-1, 3)
    n = np.array([groups[k][3] for k in keys], np.int32)
    return c, n


@pytest.mark.parametrize("seed,leaf", [(1, 0.1), (2, 0.37), (3, 1.0), (4, 0.01)])
def test_matches_dict_grouping(seed, leaf):
    rng = np.random.Generator(np.random.PCG64(seed))
    P = (rng.normal(size=(3000, 3)) * np.array([2.0, 1.0, 0.3])).astype(np.float32)
    P[::97] = np.round(P[::97] / np.float32(leaf)) * np.float32(leaf)   # near boundaries
    P[5] = [np.nan, 0, 0]
    c, n = oracle.voxel_downsample(P, leaf)
    ec, en = _by_dict(P, leaf)
    np.testing.assert_array_equal(n, en)
    np.testing.assert_array_equal(c.view(np.uint32), ec.view(np.uint32))
    assert n.sum() == 2999


def test_idempotent():
    rng = np.random.Generator(np.random.PCG64(8))
    P = (rng.random((20000, 3)) * 10).astype(np.float32)
    c, _ = oracle.voxel_downsample(P, 0.5)
    c2, n2 = oracle.voxel_downsample(c, 0.5)
    np.testing.assert_array_equal(c2.view(np.uint32), c.view(np.uint32))
    assert np.all(n2 == 1)


def test_one_voxel_is_the_mean():
    P = np.array([[0.125, 0.5, 0.75], [0.375, 0.25, 0.5], [0.25, 0.75, 0.25]], np.float32)
    c, n = oracle.voxel_downsample(P, 1.0)
    assert n.tolist() == [3]
    assert c[0].tolist() == [0.25, 0.5, 0.5]
