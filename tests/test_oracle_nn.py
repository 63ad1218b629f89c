"""Pins for the oracle's nearest-neighbour search (O1 brute force, O2 KD-tree).

Nothing here re-types the oracle's formula: the expected values come from the
hand-derived fixture, from scipy's exact float64 KD search, and from brute force
on tiny inputs.
"""

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from tests._cases import adversarial_clouds, load_nn_cases


@pytest.mark.parametrize("case", range(len(load_nn_cases())))
def test_brute_golden(case):
    T, Q, I, D = load_nn_cases()[case]
    idx, d2 = oracle.brute_nn(T, Q)
    np.testing.assert_array_equal(idx, I)
    np.testing.assert_array_equal(d2.view(np.uint32), D.view(np.uint32))


@pytest.mark.parametrize("leaf", [1, 2, 8])
@pytest.mark.parametrize("case", range(len(load_nn_cases())))
def test_kd_golden(case, leaf):
    T, Q, I, D = load_nn_cases()[case]
    idx, d2 = oracle.KDTree(T, leaf).query(Q)
    np.testing.assert_array_equal(idx, I)
    np.testing.assert_array_equal(d2.view(np.uint32), D.view(np.uint32))


def _fp32_dist(T, q, j):
    """Float32 squared distance of target j, evaluated by numpy float32 ufuncs."""
    d = T[j] - q
    return (d[..., 0] * d[..., 0] + d[..., 1] * d[..., 1]) + d[..., 2] * d[..., 2]


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_brute_against_scipy(seed):
    """scipy's exact fp64 search agrees wherever fp32 rounding cannot decide."""
    from scipy.spatial import cKDTree
    rng = np.random.Generator(np.random.PCG64(seed))
    T = (rng.random((4000, 3)) * 20 - 10).astype(np.float32)
    Q = (rng.random((2000, 3)) * 24 - 12).astype(np.float32)
    idx, d2 = oracle.brute_nn(T, Q)
    dd, ii = cKDTree(T.astype(np.float64)).query(Q.astype(np.float64), k=2)
    exact_ours = ((T[idx].astype(np.float64) - Q.astype(np.float64)) ** 2).sum(1)
    # our winner is an exact-arithmetic minimiser up to fp32 rounding (a few ulp)
    assert np.all(exact_ours <= dd[:, 0] ** 2 * (1 + 4e-7) + 1e-30)
    # when the exact runner-up is clearly farther, the index must be scipy's
    clear = dd[:, 1] ** 2 > dd[:, 0] ** 2 * (1 + 1e-5)
    assert clear.mean() > 0.95
    np.testing.assert_array_equal(idx[clear], ii[clear, 0])
    # the returned distance is within fp32 rounding of the exact distance
    np.testing.assert_allclose(d2.astype(np.float64), exact_ours, rtol=4e-7, atol=0)
    # and it is the fp32 value of the returned pair (numpy float32 ops never fuse)
    np.testing.assert_array_equal(d2, _fp32_dist(T, Q, idx))


@pytest.mark.parametrize("leaf", [1, 3, 8, 16, 64])
def test_kd_equals_brute_adversarial(leaf):
    for name, T, Q in adversarial_clouds():
        bi, bd = oracle.brute_nn(T, Q)
        ki, kd = oracle.KDTree(T, leaf).query(Q)
        np.testing.assert_array_equal(ki, bi, err_msg=name)
        np.testing.assert_array_equal(kd.view(np.uint32), bd.view(np.uint32), err_msg=name)


def test_brute_lowest_index_on_ties_grid():
    """Every grid point duplicated 3 times: a query at a grid point returns the
    first copy, with distance exactly 0."""
    g = np.stack(np.meshgrid(np.arange(4), np.arange(4), np.arange(4), indexing="ij"), -1).reshape(-1, 3)
    T = np.concatenate([g, g, g]).astype(np.float32)
    idx, d2 = oracle.brute_nn(T, g.astype(np.float32))
    np.testing.assert_array_equal(idx, np.arange(len(g)))
    assert np.all(d2 == 0)


@settings(max_examples=60, deadline=None)
@given(n=st.integers(1, 60), m=st.integers(1, 30), leaf=st.integers(1, 9),
       grid=st.booleans(), seed=st.integers(0, 2 ** 31 - 1))
def test_kd_equals_brute_hypothesis(n, m, leaf, grid, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    if grid:
        T = rng.integers(0, 4, (n, 3)).astype(np.float32)
        Q = (rng.integers(-2, 10, (m, 3)) * 0.5).astype(np.float32)
    else:
        T = rng.normal(size=(n, 3)).astype(np.float32)
        Q = rng.normal(size=(m, 3)).astype(np.float32)
    bi, bd = oracle.brute_nn(T, Q)
    ki, kd = oracle.KDTree(T, leaf).query(Q)
    np.testing.assert_array_equal(ki, bi)
    np.testing.assert_array_equal(kd.view(np.uint32), bd.view(np.uint32))


def test_kd_equals_brute_sampled_configs():
    """O2 == O1 on sampled queries of the clustered / outlier workload."""
    import synth
    p = synth.skewed(n=60_000, m=4_000)
    bi, bd = oracle.brute_nn(p.target, p.source)
    ki, kd = oracle.KDTree(p.target, 8).query(p.source)
    np.testing.assert_array_equal(ki, bi)
    np.testing.assert_array_equal(kd.view(np.uint32), bd.view(np.uint32))


def test_kd_prunes():
    """The oracle tree is an accelerator: far fewer node visits than nodes."""
    rng = np.random.Generator(np.random.PCG64(5))
    T = rng.random((20000, 3)).astype(np.float32)
    tr = oracle.KDTree(T, 8)
    _, _, vis = tr.query(rng.random((500, 3)).astype(np.float32), return_visits=True)
    assert vis.mean() < 0.02 * tr.node_count
