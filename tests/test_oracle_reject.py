"""Pins of the oracle's correspondence rejection (CUDA-KDTree ICP article,
§4.4: a distance threshold at correspondence time, and residual rejection
with the 3-sigma rule after the solve).  CPU only."""

import numpy as np
import pytest

import oracle
import synth


# ------------------------------------------------------------- max_dist bound
def test_max_dist_bound_values():
    assert oracle.max_dist_bound(0.5) == np.float32(0.25)
    assert oracle.max_dist_bound(3.0) == np.float32(9.0)
    # 0.1 * 0.1 = 0.010000000000000002 in float64, whose nearest float32 is
    # the float32 nearest to 0.01 (0.009999999776482582)
    assert oracle.max_dist_bound(0.1) == np.float32(0.01)
    assert oracle.max_dist_bound(0.1).dtype == np.float32
    for off in (None, 0.0, -1.0, np.inf, np.nan):
        assert oracle.max_dist_bound(off) == np.float32(np.inf)


def test_max_dist_keeps_pairs_at_the_bound():
    """d2 <= bound is kept; one float32 step farther is dropped."""
    T = np.array([[0, 0, 0], [8, 0, 0], [0, 4, 0], [0, 0, 4], [0, 4, 4]], np.float32)
    step = np.nextafter(np.float32(0.5), np.float32(1))
    off = np.array([0.5, 0.5, 0.5, 0.5, step], np.float32)
    S = T.copy()
    S[:, 0] += off                      # exact: every x here is representable
    assert np.all(S[:, 0] - T[:, 0] == off)
    res = oracle.icp(T, S, iters=1, nn="brute", max_dist=0.5)
    assert res["n"][0] == 4             # the four at exactly 0.5 m
    assert res["E"][0] == 4 * 0.25
    res = oracle.icp(T, S, iters=1, nn="brute")
    assert res["n"][0] == 5


# ------------------------------------------------------------------ residuals
def test_residual_sq_hand_values():
    r2 = oracle.residual_sq([[0, 0, 0]], [[0, 2, 0]], np.eye(3), [1, 0, 0])
    assert r2.tolist() == [5.0]             # e = (1, -2, 0)
    Rz = np.array([[0, -1, 0], [1, 0, 0], [0, 0, 1]], np.float64)
    r2 = oracle.residual_sq([[1, 2, 3]], [[0, 0, 0]], Rz, [0, 0, 0])
    assert r2.tolist() == [14.0]            # R s = (-2, 1, 3)
    r2 = oracle.residual_sq([[1, 2, 3]], [[-2, 1, 3]], Rz, [0, 0, 0])
    assert r2.tolist() == [0.0]


def test_residual_sq_is_not_rounded_to_float32():
    """The moved point stays float64: a 1e-9 translation shows in r^2."""
    r2 = oracle.residual_sq([[1, 1, 1]], [[1, 1, 1]], np.eye(3), [1e-9, 0, 0])
    assert r2[0] == pytest.approx(1e-18, rel=1e-9)


# ------------------------------------------------------------------- 3 sigma
def _pairs_with_residuals(res):
    """Pairs (s, m = s + e_i) with |e_i| = res_i along x, under R = I, t = 0."""
    rng = np.random.Generator(np.random.PCG64(7))
    s = np.round(rng.random((len(res), 3)) * 64).astype(np.float32)
    m = s.copy()
    m[:, 0] += np.asarray(res, np.float32)
    return s, m


def test_reject_sigma_hand_example():
    s, m = _pairs_with_residuals([1.0] * 99 + [10.0])
    keep, sigma2, thr = oracle.reject_sigma(s, m, np.eye(3), np.zeros(3), 3.0)
    assert sigma2 == (99 * 1.0 + 100.0) / 100          # 1.99
    assert thr == 9.0 * 1.99
    assert keep.tolist() == [True] * 99 + [False]


def test_reject_sigma_threshold_is_inclusive():
    s, m = _pairs_with_residuals([0.0, 0.0, 0.0, 2.0])   # r^2 = 0, 0, 0, 4: sigma^2 = 1
    keep, sigma2, thr = oracle.reject_sigma(s, m, np.eye(3), np.zeros(3), 2.0)
    assert (sigma2, thr) == (1.0, 4.0)
    assert keep.all()
    keep, _, _ = oracle.reject_sigma(s, m, np.eye(3), np.zeros(3), 1.9)
    assert keep.tolist() == [True, True, True, False]


# ------------------------------------------------------ ICP with rejection
def _outlier_case(offset_lo, offset_hi, extent=1.0, deg=2.0, seed=31):
    """Noise-free source = exact rigid copy of a target of 3000 points in a
    cube of side ``extent``, plus 2% outliers displaced by offset_lo..offset_hi
    metres from their own copy."""
    rng = np.random.Generator(np.random.PCG64(seed))
    T = (rng.random((3000, 3)) * extent).astype(np.float32)
    Rg = synth.rotation_about(synth.random_unit(rng), np.deg2rad(deg))
    tg = np.array([0.02, -0.01, 0.005])
    S = (T.astype(np.float64) @ Rg.T + tg)
    k = rng.choice(len(S), 60, replace=False)
    d = rng.normal(size=(60, 3))
    d /= np.linalg.norm(d, axis=1, keepdims=True)
    S[k] += d * rng.uniform(offset_lo, offset_hi, size=(60, 1))
    return T, S.astype(np.float32), Rg.T, -(Rg.T @ tg)


def test_max_dist_rejects_gross_outliers():
    T, S, R_ref, t_ref = _outlier_case(3.0, 5.0)
    plain = oracle.icp(T, S, iters=30, nn="brute")
    rej = oracle.icp(T, S, iters=30, nn="brute", max_dist=0.5)
    assert oracle.rot_err(plain["R"], R_ref) > 1e-3          # dragged by the outliers
    assert oracle.rot_err(rej["R"], R_ref) < 1e-6
    assert oracle.trans_err(rej["t"], t_ref) < 1e-6
    assert rej["n"][-1] == 3000 - 60


def test_three_sigma_rejects_near_outliers():
    """Target spacing ~0.7 m; outliers 0.15-0.3 m off their copies: inside any
    useful max_dist, caught by 3 sigma once the inliers have converged."""
    T, S, R_ref, t_ref = _outlier_case(0.15, 0.3, extent=10.0, deg=0.5)
    plain = oracle.icp(T, S, iters=30, nn="brute")
    rej = oracle.icp(T, S, iters=30, nn="brute", reject_k=3.0)
    assert oracle.rot_err(plain["R"], R_ref) > 1e-4
    assert oracle.rot_err(rej["R"], R_ref) < 1e-6
    assert oracle.trans_err(rej["t"], t_ref) < 1e-6
    assert rej["kept"][-1] == 3000 - 60


def test_rejection_off_is_plain_icp():
    p = synth.tiny()
    a = oracle.icp(p.target, p.source, iters=5, nn="brute")
    b = oracle.icp(p.target, p.source, iters=5, nn="brute", max_dist=np.inf, reject_k=0.0)
    np.testing.assert_array_equal(a["R"], b["R"])
    np.testing.assert_array_equal(a["E"], b["E"])
