"""GPU parity of correspondence rejection (CUDA-KDTree ICP article, §4.4):
the max_dist bound fused into the search, the residual (3-sigma) rejection
step, and ICP with both, against the oracle.  Same bar as the plain path:
pairs and the kept set bit-exact, sums within 1e-5, R and t within 1e-4."""

import functools

import numpy as np
import pytest

import oracle
import synth
from tests.test_parity_gpu import (  # noqa: F401  (fixtures)
    R_TOL, T_TOL, assert_nn_equal, bbox_diag, check_sums, dev, kdnn, lidar, say, scene,
    scene_oracle_icp, torch,
)

pytestmark = pytest.mark.gpu

SCHED = [{}, {"lanes": 4}, {"lanes": 16}, {"budget": 4}, {"budget": 1}, {"top_lds": True}]
SCHED_IDS = ["default", "L4", "L16", "twopass-b4", "twopass-b1", "toplds"]


def bounded(oi, od, max_dist):
    """The oracle's bounded answer: the plain NN if within the bound, else none."""
    tau = oracle.max_dist_bound(max_dist)
    ok = (oi >= 0) & (od <= tau)
    return np.where(ok, oi, -1).astype(np.int32), np.where(ok, od, np.float32(np.inf)).astype(np.float32)


@pytest.mark.parametrize("sched", SCHED, ids=SCHED_IDS)
def test_radius_query_tiny_and_scene(torch, kdnn, sched):
    for name, p, dists in (("tiny", synth.tiny(), (0.005, 0.02, 0.1, 0.0, np.inf)),
                           ("scene", scene(), (0.02, 0.3, 1.0, 8.0))):
        tree = kdnn.Tree(p.target, p.leaf_size)
        q = p.source
        oi, od = oracle.KDTree(p.target, 8).query(q)
        for md in dists:
            for sort in (True, False):
                say("radius", name, md, sort, sched)
                idx, d2 = tree.query(dev(torch, q), sort=sort, max_dist=md, **sched)
                ei, ed = (oi, od) if (md <= 0 or not np.isfinite(md)) else bounded(oi, od, md)
                assert_nn_equal(idx, d2, ei, ed, f"radius {name} {md} sort={sort} {sched}")


@pytest.mark.parametrize("sched", SCHED, ids=SCHED_IDS)
def test_radius_bound_is_inclusive_with_lowest_index(torch, kdnn, sched):
    """Integer grid: every query has several targets at exactly distance 1."""
    g = np.arange(6, dtype=np.float32)
    T = np.stack(np.meshgrid(g, g, g, indexing="ij"), -1).reshape(-1, 3)
    rng = np.random.Generator(np.random.PCG64(5))
    T = T[rng.permutation(len(T))]                       # index order unrelated to position
    Q = T[:50] + np.array([0.5, 0.5, 0.0], np.float32)   # ties at d2 = 0.5 ...
    Q2 = T[50:100] + np.array([1.0, 0.0, 0.0], np.float32)  # ... and exactly on a neighbour
    Q = np.concatenate([Q, Q2])
    oi, od = oracle.brute_nn(T, Q)
    tree = kdnn.Tree(T, 4)
    # sqrt(0.5)^2 rounds to 0.5 in fp32 (ties at d2 = 0.5 kept); 0.70710677^2
    # rounds just below 0.5 (those ties dropped); 1.0 keeps the d2 = 1 cases
    for md in (np.sqrt(0.5), 0.5, 1.0, 0.70710677):
        say("radius ties", md, sched)
        idx, d2 = tree.query(dev(torch, Q), max_dist=md, **sched)
        ei, ed = bounded(oi, od, md)
        assert_nn_equal(idx, d2, ei, ed, f"radius ties {md} {sched}")


def _accepted_pairs(p, R, t, otree, max_dist):
    q = oracle.transform(p.source, R, t)
    oi, od = otree.query(q)
    ei, ed = bounded(oi, od, max_dist)
    ok = ei >= 0
    return ei, ed, ok


def test_scene_correspond_with_max_dist(torch, kdnn):
    p = scene()
    otree, o = scene_oracle_icp()
    tree = kdnn.Tree(p.target, 16)
    src = dev(torch, p.source)
    diag = bbox_diag(p.target)
    for k in (0, 29):
        R = o["Rt_hist"][k, :9].reshape(3, 3)
        t = o["Rt_hist"][k, 9:]
        for md in (0.25, 1.0):
            say("scene correspond max_dist", k, md)
            ei, ed, ok = _accepted_pairs(p, R, t, otree, md)
            red = oracle.reduce_pairs(p.source[ok], p.target[ei[ok]], ed[ok])
            for f in (0, 2, 4):
                res = tree.correspond_reduce(src, R, t, return_pairs=True, flags=f, max_dist=md)
                assert_nn_equal(res["idx"], res["d2"], ei, ed, f"pairs it{k} md{md} f{f}")
                check_sums(res, red, diag, f"sums it{k} md{md} f{f}")


def test_scene_reject_step_matches_oracle(torch, kdnn):
    """Given the same first solve (R1, t1), the kept set is bit-exact."""
    p = scene()
    otree, o = scene_oracle_icp()
    tree = kdnn.Tree(p.target, 16)
    src = dev(torch, p.source)
    ws = tree.icp_workspace(len(p.source))
    diag = bbox_diag(p.target)
    for k in (0, 10, 29):
        R = o["Rt_hist"][k, :9].reshape(3, 3)
        t = o["Rt_hist"][k, 9:]
        for md, kk in ((1.0, 3.0), (np.inf, 3.0), (0.5, 2.0)):
            say("scene reject", k, md, kk)
            ei, ed, ok = _accepted_pairs(p, R, t, otree, md)
            Sp, Mp, dp = p.source[ok], p.target[ei[ok]], ed[ok]
            R1, t1 = oracle.solve_rigid(oracle.reduce_pairs(Sp, Mp, dp))
            keep, sigma2, _ = oracle.reject_sigma(Sp, Mp, R1, t1, kk)
            red2 = oracle.reduce_pairs(Sp[keep], Mp[keep], dp[keep])
            tree.correspond_reduce(src, R, t, workspace=ws, max_dist=md, reject_k=kk)
            res = tree.reject_reduce(src, R1, t1, kk, ws, return_kept=True)
            kept = res["kept"].cpu().numpy().astype(bool)
            exp = np.zeros(len(p.source), bool)
            exp[np.nonzero(ok)[0][keep]] = True
            bad = np.nonzero(kept != exp)[0]
            assert len(bad) == 0, f"kept set differs at {bad[:5]}"
            assert res["sigma2"] == pytest.approx(sigma2, rel=1e-12)
            check_sums(res, red2, diag, f"reject sums it{k} md{md} k{kk}")


@functools.lru_cache(maxsize=None)
def scene_oracle_icp_reject(md, kk):
    p = scene()
    otree, _ = scene_oracle_icp()
    return oracle.icp(p.target, p.source, p.iters, tree=otree, max_dist=md, reject_k=kk)


@pytest.mark.parametrize("md,kk", [(1.0, 0.0), (1.0, 3.0), (None, 3.0)])
def test_scene_icp_with_rejection(torch, kdnn, md, kk):
    p = scene()
    o = scene_oracle_icp_reject(md, kk)
    tree = kdnn.Tree(p.target, 16)
    for sched in ({}, {"sort": True}, {"lanes": 4}, {"budget": 8}):
        say("scene icp reject", md, kk, sched)
        g = tree.icp(dev(torch, p.source), max_iter=p.iters, max_dist=md, reject_k=kk, **sched)
        assert g["iters"] == p.iters
        np.testing.assert_allclose(g["E"], o["E"], rtol=1e-9)
        assert np.linalg.norm(g["R"] - o["R"]) <= R_TOL
        assert np.max(np.abs(g["t"] - o["t"])) <= T_TOL


def test_outlier_case_recovers_truth(torch, kdnn):
    """Noise-free copy + 2% gross outliers: max_dist and 3 sigma both recover
    the generating motion, as the oracle does."""
    rng = np.random.Generator(np.random.PCG64(31))
    T = (rng.random((3000, 3)) * 10.0).astype(np.float32)
    Rg = synth.rotation_about(synth.random_unit(rng), np.deg2rad(0.5))
    tg = np.array([0.02, -0.01, 0.005])
    S = T.astype(np.float64) @ Rg.T + tg
    k = rng.choice(len(S), 60, replace=False)
    d = rng.normal(size=(60, 3))
    S[k] += d / np.linalg.norm(d, axis=1, keepdims=True) * rng.uniform(0.15, 0.3, size=(60, 1))
    S = S.astype(np.float32)
    tree = kdnn.Tree(T, 8)
    for md, kk in ((None, 3.0), (0.1, 0.0), (0.5, 3.0)):
        say("outlier case", md, kk)
        o = oracle.icp(T, S, 30, leaf_size=8, max_dist=md, reject_k=kk)
        g = tree.icp(dev(torch, S), max_iter=30, max_dist=md, reject_k=kk)
        assert np.linalg.norm(g["R"] - o["R"]) <= R_TOL
        assert np.max(np.abs(g["t"] - o["t"])) <= T_TOL
        assert oracle.rot_err(g["R"], Rg.T) < 1e-5


def test_lidar_pair_icp_with_rejection(torch, kdnn):
    p = lidar()[3]
    o = oracle.icp(p.target, p.source, p.iters, leaf_size=16, max_dist=1.0, reject_k=3.0)
    tree = kdnn.Tree(p.target, 16)
    say("lidar pair 3 icp reject")
    g = tree.icp(dev(torch, p.source), max_iter=p.iters, max_dist=1.0, reject_k=3.0)
    assert np.linalg.norm(g["R"] - o["R"]) <= R_TOL
    assert np.max(np.abs(g["t"] - o["t"])) <= T_TOL


def test_reject_argument_errors(torch, kdnn):
    p = synth.tiny()
    tree = kdnn.Tree(p.target, 8)
    src = dev(torch, p.source)
    ws = tree.icp_workspace(len(p.source))
    for bad in (-1.0, np.inf, np.nan):
        with pytest.raises(kdnn.KdnnError, match="EINVAL"):
            tree.correspond_reduce(src, workspace=ws, reject_k=bad)
        with pytest.raises(kdnn.KdnnError, match="EINVAL"):
            tree.icp(src, max_iter=2, workspace=ws, reject_k=bad)
    for bad in (0.0, -2.0, np.nan):
        with pytest.raises(kdnn.KdnnError, match="EINVAL"):
            tree.reject_reduce(src, np.eye(3), np.zeros(3), bad, ws)
    with pytest.raises(kdnn.KdnnError, match="EINVAL"):
        tree.query(src, max_dist=np.nan)
