"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar (per the acceptance rules of the path):
  * nn_query / the fused kernel's pairs: idx and dist2 bit-exact;
  * transform_points: bit-exact;
  * correspondence sums: ||H - H_o||_F <= 1e-5 ||H_o||_F and centroids within
    1e-5 * max(||mu_o||, bbox diagonal);
  * icp_align: ||R - R_o||_F <= 1e-4, ||t - t_o||_inf <= 1e-4.
Every case prints its name before touching the device.
"""

import functools
import sys

import numpy as np
import pytest

import oracle
import synth
from tests._cases import adversarial_clouds, load_nn_cases

pytestmark = pytest.mark.gpu

# search schedules: single pass with g lanes per query, or the default two-pass
# schedule (tiny budgets push nearly every query into the second pass)
SCHED = [{}, {"lanes": 4}, {"lanes": 16}, {"budget": 64}, {"budget": 1}, {"budget": 4},
         {"top_lds": True}]
SCHED_IDS = ["default", "L4", "L16", "twopass-b64", "twopass-b1", "twopass-b4", "toplds"]
SCHED_FEW = [{}, {"budget": 64}, {"budget": 2}, {"top_lds": True}]
SCHED_FEW_IDS = ["default", "twopass-b64", "twopass-b2", "toplds"]

H_RTOL = 1e-5
MU_RTOL = 1e-5
R_TOL = 1e-4
T_TOL = 1e-4


def say(*a):
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "GPU tests need a HIP device"
    return _t


@pytest.fixture(scope="module")
def kdnn(torch):
    import kd_tree_nn_amd
    from kd_tree_nn_amd import _lib
    _lib.lib()  # fail loudly if the library is missing
    return kd_tree_nn_amd


def dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def assert_nn_equal(idx, d2, oi, od, what):
    idx = idx.cpu().numpy() if hasattr(idx, "cpu") else idx
    d2 = d2.cpu().numpy() if hasattr(d2, "cpu") else d2
    bad = np.nonzero((idx != oi) | (d2.view(np.uint32) != od.view(np.uint32)))[0]
    assert len(bad) == 0, (f"{what}: {len(bad)} mismatches, first {bad[:5]}: "
                           f"gpu {idx[bad[:5]]} {d2[bad[:5]]} oracle {oi[bad[:5]]} {od[bad[:5]]}")


def check_sums(res, red, bbox_diag, what):
    assert res["n"] == red["n"], what
    Hn = np.linalg.norm(red["H"])
    assert np.linalg.norm(res["H"] - red["H"]) <= H_RTOL * Hn, (what, res["H"], red["H"])
    for k in ("mu_s", "mu_m"):
        scale = max(np.linalg.norm(red[k]), bbox_diag)
        assert np.linalg.norm(res[k] - red[k]) <= MU_RTOL * scale, (what, k, res[k], red[k])
    assert abs(res["E"] - red["E"]) <= 1e-9 * max(red["E"], 1e-30), (what, res["E"], red["E"])


def bbox_diag(T):
    return float(np.linalg.norm(T.max(0).astype(np.float64) - T.min(0)))


# ----------------------------------------------------------- cached inputs
@functools.lru_cache(maxsize=None)
def scene():
    return synth.scene()


@functools.lru_cache(maxsize=None)
def scene_oracle_icp():
    p = scene()
    tr = oracle.KDTree(p.target, 16)
    return tr, oracle.icp(p.target, p.source, p.iters, tree=tr)


@functools.lru_cache(maxsize=None)
def lidar():
    return synth.lidar_pairs()


@functools.lru_cache(maxsize=None)
def lidar_oracle(k):
    """The oracle's KD-tree of LiDAR pair k's target and its 30-iteration ICP
    (about 7 s on the host; cached for the session)."""
    p = lidar()[k]
    tr = oracle.KDTree(p.target, 16)
    return tr, oracle.icp(p.target, p.source, p.iters, tree=tr)


# ======================================================== nearest neighbour
@pytest.mark.parametrize("sched", SCHED, ids=SCHED_IDS)
@pytest.mark.parametrize("sort", [True, False])
@pytest.mark.parametrize("leaf", [1, 2, 8])
def test_golden_nn(torch, kdnn, leaf, sort, sched):
    for k, (T, Q, I, D) in enumerate(load_nn_cases()):
        say("golden", k, "leaf", leaf, "sort", sort, sched)
        tree = kdnn.Tree(T, leaf)
        idx, d2 = tree.query(dev(torch, Q), sort=sort, **sched)
        assert_nn_equal(idx, d2, I, D, f"golden set {k}")


@pytest.mark.parametrize("sched", SCHED + [{"lanes": 2}, {"lanes": 8}],
                         ids=SCHED_IDS + ["L2", "L8"])
@pytest.mark.parametrize("sort", [True, False])
@pytest.mark.parametrize("leaf", [1, 3, 8, 16])
def test_adversarial_nn(torch, kdnn, leaf, sort, sched):
    for name, T, Q in adversarial_clouds():
        say("adversarial", name, "leaf", leaf, "sort", sort, sched, len(T), len(Q))
        oi, od = oracle.brute_nn(T, Q)
        idx, d2 = kdnn.Tree(T, leaf).query(dev(torch, Q), sort=sort, **sched)
        assert_nn_equal(idx, d2, oi, od, f"{name} {sched}")


@pytest.mark.parametrize("m", [1, 2, 63, 64, 65, 255, 256, 257, 2047, 2048, 2049, 4097, 10007])
def test_ragged_query_counts(torch, kdnn, m):
    rng = np.random.Generator(np.random.PCG64(m))
    T = rng.random((5000, 3)).astype(np.float32)
    Q = rng.random((m, 3)).astype(np.float32) * 1.2 - 0.1
    say("ragged m", m)
    oi, od = oracle.brute_nn(T, Q)
    tree = kdnn.Tree(T, 8)
    for sort in (True, False):
        for sched in SCHED:
            idx, d2 = tree.query(dev(torch, Q), sort=sort, **sched)
            assert_nn_equal(idx, d2, oi, od, f"m={m} sort={sort} {sched}")


@pytest.mark.parametrize("n", [1000, 2000, 4000, 8000])
def test_depth_around_the_lds_planes(torch, kdnn, n):
    """Point location reads the top 8 levels' planes from LDS and the rest
    from memory: trees of depth 7-10 (all planes in LDS, exactly the LDS
    levels, one and two levels below them), searches without a start leaf
    (nn_query, the instrumented search, the fused correspondence kernel)."""
    rng = np.random.Generator(np.random.PCG64(n))
    T = rng.normal(size=(n, 3)).astype(np.float32)
    Q = (rng.normal(size=(3001, 3)) * 1.1).astype(np.float32)
    tree = kdnn.Tree(T, 8)
    D = tree.info["depth"]
    say("depth around the LDS planes", n, "depth", D)
    assert D == {1000: 7, 2000: 8, 4000: 9, 8000: 10}[n]
    oi, od = oracle.brute_nn(T, Q)
    for sort in (True, False):
        idx, d2 = tree.query(dev(torch, Q), sort=sort)
        assert_nn_equal(idx, d2, oi, od, f"n={n} sort={sort}")
    si, sd, cn, _ = tree.query_stats(dev(torch, Q))
    assert_nn_equal(si, sd, oi, od, f"n={n} stats")
    assert int(cn.min()) >= D - min(D, 8) + 2
    R, t = synth.rotation_about(synth.random_unit(rng), 0.2), rng.normal(size=3) * 0.1
    oi, od, red = _pairs_oracle(T, Q, R, t)
    res = tree.correspond_reduce(dev(torch, Q), R, t, return_pairs=True)
    assert_nn_equal(res["idx"], res["d2"], oi, od, f"n={n} correspond_reduce")
    check_sums(res, red, bbox_diag(T), f"n={n} correspond_reduce sums")


def test_nonfinite_and_empty(torch, kdnn):
    say("nonfinite / empty")
    rng = np.random.Generator(np.random.PCG64(3))
    T = rng.random((300, 3)).astype(np.float32)
    Q = rng.random((40, 3)).astype(np.float32)
    Q[3, 0] = np.nan
    Q[7, 2] = np.inf
    Q[11, 1] = -np.inf
    Q[20] = [1e30, 0, 0]          # every distance overflows to +inf
    oi, od = oracle.brute_nn(T, Q)
    assert oi[3] == -1 and oi[7] == -1 and oi[20] == -1
    tree = kdnn.Tree(T, 8)
    for sort in (True, False):
        for sched in SCHED:
            idx, d2 = tree.query(dev(torch, Q), sort=sort, **sched)
            assert_nn_equal(idx, d2, oi, od, f"nonfinite {sched}")
    idx, d2 = tree.query(torch.empty((0, 3), dtype=torch.float32, device="cuda"))
    assert idx.numel() == 0 and d2.numel() == 0


def test_single_point_tree(torch, kdnn):
    say("single point tree")
    T = np.array([[0.5, -2.0, 7.0]], np.float32)
    Q = np.random.Generator(np.random.PCG64(1)).normal(size=(100, 3)).astype(np.float32)
    oi, od = oracle.brute_nn(T, Q)
    idx, d2 = kdnn.Tree(T, 16).query(dev(torch, Q))
    assert_nn_equal(idx, d2, oi, od, "single")
    assert kdnn.Tree(T, 16).info["depth"] == 0


def test_depth_cap_and_round_robin(torch, kdnn):
    rng = np.random.Generator(np.random.PCG64(8))
    T = np.concatenate([rng.random((3000, 3)), rng.random((3000, 3)) * [1, 0.01, 0.01]]).astype(np.float32)
    Q = rng.random((2000, 3)).astype(np.float32)
    oi, od = oracle.brute_nn(T, Q)
    for kw in ({"max_depth": 4}, {"round_robin": True}, {"max_depth": 6, "round_robin": True}):
        for sched in SCHED:
            say("build variant", kw, sched)
            idx, d2 = kdnn.Tree(T, 8, **kw).query(dev(torch, Q), **sched)
            assert_nn_equal(idx, d2, oi, od, f"{kw} {sched}")


def test_query_stats_consistent(torch, kdnn):
    say("query stats")
    p = synth.tiny()
    tree = kdnn.Tree(p.target, 8)
    q = dev(torch, p.source)
    idx, d2 = tree.query(q)
    D = tree.info["depth"]
    for sched in SCHED:
        si, sd, cn, cp = tree.query_stats(q, **sched)
        assert torch.equal(idx, si) and torch.equal(d2.view(torch.int32), sd.view(torch.int32))
        # at least the location planes below the 8 levels kept in LDS and the
        # start leaf's plane record (two records)
        assert int(cn.min()) >= D - min(D, 8) + 2 and int(cp.min()) >= 1
        # a search never loads a node twice, except the greedy descent a second
        # pass repeats; a pruning search loads far fewer than all of them
        assert int(cn.max()) <= 2 ** (D + 1) + 2 * (D + 1)
        if sched in ({"lanes": 1}, {}, {"budget": 64}):
            assert float(cn.float().mean()) < 0.25 * 2 ** (D + 1)
    # default schedule: each query's own single-lane counts, whichever queries
    # share its wavefront (given order, a permutation, the Morton order)
    perm = torch.randperm(len(q), generator=torch.Generator().manual_seed(3)).cuda()
    _, _, cn1, cp1 = tree.query_stats(q)
    _, _, cn2, cp2 = tree.query_stats(q[perm].contiguous())
    assert torch.equal(cn1[perm], cn2) and torch.equal(cp1[perm], cp2)
    _, _, cn3, cp3 = tree.query_stats(q, sort=True)
    assert torch.equal(cn1, cn3) and torch.equal(cp1, cp3)


# ================================================================ transform
def test_transform_bit_exact(torch, kdnn):
    say("transform")
    rng = np.random.Generator(np.random.PCG64(12))
    P = (rng.normal(size=(100_003, 3)) * 40).astype(np.float32)
    for R, t in [(np.eye(3), np.zeros(3)),
                 (synth.rotation_about(synth.random_unit(rng), 0.7), rng.normal(size=3) * 5),
                 (synth.rot_z(np.pi / 2), np.array([1.0, -2.0, 0.25]))]:
        exp = oracle.transform(P, R, t)
        x = dev(torch, P)
        out = kdnn.transform(x, R, t)
        np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), exp.view(np.uint32))
        kdnn.transform(x, R, t, out=x)           # in place
        np.testing.assert_array_equal(x.cpu().numpy().view(np.uint32), exp.view(np.uint32))
    # fixed association (see the oracle pin): left-to-right fp64 sums, one cast
    R = np.eye(3)
    R[0] = [1.0, 2.0 ** -53, 2.0 ** -53]
    out = kdnn.transform(dev(torch, np.ones((1, 3))), R, [2.0 ** -24, 0.0, 0.0])
    assert out[0, 0].item() == 1.0
    empty = torch.empty((0, 3), dtype=torch.float32, device="cuda")
    assert kdnn.transform(empty, np.eye(3), np.zeros(3)).numel() == 0


# ===================================================================== ICP
def _pairs_oracle(T, S, R, t, tree=None):
    q = oracle.transform(S, R, t)
    oi, od = tree.query(q) if tree is not None else oracle.brute_nn(T, q)
    ok = oi >= 0
    return oi, od, oracle.reduce_pairs(S[ok], T[oi[ok]], od[ok])


def test_tiny_correspond_reduce_and_icp(torch, kdnn):
    p = synth.tiny()
    tree = kdnn.Tree(p.target, 8)
    src = dev(torch, p.source)
    diag = bbox_diag(p.target)
    from kd_tree_nn_amd import _lib
    for name, R, t in [("identity", np.eye(3), np.zeros(3)), ("truth", p.R_true, p.t_true)]:
        oi, od, red = _pairs_oracle(p.target, p.source, R, t)
        for f in (0, _lib.lanes_flag(None, 1), _lib.lanes_flag(None, 5), _lib.lanes_flag(1),
                  _lib.lanes_flag(4) | 2, _lib.KDNN_ICP_SORT, _lib.KDNN_ICP_SORT | _lib.lanes_flag(None, 3)):
            say("tiny correspond_reduce", name, hex(f))
            res = tree.correspond_reduce(src, R, t, return_pairs=True, flags=f)
            assert_nn_equal(res["idx"], res["d2"], oi, od, f"tiny pairs {name} {f:#x}")
            check_sums(res, red, diag, f"tiny sums {name} {f:#x}")
    o = oracle.icp(p.target, p.source, p.iters, nn="brute")
    oe = oracle.icp(p.target, p.source, 50, nn="brute", eps=1e-7)
    for kw in ({}, {"device_loop": True}):
        say("tiny icp_align", kw)
        g = tree.icp(src, max_iter=p.iters, **kw)
        assert g["iters"] == p.iters
        assert np.linalg.norm(g["R"] - o["R"]) <= R_TOL and np.max(np.abs(g["t"] - o["t"])) <= T_TOL
        np.testing.assert_allclose(g["E"], o["E"], rtol=1e-6)
        # recovers the generating motion within the noise
        assert np.degrees(oracle.rot_err(g["R"], p.R_true)) < 0.1
        # convergence rule matches the oracle's
        say("tiny icp eps", kw)
        ge = tree.icp(src, max_iter=50, eps=1e-7, **kw)
        assert ge["iters"] == oe["iters"]


def test_scene_nn_full(torch, kdnn):
    p = scene()
    otree, o = scene_oracle_icp()
    tree = kdnn.Tree(p.target, 16)
    info = tree.info
    assert info["depth"] == 13 and info["min_leaf"] == 12 and info["max_leaf"] == 13
    for name, Q in [("iteration-0 queries", p.source),
                    ("converged queries", oracle.transform(p.source, o["R"], o["t"]))]:
        oi, od = otree.query(Q)
        for sort in (True, False):
            for sched in SCHED:
                say("scene nn", name, "sort", sort, sched)
                idx, d2 = tree.query(dev(torch, Q), sort=sort, **sched)
                assert_nn_equal(idx, d2, oi, od, f"scene {name} sort={sort} {sched}")


def test_scene_correspond_reduce(torch, kdnn):
    p = scene()
    otree, o = scene_oracle_icp()
    tree = kdnn.Tree(p.target, 16)
    src = dev(torch, p.source)
    diag = bbox_diag(p.target)
    for k in (0, 1, 10, 29):
        R = o["Rt_hist"][k, :9].reshape(3, 3)
        t = o["Rt_hist"][k, 9:]
        say("scene correspond_reduce iteration", k)
        oi, od, red = _pairs_oracle(p.target, p.source, R, t, otree)
        from kd_tree_nn_amd import _lib
        for f in (0, _lib.lanes_flag(None, 2), _lib.lanes_flag(1), _lib.lanes_flag(16),
                  _lib.lanes_flag(top_lds=True), _lib.KDNN_ICP_SORT, _lib.KDNN_ICP_NO_SORT,
                  _lib.KDNN_ICP_SORT | _lib.lanes_flag(None, 2)):
            res = tree.correspond_reduce(src, R, t, return_pairs=True, flags=f)
            assert_nn_equal(res["idx"], res["d2"], oi, od, f"scene pairs it{k} flags {f:#x}")
            check_sums(res, red, diag, f"scene sums it{k} flags {f:#x}")
            assert res["E"] == pytest.approx(o["E"][k], rel=1e-12)


def test_scene_icp_align(torch, kdnn):
    p = scene()
    _, o = scene_oracle_icp()
    tree = kdnn.Tree(p.target, 16)
    for sched in SCHED + [{"lanes": 1}, {"sort": False}, {"sort": False, "budget": 3},
                          {"sort": True}, {"sort": True, "budget": 3}, {"device_loop": True},
                          {"device_loop": True, "sort": True}]:
        say("scene icp_align 30", sched)
        g = tree.icp(dev(torch, p.source), max_iter=p.iters, **sched)
        assert g["iters"] == p.iters
        dR = np.linalg.norm(g["R"] - o["R"])
        dt = np.max(np.abs(g["t"] - o["t"]))
        assert dR <= R_TOL and dt <= T_TOL, (sched, dR, dt)
        np.testing.assert_allclose(g["E"], o["E"], rtol=1e-6)
        np.testing.assert_allclose(g["Rt_hist"], o["Rt_hist"], atol=1e-6)


def test_device_loop_matches_host_loop(torch, kdnn):
    """icp_align solves each iteration on the host (SVD) unless asked to keep
    the iterations on the device (the step kernel sums the same partials in
    the same order and solves with Horn's quaternion form; with residual
    rejection both solves of an iteration): both must follow the same
    iterates.  The two solvers agree to ~1e-15, so the searches see the same
    queries except where a coordinate sits within that of an fp32 rounding
    boundary; the bar is 1e-9."""
    for name, p, leaf in [("tiny", synth.tiny(), 8), ("scene", scene(), 16),
                          ("lidar 5", lidar()[5], 16)]:
        tree = kdnn.Tree(p.target, leaf)
        src = dev(torch, p.source)
        for kw in ({}, {"sort": True}, {"max_dist": 1.0}, {"max_dist": 1.0, "reject_k": 3.0},
                   {"reject_k": 2.5}):
            say("device vs host loop", name, kw)
            d = tree.icp(src, max_iter=p.iters, device_loop=True, **kw)
            h = tree.icp(src, max_iter=p.iters, **kw)
            assert d["iters"] == h["iters"] == p.iters, (name, kw)
            np.testing.assert_allclose(d["E"], h["E"], rtol=1e-9, err_msg=f"{name} {kw}")
            np.testing.assert_allclose(d["Rt_hist"], h["Rt_hist"], rtol=0, atol=1e-9)
            assert np.linalg.norm(d["R"] - h["R"]) <= 1e-9 and np.max(np.abs(d["t"] - h["t"])) <= 1e-9
            say("  bit-identical:", bool(np.array_equal(d["Rt_hist"], h["Rt_hist"])))


def _step_by_step(kdnn, tree, src, iters, sort, max_dist=None, eps=0.0):
    """icp_align's host loop spelled out through the C ABI: one
    icp_correspond_reduce per iteration (the transform as kernel arguments),
    kdnn_procrustes on its sums, the convergence rule in Python."""
    from kd_tree_nn_amd import _lib
    first = _lib.KDNN_ICP_SORT if sort else _lib.KDNN_ICP_NO_SORT
    R, t = np.eye(3), np.zeros(3)
    ws = tree.icp_workspace(src.shape[0])
    E, hist = [], []
    prev, small = 0.0, 0
    for k in range(iters):
        hist.append(np.concatenate([R.ravel(), t]))
        flags = first if k == 0 else first | _lib.KDNN_ICP_REUSE_ORDER
        sums = tree.correspond_reduce(src, R, t, flags=flags, workspace=ws, max_dist=max_dist)
        E.append(sums["E"])
        R, t = kdnn.procrustes(sums)
        mse = sums["E"] / sums["n"]
        if eps > 0.0 and k > 0:
            small = small + 1 if abs(mse - prev) < eps else 0
            if small >= 2:
                break
        prev = mse
    return R, t, np.array(E), np.array(hist)


def test_host_loop_matches_step_by_step(torch, kdnn):
    """icp_align's host loop (sums into the tree's pinned slot, completion
    word, host SVD, next launch) must follow, bit for bit, the same loop made
    of separate icp_correspond_reduce and kdnn_procrustes calls -- including
    where the convergence rule stops it."""
    for name, p, leaf in [("tiny", synth.tiny(), 8), ("scene", scene(), 16),
                          ("lidar 5", lidar()[5], 16)]:
        tree = kdnn.Tree(p.target, leaf)
        src = dev(torch, p.source)
        auto = bool(tree.info["auto_sort_icp"])
        for kw in ({}, {"sort": True}, {"sort": False}, {"max_dist": 1.0}, {"eps": 1e-7}):
            say("host loop vs step by step", name, kw)
            sort = kw.get("sort", auto)
            g = tree.icp(src, max_iter=p.iters, **kw)
            R, t, E, hist = _step_by_step(kdnn, tree, src, p.iters, sort, kw.get("max_dist"),
                                          kw.get("eps", 0.0))
            assert g["iters"] == len(E), (name, kw, g["iters"], len(E))
            np.testing.assert_array_equal(g["E"][:len(E)], E)
            np.testing.assert_array_equal(g["Rt_hist"][:len(E)], hist)
            np.testing.assert_array_equal(g["R"], R)
            np.testing.assert_array_equal(g["t"], t)
    # a failed solve: the call reports it, and the tree's slot and the stream
    # are left ready for the next call
    p = synth.tiny()
    tree = kdnn.Tree(p.target, 8)
    src = dev(torch, p.source)
    say("host loop, degenerate first iteration")
    with pytest.raises(kdnn.KdnnError, match="EDEGENERATE"):
        tree.icp(src, max_iter=5, R0=synth.rot_z(0.0), t0=[100.0, 0.0, 0.0], max_dist=0.01)
    g = tree.icp(src, max_iter=p.iters)
    o = oracle.icp(p.target, p.source, p.iters, nn="brute")
    assert g["iters"] == p.iters
    assert np.linalg.norm(g["R"] - o["R"]) <= R_TOL and np.max(np.abs(g["t"] - o["t"])) <= T_TOL


def test_warm_start_ties_and_gaps(torch, kdnn):
    """Iterations after the first start each search at the leaf of the point's
    previous match.  On a lattice target with sources at cell centres (8 target
    points at exactly the same distance, lowest index wins), with NaN sources
    (no match, no warm start) and far outliers, every iterate must still equal
    the loop of separate root-start calls bit for bit, under max_dist too.
    Lattice coordinates put many points exactly on split planes (on both
    sides of them), the case the plane bounds of the warm start must get
    right; the 26^3 lattice with one point per leaf is deeper (D = 15) than
    the 14 levels of a leaf's plane record, so its searches also bound the
    subtree below the root by its box."""
    for side, leaf in ((12, 1), (12, 8), (12, 16), (26, 1)):
        g = np.stack(np.meshgrid(*(np.arange(side, dtype=np.float32),) * 3, indexing="ij"), -1)
        tgt = g.reshape(-1, 3)
        rng = np.random.Generator(np.random.PCG64(17))
        tgt = tgt[rng.permutation(len(tgt))]                  # ties between unrelated indices
        src = (g[:-1, :-1, :-1] + 0.5).reshape(-1, 3).astype(np.float32)
        src = np.concatenate([src, np.full((3, 3), np.nan, np.float32),
                              np.array([[60.0, 5.0, 5.0], [-40.0, -40.0, 3.0]], np.float32)])
        tree = kdnn.Tree(tgt, leaf)
        if side == 26:
            assert tree.info["depth"] > 14
        sd = dev(torch, src)
        auto = bool(tree.info["auto_sort_icp"])
        for kw in ({}, {"max_dist": 0.9}, {"sort": True}):
            say("warm start ties and gaps, lattice", side, "leaf", leaf, kw)
            gi = tree.icp(sd, max_iter=6, R0=synth.rot_z(0.0), t0=[0.0, 0.0, 0.0], **kw)
            R, t, E, hist = _step_by_step(kdnn, tree, sd, 6, kw.get("sort", auto),
                                          kw.get("max_dist"))
            assert gi["iters"] == len(E) == 6
            np.testing.assert_array_equal(gi["E"], E)
            np.testing.assert_array_equal(gi["Rt_hist"], hist)
            np.testing.assert_array_equal(gi["R"], R)
            np.testing.assert_array_equal(gi["t"], t)


@pytest.mark.parametrize("leaf", [1, 3, 16])
def test_warm_start_adversarial(torch, kdnn, leaf):
    """Warm-started iterations on the adversarial clouds (exact ties on grids,
    heavy duplication, coplanar and collinear targets, tight clusters with far
    queries, trees with empty leaves): the host loop, whose iterations after
    the first start at each point's previous leaf, must equal the loop of
    separate calls bit for bit; a degenerate registration must fail the same
    way in both."""
    compared = 0
    for name, T, Q in adversarial_clouds():
        if len(Q) < 3:
            continue
        tree = kdnn.Tree(T, leaf)
        sd = dev(torch, Q)
        auto = bool(tree.info["auto_sort_icp"])
        say("warm start adversarial", name, "leaf", leaf, len(T), len(Q))
        status = []
        try:
            gi = tree.icp(sd, max_iter=5, R0=synth.rot_z(0.0), t0=[0.0, 0.0, 0.0])
            status.append(None)
        except kdnn.KdnnError as err:
            status.append(err.status)
        try:
            R, t, E, hist = _step_by_step(kdnn, tree, sd, 5, auto)
            status.append(None)
        except kdnn.KdnnError as err:
            status.append(err.status)
        assert status[0] == status[1], (name, status)
        if status[0] is not None:
            continue
        assert gi["iters"] == len(E), name
        np.testing.assert_array_equal(gi["E"], E, err_msg=name)
        np.testing.assert_array_equal(gi["Rt_hist"], hist, err_msg=name)
        np.testing.assert_array_equal(gi["R"], R, err_msg=name)
        np.testing.assert_array_equal(gi["t"], t, err_msg=name)
        compared += 1
    assert compared >= 5  # the grid, duplicate, planar, cluster and coarse sets at least


def test_device_loop_eps_and_limits(torch, kdnn):
    """Convergence stop at every phase of the 4-iteration chunks, the host
    fallback beyond the record's 512 iterations, and a degenerate first
    iteration (no pair within max_dist): EDEGENERATE, transform unchanged."""
    p = synth.tiny()
    tree = kdnn.Tree(p.target, 8)
    src = dev(torch, p.source)
    for eps in (1e-5, 1e-6, 1e-7, 1e-8, 1e-9):
        say("device loop eps", eps)
        o = oracle.icp(p.target, p.source, 60, nn="brute", eps=eps)
        d = tree.icp(src, max_iter=60, eps=eps, device_loop=True)
        h = tree.icp(src, max_iter=60, eps=eps)
        assert d["iters"] == h["iters"] == o["iters"], (eps, d["iters"], h["iters"], o["iters"])
        np.testing.assert_allclose(d["E"], o["E"], rtol=1e-6)
    say("host loop beyond the device record")
    g = tree.icp(src, max_iter=520)
    assert g["iters"] == 520 and len(g["E"]) == 520
    with pytest.raises(kdnn.KdnnError, match="EINVAL"):
        tree.icp(src, max_iter=520, device_loop=True)
    with pytest.raises(kdnn.KdnnError, match="EINVAL"):
        tree.icp(src, max_iter=5, device_loop=True, lanes=4)
    from kd_tree_nn_amd import _lib
    import ctypes
    far = dev(torch, (p.source + np.float32(100.0)).astype(np.float32))
    ws = tree.icp_workspace(len(p.source))
    R0 = synth.rotation_about([0, 0, 1], 0.1)
    t0 = np.array([0.5, -0.25, 2.0])
    for flags in (_lib.KDNN_ICP_DEVICE_LOOP, 0, _lib.KDNN_ICP_HOST_LOOP):
        say("device loop degenerate, flags", flags)
        R, t, E = np.zeros(9), np.zeros(3), np.zeros(5)
        it = ctypes.c_int32(-1)
        st = _lib.lib().icp_align(
            tree._h, ctypes.c_void_p(far.data_ptr()), len(p.source),
            np.ascontiguousarray(R0).ctypes.data_as(_lib.c_dp), t0.ctypes.data_as(_lib.c_dp), 5, 0.0,
            R.ctypes.data_as(_lib.c_dp), t.ctypes.data_as(_lib.c_dp), E.ctypes.data_as(_lib.c_dp),
            None, ctypes.byref(it), flags, ctypes.byref(_lib.IcpReject(0.5, 0.0)),
            ctypes.c_void_p(ws.data_ptr()), ws.numel(), None)
        assert st == _lib.KDNN_EDEGENERATE, st
        assert b"iteration 0" in _lib.lib().kdnn_last_error()
        assert it.value == 0
        np.testing.assert_array_equal(R.reshape(3, 3), R0)
        np.testing.assert_array_equal(t, t0)
        assert E[0] == 0.0  # no pair: the iteration's sum of squared distances


def test_determinism(torch, kdnn):
    p = scene()
    tree = kdnn.Tree(p.target, 16)
    src = dev(torch, p.source)
    say("determinism")
    R = synth.rot_z(0.05)
    a = tree.correspond_reduce(src, R, [0.1, 0.2, 0.0])
    b = tree.correspond_reduce(src, R, [0.1, 0.2, 0.0])
    for k in ("sum_s", "sum_m", "sum_sm"):
        np.testing.assert_array_equal(a[k], b[k])
    assert a["E"] == b["E"]
    for kw in ({}, {"device_loop": True}):
        g1 = tree.icp(src, max_iter=5, **kw)
        g2 = tree.icp(src, max_iter=5, **kw)
        np.testing.assert_array_equal(g1["R"], g2["R"])
    # the async entry point writes the same sums
    import torch as T
    ws = tree.icp_workspace(len(p.source))
    sums = T.zeros(17, dtype=T.float64, device="cuda")
    tree.correspond_reduce_async(src, R, [0.1, 0.2, 0.0], sums, ws)
    tree.correspond_reduce_async(src, R, [0.1, 0.2, 0.0], sums, ws, flags=kdnn.KDNN_ICP_REUSE_ORDER)
    s = sums.cpu().numpy()
    np.testing.assert_array_equal(s[0:3], a["sum_s"])
    np.testing.assert_array_equal(s[6:15].reshape(3, 3), a["sum_sm"])
    assert s[15] == a["E"] and s[16] == a["n"]
    # no-sort traversal gives the same pairs (sums may differ in the last bits)
    c = tree.correspond_reduce(src, R, [0.1, 0.2, 0.0], flags=kdnn.KDNN_ICP_NO_SORT)
    assert c["n"] == a["n"] and c["E"] == pytest.approx(a["E"], rel=1e-12)


def test_workspace_checks(torch, kdnn):
    say("workspace checks")
    p = synth.tiny()
    tree = kdnn.Tree(p.target, 8)
    src = dev(torch, p.source)
    small = torch.empty(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(kdnn.KdnnError, match="EINVAL"):
        tree.correspond_reduce(src, np.eye(3), np.zeros(3), workspace=small)
    with pytest.raises(kdnn.KdnnError, match="EINVAL"):
        tree.query(src, workspace=small)
    from kd_tree_nn_amd import _lib
    with pytest.raises(kdnn.KdnnError, match="EINVAL"):
        tree.correspond_reduce(src, np.eye(3), np.zeros(3),
                               flags=_lib.KDNN_ICP_SORT | _lib.KDNN_ICP_NO_SORT)
    m = src.shape[0]
    idx = torch.empty(m, dtype=torch.int32, device="cuda")
    d2 = torch.empty(m, dtype=torch.float32, device="cuda")
    ws = tree.query_workspace(m)
    L = _lib.lib()
    args = (tree._h, src.data_ptr(), m, idx.data_ptr(), d2.data_ptr())
    # the ordering and the two-pass schedule need a workspace; conflicting
    # order flags are rejected
    assert L.nn_query(*args, _lib.KDNN_QUERY_SORT, None, 0, None) == _lib.KDNN_EINVAL
    assert L.nn_query(*args, _lib.KDNN_QUERY_SORT | _lib.KDNN_QUERY_NO_SORT, ws.data_ptr(),
                      ws.numel(), None) == _lib.KDNN_EINVAL
    assert L.nn_query(*args, _lib.lanes_flag(None, 8), None, 0, None) == _lib.KDNN_EINVAL
    # automatic mode without a workspace: single pass in the given order
    assert L.nn_query(*args, 0, None, 0, None) == _lib.KDNN_OK
    for bad in (_lib.lanes_flag(4, 8), _lib.lanes_flag(1, None, True), _lib.lanes_flag(None, 8, True),
                _lib.lanes_flag(3)):
        assert L.nn_query(*args, bad, ws.data_ptr(), ws.numel(), None) == _lib.KDNN_EINVAL
    torch.cuda.synchronize()
    ri, rd = tree.query(src, sort=True)
    assert torch.equal(idx, ri) and torch.equal(d2.view(torch.int32), rd.view(torch.int32))


@functools.lru_cache(maxsize=None)
def stress_oracle():
    p = synth.stress()
    return p, oracle.KDTree(p.target, 8).query(p.source)


@pytest.mark.parametrize("sched", SCHED_FEW + [{"lanes": 4}], ids=SCHED_FEW_IDS + ["L4"])
@pytest.mark.parametrize("leaf", [8, 16])
def test_stress_nn(torch, kdnn, leaf, sched):
    p, (oi, od) = stress_oracle()
    say("stress 1M x 1M leaf", leaf, sched)
    tree = kdnn.Tree(p.target, leaf)
    assert tree.info["depth"] == (17 if leaf == 8 else 16)
    idx, d2 = tree.query(dev(torch, p.source), **sched)
    assert_nn_equal(idx, d2, oi, od, f"stress leaf {leaf} {sched}")


@functools.lru_cache(maxsize=None)
def skewed_oracle():
    p = synth.skewed()
    return p, oracle.KDTree(p.target, 8).query(p.source)


@pytest.mark.parametrize("sched", SCHED_FEW + [{"lanes": 16}], ids=SCHED_FEW_IDS + ["L16"])
@pytest.mark.parametrize("leaf", [8, 16])
def test_skewed_nn(torch, kdnn, leaf, sched):
    p, (oi, od) = skewed_oracle()
    say("skewed 500k leaf", leaf, sched)
    idx, d2 = kdnn.Tree(p.target, leaf).query(dev(torch, p.source), **sched)
    assert_nn_equal(idx, d2, oi, od, f"skewed leaf {leaf} {sched}")


@pytest.mark.parametrize("k", range(16))
def test_lidar_pairs(torch, kdnn, k):
    """Every one of the 16 consecutive-frame registrations (article §3.4):
    identity-pose pairs bit-exact, then the whole 30-iteration ICP -- host
    loop (the default) and device loop -- against the oracle's transform and
    error history."""
    pairs = lidar()
    assert len(pairs) == 16
    p = pairs[k]
    say("lidar pair", k, len(p.target), len(p.source))
    otree, o = lidar_oracle(k)
    tree = kdnn.Tree(p.target, 16)
    src = dev(torch, p.source)
    oi, od, red = _pairs_oracle(p.target, p.source, np.eye(3), np.zeros(3), otree)
    res = tree.correspond_reduce(src, np.eye(3), np.zeros(3), return_pairs=True)
    assert_nn_equal(res["idx"], res["d2"], oi, od, f"lidar {k} pairs")
    check_sums(res, red, bbox_diag(p.target), f"lidar {k}")
    for kw in ({}, {"device_loop": True}):
        say("lidar icp_align pair", k, kw)
        g = tree.icp(src, max_iter=p.iters, **kw)
        assert g["iters"] == p.iters
        assert np.linalg.norm(g["R"] - o["R"]) <= R_TOL, (k, kw)
        assert np.max(np.abs(g["t"] - o["t"])) <= T_TOL, (k, kw)
        np.testing.assert_allclose(g["E"], o["E"], rtol=1e-6, err_msg=f"pair {k} {kw}")
    assert np.degrees(oracle.rot_err(o["R"], p.R_true)) < 0.5


def test_page_recipe_registration(torch, kdnn):
    """The article's own regression recipe (§6): 200k points uniform in
    [-25, 25]^3 m, moved by 10 degrees about a random axis and 0.5 m, with
    N(0, 0.01^2) noise, 30 iterations -- host and device loops against the
    oracle's registration, and the recovered motion against the truth (the
    §6 metrics, rotation and translation error)."""
    p = synth.recipe()
    say("recipe 200k: oracle")
    otree = oracle.KDTree(p.target, 16)
    o = oracle.icp(p.target, p.source, p.iters, tree=otree)
    tree = kdnn.Tree(p.target, 16)
    src = dev(torch, p.source)
    for kw in ({}, {"device_loop": True}):
        say("recipe 200k icp_align", kw)
        g = tree.icp(src, max_iter=p.iters, **kw)
        assert g["iters"] == p.iters
        assert np.linalg.norm(g["R"] - o["R"]) <= R_TOL, kw
        assert np.max(np.abs(g["t"] - o["t"])) <= T_TOL, kw
        np.testing.assert_allclose(g["E"], o["E"], rtol=1e-6)
    # §6's metrics: plain point-to-point ICP on this uniform cloud (0.85 m point
    # spacing, 10 degrees) is still approaching the truth after 30 iterations
    # (~5.2 degrees left); the error must shrink and E decrease
    assert np.degrees(oracle.rot_err(o["R"], p.R_true)) < 9.0
    assert oracle.trans_err(o["t"], p.t_true) < 0.5
    assert np.all(o["E"][1:] <= o["E"][:-1] * (1 + 1e-6))


# ------------------------------------------------ builder variants (leaf sweep)
@pytest.mark.parametrize("leaf", [1, 4, 32, 64])
@pytest.mark.parametrize("round_robin", [False, True], ids=["maxvar", "roundrobin"])
def test_scene_builder_variants(torch, kdnn, leaf, round_robin):
    """The tree's shape (leaf size, split-axis rule) never changes a result:
    same pairs as the oracle, and the same registration."""
    p = scene()
    otree, o = scene_oracle_icp()
    tree = kdnn.Tree(p.target, leaf, round_robin=round_robin)
    n = len(p.target)
    D = tree.info["depth"]
    assert 2 ** D * leaf >= n and (D == 0 or 2 ** (D - 1) * leaf < n)
    src = dev(torch, p.source)
    for k in (0, p.iters - 1):
        R = o["Rt_hist"][k, :9].reshape(3, 3)
        t = o["Rt_hist"][k, 9:]
        say("builder variant", leaf, round_robin, "iteration", k)
        oi, od, red = _pairs_oracle(p.target, p.source, R, t, otree)
        res = tree.correspond_reduce(src, R, t, return_pairs=True)
        assert_nn_equal(res["idx"], res["d2"], oi, od, f"leaf {leaf} rr {round_robin} it{k}")
        check_sums(res, red, bbox_diag(p.target), f"leaf {leaf} rr {round_robin} it{k}")
    g = tree.icp(src, max_iter=p.iters)
    assert np.linalg.norm(g["R"] - o["R"]) <= R_TOL
    assert np.max(np.abs(g["t"] - o["t"])) <= T_TOL


def test_fused_kernel_several_chunks_per_work_group(torch, kdnn):
    """More than 4096 x 256 source points: the fused kernel's work-groups each
    take several 256-point chunks in turn (its grid is capped at 4096)."""
    p = synth.stress()
    rng = np.random.Generator(np.random.PCG64(77))
    S = rng.uniform(-50, 50, size=(1_100_000, 3)).astype(np.float32)
    tree = kdnn.Tree(p.target, 8)
    R = synth.rotation_about(synth.random_unit(rng), 0.01)
    t = np.array([0.05, -0.02, 0.01])
    say("fused kernel, 1.1M source points")
    oi, od, red = _pairs_oracle(p.target, S, R, t, stress_oracle_tree())
    for f in (0, _lib_flags().KDNN_ICP_NO_SORT, _lib_flags().KDNN_ICP_SORT):
        res = tree.correspond_reduce(dev(torch, S), R, t, return_pairs=True, flags=f)
        assert_nn_equal(res["idx"], res["d2"], oi, od, f"1.1M pairs flags {f}")
        check_sums(res, red, bbox_diag(p.target), f"1.1M sums flags {f}")


def test_automatic_order_rule(torch, kdnn):
    """nn_query orders its queries by default only for trees (node records +
    points) above 4 L2s, the ICP entry points above one L2; Scene stays
    unordered, Skewed 500k (leaf 8) is ordered for ICP only, Stress 1M both."""
    for name, gen, leaf, want in (("scene", scene, 16, (0, 0)),
                                  ("skewed", synth.skewed, 8, (0, 1)),
                                  ("stress", synth.stress, 8, (1, 1))):
        say("automatic order rule", name)
        info = kdnn.Tree(gen().target, leaf).info
        fp = info["node_slots"] * 32 + info["n"] * 16
        l2 = info["l2_bytes"]
        assert (info["auto_sort"], info["auto_sort_icp"]) == (int(fp > 4 * l2), int(fp > l2))
        if l2 == 4 * 2**20:
            assert (info["auto_sort"], info["auto_sort_icp"]) == want, name


def test_kernel_timing(torch, kdnn):
    """The timing facility records one positive duration per correspondence
    launch, up to its cap, and leaves the results unchanged."""
    p = scene()
    tree = kdnn.Tree(p.target, 16)
    src = dev(torch, p.source)
    R, t = np.eye(3), np.zeros(3)
    say("kernel timing, scene")
    ref = tree.correspond_reduce(src, R, t, return_pairs=True)
    ref_idx, ref_d2 = ref["idx"].cpu().numpy(), ref["d2"].cpu().numpy()
    kdnn.timing_begin(3)
    for _ in range(5):
        res = tree.correspond_reduce(src, R, t, return_pairs=True)
    ms = kdnn.timing_end()
    assert len(ms) == 3 and np.all(ms > 0) and np.all(ms < 1e3)
    assert np.array_equal(res["idx"].cpu().numpy(), ref_idx)
    assert np.array_equal(res["d2"].cpu().numpy(), ref_d2)
    assert res["E"] == ref["E"]
    kdnn.timing_begin(2)
    tree.correspond_reduce(src, R, t)
    assert len(kdnn.timing_end()) == 1
    with pytest.raises(Exception, match="not started"):
        kdnn.timing_end()


def _lib_flags():
    from kd_tree_nn_amd import _lib
    return _lib


@functools.lru_cache(maxsize=None)
def stress_oracle_tree():
    return oracle.KDTree(synth.stress().target, 8)


@functools.lru_cache(maxsize=None)
def shapes_target():
    rng = np.random.Generator(np.random.PCG64(4242))
    T = rng.uniform(-10, 10, size=(50_000, 3)).astype(np.float32)
    return T, oracle.KDTree(T, 16)


# Source sizes that reach each launch shape of the one-lane-per-point kernels:
# a few points (fewer work-groups than CUs), one round with 1 to 5 groups per
# CU and a non-power-of-two number of points per wave, the full machine, and
# more than one round (64 points per wave, several sweeps).
SHAPE_SIZES = [1, 5, 31, 257, 4097, 33_793, 50_001, 131_065, 163_841, 300_001, 330_001]


@pytest.mark.parametrize("n", SHAPE_SIZES)
def test_fused_kernel_launch_shapes(torch, kdnn, n):
    T, otree = shapes_target()
    rng = np.random.Generator(np.random.PCG64(n))
    S = rng.uniform(-11, 11, size=(n, 3)).astype(np.float32)
    R = synth.rotation_about(synth.random_unit(rng), 0.02)
    t = np.array([0.1, -0.05, 0.02])
    say("fused kernel launch shape, n", n)
    oi, od, red = _pairs_oracle(T, S, R, t, otree)
    tree = kdnn.Tree(T, 16)
    src = dev(torch, S)
    for f in (0, _lib_flags().KDNN_ICP_NO_SORT, _lib_flags().KDNN_ICP_SORT):
        res = tree.correspond_reduce(src, R, t, return_pairs=True, flags=f)
        assert_nn_equal(res["idx"], res["d2"], oi, od, f"n={n} flags {f}")
        check_sums(res, red, bbox_diag(T), f"n={n} flags {f}")
    q = dev(torch, oracle.transform(S, R, t))
    for sort in (True, False):
        idx, d2 = tree.query(q, sort=sort)
        assert_nn_equal(idx, d2, oi, od, f"nn_query n={n} sort={sort}")
