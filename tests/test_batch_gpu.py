"""GPU parity of the batched registration (icp_align_batch; CUDA-KDTree ICP
article §3.4: consecutive frames in flight together): every pair of a batch
must give the single-pair result and the oracle's, to the ICP bar."""

import functools

import numpy as np
import pytest

import oracle
import synth
from tests.test_parity_gpu import (  # noqa: F401  (fixtures)
    R_TOL, T_TOL, dev, kdnn, lidar, lidar_oracle, say, scene, torch,
)

pytestmark = pytest.mark.gpu


def _single(kdnn, torch, tree, src, iters, **kw):
    """The single-pair registration with the batch's own loop (device) and order."""
    kw.setdefault("device_loop", True)
    return tree.icp(dev(torch, src), max_iter=iters, sort=False, **kw)


@functools.lru_cache(maxsize=None)
def _lidar_batch(kdnn):
    """All 16 LiDAR pairs in one batched call (device loop, the default) and in
    one with a host solve per iteration; each pair's single-pair registration."""
    import torch as T
    pairs = lidar()
    trees = [kdnn.Tree(p.target, 16) for p in pairs]
    srcs = [T.from_numpy(np.ascontiguousarray(p.source, np.float32)).cuda() for p in pairs]
    say("lidar batch of 16 (device loop)")
    res = kdnn.icp_batch(trees, srcs, max_iter=30)
    say("lidar batch of 16 (host loop)")
    resh = kdnn.icp_batch(trees, srcs, max_iter=30, device_loop=False)
    single = [tr.icp(x, max_iter=30, sort=False, device_loop=True) for tr, x in zip(trees, srcs)]
    return res, resh, single


def _close_to_single(b, s, what):
    assert b["iters"] == s["iters"], what
    np.testing.assert_allclose(b["E"], s["E"], rtol=1e-9, err_msg=what)
    assert np.linalg.norm(b["R"] - s["R"]) <= 1e-9, what
    assert np.max(np.abs(b["t"] - s["t"])) <= 1e-9, what


@pytest.mark.parametrize("k", range(16))
def test_lidar_16_pairs_batch(torch, kdnn, k):
    """Pair k of the 16-pair batch, with the iterations on the device and with
    a host solve per iteration: the oracle's transform and error history, and
    the single-pair registration's iterates."""
    res, resh, single = _lidar_batch(kdnn)
    _, o = lidar_oracle(k)
    say("lidar batch pair", k)
    for name, b in (("device loop", res[k]), ("host loop", resh[k])):
        assert b["status"] == 0 and b["iters"] == 30, name
        assert np.linalg.norm(b["R"] - o["R"]) <= R_TOL, (k, name)
        assert np.max(np.abs(b["t"] - o["t"])) <= T_TOL, (k, name)
        np.testing.assert_allclose(b["E"], o["E"], rtol=1e-6, err_msg=f"pair {k} {name}")
    _close_to_single(res[k], single[k], f"lidar pair {k}")


def test_mixed_sizes_and_chunks(torch, kdnn):
    """B = 3 pairs of different sizes (XCD groups of 3/3/2), then B = 9 (a launch
    of 8 and a launch of 1), with initial transforms and early stopping."""
    tiny = synth.tiny()
    sc = scene()
    pairs = [(tiny.target, tiny.source, 8, 20), (sc.target, sc.source, 16, 30),
             (lidar()[2].target, lidar()[2].source, 16, 30)]
    trees = [kdnn.Tree(T, leaf) for T, _, leaf, _ in pairs]
    say("batch of 3 mixed sizes")
    res = kdnn.icp_batch(trees, [dev(torch, S) for _, S, _, _ in pairs], max_iter=30)
    for k, ((T, S, leaf, _), tr, b) in enumerate(zip(pairs, trees, res)):
        _close_to_single(b, _single(kdnn, torch, tr, S, 30), f"mixed pair {k}")

    rng = np.random.Generator(np.random.PCG64(9))
    R0 = np.stack([synth.rotation_about(synth.random_unit(rng), 0.01 * k) for k in range(9)])
    t0 = rng.normal(size=(9, 3)) * 0.01
    lp = lidar()[:9]
    trees9 = [kdnn.Tree(p.target, 16) for p in lp]
    say("batch of 9 with R0, t0, eps")
    res = kdnn.icp_batch(trees9, [dev(torch, p.source) for p in lp], R0=R0, t0=t0,
                         max_iter=40, eps=1e-5)
    for k, (p, tr, b) in enumerate(zip(lp, trees9, res)):
        s = tr.icp(dev(torch, p.source), R0=R0[k], t0=t0[k], max_iter=40, eps=1e-5, sort=False,
                   device_loop=True)
        _close_to_single(b, s, f"pair {k} of 9")


def test_batch_max_dist(torch, kdnn):
    lp = lidar()[4:7]
    trees = [kdnn.Tree(p.target, 16) for p in lp]
    say("batch max_dist")
    res = kdnn.icp_batch(trees, [dev(torch, p.source) for p in lp], max_iter=30, max_dist=1.0)
    for k, (p, tr, b) in enumerate(zip(lp, trees, res)):
        s = _single(kdnn, torch, tr, p.source, 30, max_dist=1.0)
        _close_to_single(b, s, f"max_dist pair {k}")
    for k, p in enumerate(lp):
        o = oracle.icp(p.target, p.source, 30, leaf_size=16, max_dist=1.0)
        assert np.linalg.norm(res[k]["R"] - o["R"]) <= R_TOL, k
        assert np.max(np.abs(res[k]["t"] - o["t"])) <= T_TOL, k


def test_batch_degenerate_pair_and_errors(torch, kdnn):
    tiny = synth.tiny()
    far = (tiny.source + np.float32(100.0)).astype(np.float32)
    trees = [kdnn.Tree(tiny.target, 8), kdnn.Tree(tiny.target, 8)]
    say("batch degenerate pair")
    res = kdnn.icp_batch(trees, [dev(torch, tiny.source), dev(torch, far)], max_iter=5,
                         max_dist=0.5)
    assert res[0]["status"] == 0 and res[0]["iters"] == 5
    assert res[1]["status"] == 5 and res[1]["iters"] == 0           # EDEGENERATE
    np.testing.assert_array_equal(res[1]["R"], np.eye(3))
    s = trees[0].icp(dev(torch, tiny.source), max_iter=5, max_dist=0.5, sort=False,
                     device_loop=True)
    _close_to_single(res[0], s, "healthy pair next to a degenerate one")
    from kd_tree_nn_amd import _lib
    import ctypes
    n = np.array([len(tiny.source)], np.int64)
    ws = kdnn.icp_batch_workspace(n)
    R = np.zeros(9)
    t = np.zeros(3)
    th = (ctypes.c_void_p * 1)(trees[0]._h.value)
    sp = (ctypes.c_void_p * 1)(dev(torch, tiny.source).data_ptr())
    L = _lib.lib()
    args = lambda flags, rej, wsz: L.icp_align_batch(  # noqa: E731
        1, th, sp, n.ctypes.data_as(ctypes.POINTER(_lib.c_i64)), None, None, 3, 0.0,
        R.ctypes.data_as(_lib.c_dp), t.ctypes.data_as(_lib.c_dp), None, None, None, flags,
        rej, ws.data_ptr(), wsz, None)
    assert args(_lib.lanes_flag(4), None, ws.numel()) == _lib.KDNN_EINVAL  # a schedule flag
    assert args(0, None, ws.numel() - 256) == _lib.KDNN_EINVAL              # no room for the loop
    assert args(0, ctypes.byref(_lib.IcpReject(1.0, 3.0)), ws.numel()) == _lib.KDNN_EINVAL
    assert args(0, None, 16) == _lib.KDNN_EINVAL                           # workspace too small
    assert args(0, None, ws.numel()) == _lib.KDNN_OK


def test_batch_leaf8_trees(torch, kdnn):
    """Trees whose leaves hold at most 8 points take the batched kernel's 8-point
    leaf batches and depth-sized LDS; each pair must match its single-pair ICP."""
    lp = lidar()[:3]
    trees = [kdnn.Tree(p.target, 8) for p in lp]
    assert all(tr.info["max_leaf"] <= 8 for tr in trees)
    say("batch of 3 LiDAR pairs, leaf 8")
    res = kdnn.icp_batch(trees, [dev(torch, p.source) for p in lp], max_iter=10)
    for k, (p, tr, b) in enumerate(zip(lp, trees, res)):
        _close_to_single(b, _single(kdnn, torch, tr, p.source, 10), f"leaf-8 pair {k}")


def test_batch_device_loop_matches_host_loop(torch, kdnn):
    """The batched call keeps its iterations on the device (per pair: reduction,
    solve and loop state in one group) unless asked to solve on the host; same
    kernels, same sums, same solve code: the same iterates."""
    lp = lidar()[:5]
    tiny = synth.tiny()
    trees = [kdnn.Tree(p.target, 16) for p in lp] + [kdnn.Tree(tiny.target, 8)]
    srcs = [dev(torch, p.source) for p in lp] + [dev(torch, tiny.source)]
    for kw in ({"max_iter": 30}, {"max_iter": 40, "eps": 1e-6}, {"max_iter": 12, "max_dist": 1.0}):
        say("batch device vs host loop", kw)
        d = kdnn.icp_batch(trees, srcs, **kw)
        h = kdnn.icp_batch(trees, srcs, device_loop=False, **kw)
        for k, (a, b) in enumerate(zip(d, h)):
            # device: Horn's quaternion solve; host: the SVD route (agree to ~1e-15)
            assert a["status"] == b["status"] == 0 and a["iters"] == b["iters"], (kw, k)
            np.testing.assert_allclose(a["E"], b["E"], rtol=1e-9, err_msg=f"{kw} pair {k}")
            assert np.linalg.norm(a["R"] - b["R"]) <= 1e-9, (kw, k)
            assert np.max(np.abs(a["t"] - b["t"])) <= 1e-9, (kw, k)
