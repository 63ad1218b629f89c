"""Replay ceiling of a search launch (kdnn_replay_bench) through the C ABI.

The replay must load exactly the records the instrumented single-lane search
visits: its tallies of node records and leaf points equal the sums of
nn_query_stats' per-query counts, its byte count follows from them, rows
longer than KDNN_REPLAY_CAP are reported as truncated, and bad arguments are
rejected on the host before any launch.  Every case prints its name before
touching the device.
"""

import ctypes
import sys

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

# point location reads the split planes of the top 8 levels from a work-group
# copy in LDS: they are no memory records
TOP_LOC_LEVELS = 8


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
    _lib.lib()
    return kd_tree_nn_amd


def dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def _uniform(seed, n, m):
    rng = np.random.Generator(np.random.PCG64(seed))
    tgt = rng.uniform(-10.0, 10.0, (n, 3)).astype(np.float32)
    q = rng.uniform(-11.0, 11.0, (m, 3)).astype(np.float32)
    return tgt, q


def _case(name):
    if name == "tiny_leaf8":
        p = synth.tiny()
        return p.target, p.source, 8
    if name == "uniform_ragged_leaf16":
        tgt, q = _uniform(7, 20_003, 12_345)
        q[17] = np.nan  # a query that visits nothing
        return tgt, q, 16
    if name == "scene_leaf16":
        p = synth.scene()
        return p.target, p.source, 16
    if name == "uniform_leaf1_deep":  # depth 15: one level above the plane record
        tgt, q = _uniform(9, 20_000, 4_000)
        return tgt, q, 1
    raise KeyError(name)


@pytest.mark.parametrize("name,icp,sort", [
    ("tiny_leaf8", False, None), ("tiny_leaf8", True, True),
    ("uniform_ragged_leaf16", False, False), ("uniform_ragged_leaf16", False, True),
    ("uniform_ragged_leaf16", True, None),
    ("scene_leaf16", True, False), ("scene_leaf16", True, True), ("scene_leaf16", False, None),
    ("uniform_leaf1_deep", False, None), ("uniform_leaf1_deep", True, None),
])
def test_replay_tallies_match_instrumented_counts(torch, kdnn, name, icp, sort):
    tgt, q, leaf = _case(name)
    say("replay tallies", name, "icp" if icp else "nn", "sort", sort, "queries", len(q))
    tree = kdnn.Tree(tgt, leaf)
    qd = dev(torch, q)
    _, _, cn, cp = tree.query_stats(qd)
    cn = cn.cpu().numpy().astype(np.int64)
    cp = cp.cpu().numpy().astype(np.int64)
    ms, info = tree.replay_bench(qd, icp=icp, sort=sort, reps=3)
    assert ms.shape == (3,) and np.all(np.isfinite(ms)) and np.all(ms > 0.0)
    assert info["truncated"] == 0
    assert info["node_records"] == int(cn.sum())
    assert info["leaf_points"] == int(cp.sum())
    assert 1 <= info["queries_per_wave"] <= 64 and info["blocks"] >= 1
    # visits of each searched query: the split planes of its point location
    # below the top TOP_LOC_LEVELS levels (8 B, one record each; the top ones
    # come from LDS), its leaf's plane record (64 B, two records), the sibling
    # boxes above the record's 14 levels (32 B, one record each), one box run
    # per internal node entered (48 B, two records), one per leaf scanned
    # (whole chunks)
    finite = int(np.isfinite(q).all(axis=1).sum())
    D = tree.info["depth"]
    loc = D - min(D, TOP_LOC_LEVELS)
    top = max(0, D - 14)
    pairs2 = int(cn.sum()) - finite * (loc + 2 + top)
    assert pairs2 >= 0 and pairs2 % 2 == 0
    pairs = pairs2 // 2
    leaves = info["visits"] - finite * (loc + 1 + top) - pairs
    assert leaves >= finite  # every searched query scans at least one leaf
    chunk = 8 if tree.info["max_leaf"] <= 8 else 16
    assert info["bytes"] == finite * (8 * loc + 64 + 32 * top) + 48 * pairs + 16 * chunk * leaves


def test_replay_truncates_long_rows(torch, kdnn):
    # points on a sphere and one query at its centre: every leaf box is within
    # the best distance, so that query visits far more than KDNN_REPLAY_CAP
    rng = np.random.Generator(np.random.PCG64(11))
    v = rng.normal(size=(20_000, 3))
    sph = (v / np.linalg.norm(v, axis=1, keepdims=True)).astype(np.float32)
    q = np.concatenate([np.zeros((1, 3), np.float32), sph[:999] * 1.01]).astype(np.float32)
    say("replay truncation, sphere of 20000, centre query")
    tree = kdnn.Tree(sph, 8)
    qd = dev(torch, q)
    _, _, cn, cp = tree.query_stats(qd)
    cn = cn.cpu().numpy().astype(np.int64)
    assert cn[0] > 2 * 512  # the centre query's row overflows
    ms, info = tree.replay_bench(qd, reps=2)
    assert info["truncated"] == 1
    assert info["node_records"] < int(cn.sum())
    assert np.all(ms > 0.0)


def test_replay_argument_checks(torch, kdnn):
    from kd_tree_nn_amd import _lib
    L = _lib.lib()
    tgt, q = _uniform(3, 2000, 500)
    tree = kdnn.Tree(tgt, 8)
    qd = dev(torch, q)
    need = int(L.kdnn_replay_workspace_bytes(tree._h, 500, 0))
    assert need > 0
    assert L.kdnn_replay_workspace_bytes(None, 500, 0) == 0
    assert L.kdnn_replay_workspace_bytes(tree._h, 0, 0) == 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ms = (ctypes.c_float * 4)()
    info = _lib.ReplayInfo()
    say("replay argument checks")
    bad = [
        (500, 0, 0, need),                                    # reps < 1
        (500, 1 << 7, 4, need),                               # unknown flag
        (500, _lib.KDNN_QUERY_SORT | _lib.KDNN_QUERY_NO_SORT, 4, need),
        (500, 0, 4, need - 256),                              # small workspace
        (0, 0, 4, need),                                      # no queries
    ]
    for m, flags, reps, nbytes in bad:
        st = L.kdnn_replay_bench(tree._h, qd.data_ptr(), None, m, flags, reps, ws.data_ptr(),
                                 nbytes, ms, ctypes.byref(info), None)
        assert st == _lib.KDNN_EINVAL, (m, flags, reps, nbytes)
    st = L.kdnn_replay_bench(tree._h, qd.data_ptr(), None, 500, 0, 4, ws.data_ptr(), need, None,
                             ctypes.byref(info), None)
    assert st == _lib.KDNN_EINVAL
    st = L.kdnn_replay_bench(tree._h, qd.data_ptr(), qd.data_ptr() + 2, 500, 0, 4,
                             ws.data_ptr(), need, ms, ctypes.byref(info), None)
    assert st == _lib.KDNN_EINVAL  # misaligned previous queries
    # and good calls on the same buffers, cold and warm
    st = L.kdnn_replay_bench(tree._h, qd.data_ptr(), None, 500, 0, 4, ws.data_ptr(), need, ms,
                             ctypes.byref(info), None)
    assert st == _lib.KDNN_OK and info.visits > 0
    st = L.kdnn_replay_bench(tree._h, qd.data_ptr(), qd.data_ptr(), 500, 0, 4, ws.data_ptr(),
                             need, ms, ctypes.byref(info), None)
    assert st == _lib.KDNN_OK and info.visits > 0


@pytest.mark.parametrize("name", ["tiny_leaf8", "uniform_ragged_leaf16", "scene_leaf16"])
def test_replay_warm_start_tallies(torch, kdnn, name):
    """Warm-started replay (the previous iteration's queries given): every
    searched query records its start leaf's 64-byte plane record (two node
    records), the sibling boxes above the record's 14 levels (none in these
    trees) and at least one leaf -- its start leaf, with the queries
    themselves as the previous iteration their own answer's leaf; bytes
    follow from the tallies.  (A plane bounds its sibling more loosely than
    the sibling's box, so a warm search may scan a leaf the search from the
    root skips: no comparison of point counts holds in general.)"""
    tgt, q, leaf = _case(name)
    say("replay warm start", name, "queries", len(q))
    tree = kdnn.Tree(tgt, leaf)
    qd = dev(torch, q)
    ms, info = tree.replay_bench(qd, icp=True, reps=2, prev=qd)
    assert np.all(ms > 0.0) and info["truncated"] == 0
    D = tree.info["depth"]
    assert D <= 14
    finite = int(np.isfinite(q).all(axis=1).sum())
    pairs2 = info["node_records"] - 2 * finite
    assert pairs2 >= 0 and pairs2 % 2 == 0
    pairs = pairs2 // 2
    leaves = info["visits"] - finite - pairs
    assert leaves >= finite
    chunk = 8 if tree.info["max_leaf"] <= 8 else 16
    assert info["bytes"] == 64 * finite + 48 * pairs + 16 * chunk * leaves
    assert info["leaf_points"] >= finite * tree.info["min_leaf"]


def test_replay_warm_start_deep_tree(torch, kdnn):
    """A tree deeper than the plane record (leaf size 1, 2^15 leaves): every
    warm search also loads the D - 14 sibling boxes nearest the root, one
    node record and 32 bytes each."""
    tgt, q = _uniform(5, 20_000, 3_000)
    say("replay warm start, deep tree, 20000 points leaf 1, 3000 queries")
    tree = kdnn.Tree(tgt, 1)
    D = tree.info["depth"]
    assert D > 14
    qd = dev(torch, q)
    ms, info = tree.replay_bench(qd, icp=True, reps=2, prev=qd)
    assert np.all(ms > 0.0) and info["truncated"] == 0
    m = len(q)
    top = D - 14
    pairs2 = info["node_records"] - (2 + top) * m
    assert pairs2 >= 0 and pairs2 % 2 == 0
    pairs = pairs2 // 2
    leaves = info["visits"] - (1 + top) * m - pairs
    assert leaves >= m
    assert info["bytes"] == (64 + 32 * top) * m + 48 * pairs + 16 * 8 * leaves
