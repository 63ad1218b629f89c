"""CPU tests of libkdnn.so: exported symbols, host builder invariants, host
rigid solve, argument checking.  No device work is launched here."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def kdnn():
    from kd_tree_nn_amd import _lib
    if not os.path.exists(_lib.LIBPATH):
        from kd_tree_nn_amd import build
        build.build()
    import kd_tree_nn_amd
    return kd_tree_nn_amd


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "kdnn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_symbols_exported(kdnn):
    from kd_tree_nn_amd import _lib
    names = _declared_functions()
    assert len(names) >= 15, names
    L = ctypes.CDLL(_lib.LIBPATH)
    for n in names:
        assert hasattr(L, n), f"{n} declared in kdnn.h but not exported"
    assert set(names) == set(_lib.SIGNATURES), set(names) ^ set(_lib.SIGNATURES)
    assert kdnn.version() == 5


@pytest.mark.parametrize("n,leaf,D", [(1, 16, 0), (16, 16, 0), (17, 16, 1), (1024, 8, 7),
                                      (100_000, 16, 13), (1_000_000, 8, 17),
                                      (1_000_000, 16, 16), (500_000, 8, 16), (500_000, 16, 15),
                                      (131_072, 16, 13), (3, 1, 2)])
def test_layout_depth(kdnn, n, leaf, D):
    d, slots = kdnn.layout(n, leaf)
    assert d == D and slots == 2 ** (D + 1)
    # the definition: smallest d with ceil(n / 2^d) <= leaf
    assert -(-n // 2 ** d) <= leaf and (d == 0 or -(-n // 2 ** (d - 1)) > leaf)


def _check_tree(pts, bt, leaf, max_depth=0, round_robin=False):
    n = len(pts)
    D = bt["depth"]
    nodes, P = bt["nodes"], bt["points"]
    L0 = 2 ** D
    assert nodes.shape == (2 * L0, 8)
    # every original point exactly once, coordinates carried unchanged
    orig = P[:, 3].view(np.int32)
    assert np.array_equal(np.sort(orig), np.arange(n))
    np.testing.assert_array_equal(P[:, :3], pts[orig])
    # leaves: contiguous runs, balanced sizes, in order
    begin = nodes[L0:, 6].view(np.int32)
    count = nodes[L0:, 7].view(np.int32)
    assert begin[0] == 0 and np.all(begin[1:] == begin[:-1] + count[:-1]) and count.sum() == n
    # leaf j owns slots [floor(j n / 2^D), floor((j + 1) n / 2^D))
    np.testing.assert_array_equal(begin, (np.arange(L0, dtype=np.int64) * n) >> D)
    assert set(np.unique(count)) <= {n // L0, -(-n // L0)}
    if max_depth == 0:
        assert count.max() <= leaf
    # 2 * leaves - 1 real nodes (slot 0 unused), parent i before children 2i, 2i+1
    assert (len(nodes) - 1) == 2 * L0 - 1

    def box_of(i):
        d = int(np.floor(np.log2(i)))
        first = i << (D - d)
        last = ((i + 1) << (D - d)) - 1
        a = begin[first - L0]
        e = begin[last - L0] + count[last - L0]
        return a, e

    for i in range(1, 2 * L0):
        a, e = box_of(i)
        lo, hi = nodes[i, :3], nodes[i, 3:6]
        if e > a:
            np.testing.assert_array_equal(lo, P[a:e, :3].min(0))
            np.testing.assert_array_equal(hi, P[a:e, :3].max(0))
        else:
            assert np.all(np.isinf(lo)) and np.all(lo > 0) and np.all(hi < 0)
        if i < L0:
            axis = int(nodes[i, 7].view(np.uint32))
            split = nodes[i, 6]
            la, le = box_of(2 * i)
            ra, re_ = box_of(2 * i + 1)
            assert le == ra and (le - la) in ((e - a) // 2, (e - a + 1) // 2)
            assert np.all(P[la:le, axis] <= split) and np.all(P[ra:re_, axis] >= split)
            if re_ > ra:
                assert split in P[ra:re_, axis]
            else:
                assert split == np.inf
            if e > a:
                d = int(np.floor(np.log2(i)))
                if round_robin:
                    assert axis == d % 3
                elif e - a >= 2:
                    v = P[a:e, :3].astype(np.float64).var(0)
                    assert v[axis] == v.max() or np.isclose(v[axis], v.max(), rtol=1e-12)


@pytest.mark.parametrize("leaf", [1, 2, 8, 16])
def test_builder_invariants_small(kdnn, leaf):
    for name, T, _ in __import__("tests._cases", fromlist=["x"]).adversarial_clouds():
        if len(T) > 600:
            continue
        bt = kdnn.build_host(T, leaf)
        _check_tree(T, bt, leaf)


def test_builder_invariants_tiny_and_round_robin(kdnn):
    p = synth.tiny()
    _check_tree(p.target, kdnn.build_host(p.target, 8), 8)
    _check_tree(p.target, kdnn.build_host(p.target, 8, round_robin=True), 8, round_robin=True)


def test_builder_max_depth_cap(kdnn):
    rng = np.random.Generator(np.random.PCG64(4))
    T = rng.random((5000, 3)).astype(np.float32)
    bt = kdnn.build_host(T, 8, max_depth=5)
    assert bt["depth"] == 5
    _check_tree(T, bt, 8, max_depth=5)
    cnt = bt["nodes"][32:, 7].view(np.int32)
    assert cnt.max() > 8


def test_builder_scene_depth_and_sizes(kdnn):
    p = synth.scene()
    bt = kdnn.build_host(p.target, 16)
    assert bt["depth"] == 13
    cnt = bt["nodes"][2 ** 13:, 7].view(np.int32)
    assert cnt.min() == 12 and cnt.max() == 13


def test_builder_deterministic(kdnn):
    p = synth.tiny()
    a = kdnn.build_host(p.target, 8)
    b = kdnn.build_host(p.target, 8)
    np.testing.assert_array_equal(a["nodes"].view(np.uint32), b["nodes"].view(np.uint32))
    np.testing.assert_array_equal(a["points"].view(np.uint32), b["points"].view(np.uint32))


def test_builder_errors(kdnn):
    from kd_tree_nn_amd import KdnnError
    with pytest.raises(KdnnError, match="EINVAL"):
        kdnn.build_host(np.zeros((0, 3), np.float32))
    with pytest.raises(KdnnError, match="EINVAL"):
        kdnn.build_host(np.zeros((10, 3), np.float32), leaf_size=2000)
    with pytest.raises(KdnnError, match="EINVAL"):
        kdnn.layout(10, 16, max_depth=40)
    bad = np.zeros((10, 3), np.float32)
    bad[7, 1] = np.nan
    with pytest.raises(KdnnError, match="ENONFINITE"):
        kdnn.build_host(bad)
    bad[7, 1] = np.inf
    with pytest.raises(KdnnError, match="ENONFINITE"):
        kdnn.build_host(bad)
    # leaf_size 0 means the default 16
    assert kdnn.layout(100, 0)[0] == kdnn.layout(100, 16)[0]


# ------------------------------------------------------------- host solve
def _sums_from_pairs(s, m, d2, c):
    s = np.asarray(s, np.float64) - c
    m = np.asarray(m, np.float64) - c
    return {"n": len(s), "c": np.asarray(c, np.float64), "sum_s": s.sum(0), "sum_m": m.sum(0),
            "sum_sm": s.T @ m, "E": float(np.sum(d2))}


@pytest.mark.parametrize("seed", range(6))
def test_procrustes_matches_oracle_horn(kdnn, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    s = rng.normal(size=(500, 3)) * [4, 2, 0.5] + [30, -20, 1]
    R0 = synth.rotation_about(synth.random_unit(rng), rng.uniform(0.05, 3.0))
    m = s @ R0.T + rng.normal(size=3) * 3 + rng.normal(scale=0.05, size=s.shape)
    R, t = kdnn.procrustes(_sums_from_pairs(s, m, np.zeros(500), [29.0, -21.0, 0.5]))
    red = oracle.reduce_pairs(s, m, np.zeros(500))
    Ro = oracle.horn(red["H"])
    to = red["mu_m"] - Ro @ red["mu_s"]
    np.testing.assert_allclose(R, Ro, atol=1e-10)
    np.testing.assert_allclose(t, to, atol=1e-9)
    assert abs(np.linalg.det(R) - 1) < 1e-12


def test_procrustes_exact_recovery(kdnn):
    rng = np.random.Generator(np.random.PCG64(77))
    R0 = synth.rotation_about([0.3, -1, 2], 2.2)
    t0 = np.array([1.5, -0.25, 10.0])
    s = rng.normal(size=(100, 3))
    R, t = kdnn.procrustes(_sums_from_pairs(s, s @ R0.T + t0, np.zeros(100), [0, 0, 0]))
    np.testing.assert_allclose(R, R0, atol=1e-12)
    np.testing.assert_allclose(t, t0, atol=1e-12)


def test_procrustes_planar_reflection(kdnn):
    rng = np.random.Generator(np.random.PCG64(11))
    s = np.concatenate([rng.normal(size=(100, 2)) * [3, 1], np.zeros((100, 1))], 1)
    m = s * [1, 1, -1] + rng.normal(scale=1e-3, size=s.shape) * [0, 0, 1]
    R, _ = kdnn.procrustes(_sums_from_pairs(s, m, np.zeros(100), [0, 0, 0]))
    assert abs(np.linalg.det(R) - 1) < 1e-12
    np.testing.assert_allclose(R, oracle.horn(oracle.reduce_pairs(s, m, np.zeros(100))["H"]), atol=1e-8)
    # exactly planar pairs (rank-2 H): still a proper rotation, equal to the oracle's
    m2 = s @ synth.rot_z(0.4).T
    R2, _ = kdnn.procrustes(_sums_from_pairs(s, m2, np.zeros(100), [0, 0, 0]))
    np.testing.assert_allclose(R2, synth.rot_z(0.4), atol=1e-12)


@pytest.mark.parametrize("scale", [1e-6, 1.0, 1e5])
def test_procrustes_random_rotations_vs_svd(kdnn, scale):
    """The quaternion solve (Newton on the characteristic polynomial, adjugate
    column) against the SVD route with the reflection fix, over rotations of
    every angle up to a half turn, anisotropic clouds and three length scales."""
    rng = np.random.Generator(np.random.PCG64(2024))
    for k in range(60):
        ang = np.pi if k % 10 == 0 else rng.uniform(0.0, np.pi)
        R0 = synth.rotation_about(synth.random_unit(rng), ang)
        s = rng.normal(size=(200, 3)) * rng.uniform(0.2, 5.0, size=3) * scale
        m = s @ R0.T + rng.normal(size=3) * scale + rng.normal(scale=0.01 * scale, size=s.shape)
        R, t = kdnn.procrustes(_sums_from_pairs(s, m, np.zeros(200), [0, 0, 0]))
        red = oracle.reduce_pairs(s, m, np.zeros(200))
        Rs = oracle.kabsch_svd(red["H"])
        np.testing.assert_allclose(R, Rs, atol=1e-9, err_msg=f"case {k}, angle {ang:.3f}")
        np.testing.assert_allclose(t, red["mu_m"] - Rs @ red["mu_s"], atol=1e-8 * scale)
        assert abs(np.linalg.det(R) - 1) < 1e-12


def test_procrustes_half_turn_exact(kdnn):
    """Half turns about the axes and a diagonal: the quaternion's scalar part is
    zero, so its eigenvector column must come from another adjugate column."""
    s = np.random.Generator(np.random.PCG64(5)).normal(size=(50, 3)) * [3, 2, 1]
    for axis in ([1, 0, 0], [0, 1, 0], [0, 0, 1], [1, 1, 1]):
        R0 = synth.rotation_about(axis, np.pi)
        R, t = kdnn.procrustes(_sums_from_pairs(s, s @ R0.T, np.zeros(50), [0, 0, 0]))
        np.testing.assert_allclose(R, R0, atol=1e-12)
        np.testing.assert_allclose(t, 0.0, atol=1e-12)


def test_procrustes_close_top_eigenvalues(kdnn):
    """sigma2 ~ sigma3 with det H < 0 makes the two largest eigenvalues of
    Horn's matrix close (gap 2 (sigma2 - sigma3)): the solve must still match
    the SVD route; with the gap zero the best rotation is not unique and any
    returned one must reach the same minimum."""
    e = np.eye(3)

    def cost(R, s, m):
        red = oracle.reduce_pairs(s, m, np.zeros(len(s)))
        d = (s - red["mu_s"]) @ R.T - (m - red["mu_m"])
        return float(np.sum(d * d))

    rng = np.random.Generator(np.random.PCG64(31))
    for gap in (1e-2, 1e-5, 1e-7, 1e-9, 0.0):
        s0 = np.concatenate([e * [3.0, 1.0 + gap, 1.0], -e * [3.0, 1.0 + gap, 1.0]])
        # a reflection, H = diag(18, 2 (1 + gap)^2, -2), seen in rotated frames
        A = synth.rotation_about(synth.random_unit(rng), rng.uniform(0, np.pi))
        B = synth.rotation_about(synth.random_unit(rng), rng.uniform(0, np.pi))
        s, m = s0 @ A.T, (s0 * [1.0, 1.0, -1.0]) @ B.T
        R, _ = kdnn.procrustes(_sums_from_pairs(s, m, np.zeros(len(s)), [0, 0, 0]))
        Rs = oracle.kabsch_svd(oracle.reduce_pairs(s, m, np.zeros(len(s)))["H"])
        assert abs(np.linalg.det(R) - 1) < 1e-12 and np.allclose(R @ R.T, np.eye(3), atol=1e-12)
        assert cost(R, s, m) <= cost(Rs, s, m) * (1 + 1e-12) + 1e-12, gap
        if gap > 0:
            # the rotation's own sensitivity to rounding in H is about 1e-16 / gap
            np.testing.assert_allclose(R, Rs, atol=max(1e-12, 1e-14 / gap), err_msg=f"gap {gap}")


def test_procrustes_degenerate(kdnn):
    from kd_tree_nn_amd import KdnnError
    s = np.tile([[1.0, 2.0, 3.0]], (10, 1))
    with pytest.raises(KdnnError, match="EDEGENERATE"):
        kdnn.procrustes(_sums_from_pairs(s, s, np.zeros(10), [0, 0, 0]))
    line = np.outer(np.arange(10.0), [1, 2, 3])
    with pytest.raises(KdnnError, match="EDEGENERATE"):
        kdnn.procrustes(_sums_from_pairs(line, line + 1, np.zeros(10), [0, 0, 0]))
    with pytest.raises(KdnnError, match="EDEGENERATE"):
        kdnn.procrustes(_sums_from_pairs(np.eye(3)[:2], np.eye(3)[:2], np.zeros(2), [0, 0, 0]))


def test_kdtree_build_rejects_before_device(kdnn):
    """Argument errors are reported without touching the device."""
    from kd_tree_nn_amd import _lib
    h = ctypes.c_void_p()
    p = _lib.BuildParams(16, 0, 0)
    st = _lib.lib().kdtree_build(None, 10, ctypes.byref(p), ctypes.byref(h))
    assert st == _lib.KDNN_EINVAL and b"null" in _lib.lib().kdnn_last_error()
    bad = np.full((4, 3), np.nan, np.float32)
    st = _lib.lib().kdtree_build(bad.ctypes.data, 4, ctypes.byref(p), ctypes.byref(h))
    assert st == _lib.KDNN_ENONFINITE
    assert _lib.lib().nn_query_workspace_bytes(0) == 0
    assert _lib.lib().icp_workspace_bytes(100_000) > 100_000 * 12


def test_timing_argument_errors(kdnn):
    """kdnn_timing_begin / _end reject bad arguments before any event exists."""
    from kd_tree_nn_amd import _lib
    from kd_tree_nn_amd._lib import KdnnError
    L = _lib.lib()
    assert L.kdnn_timing_begin(0) == _lib.KDNN_EINVAL
    assert L.kdnn_timing_begin(kdnn.KDNN_TIMING_MAX + 1) == _lib.KDNN_EINVAL
    assert b"cap" in L.kdnn_last_error()
    with pytest.raises(KdnnError, match="not started"):
        kdnn.timing_end()


@pytest.mark.parametrize("seed", range(4))
def test_moments_match_oracle_reduction(kdnn, seed):
    """kdnn_moments: centroids and H from the shifted sums equal the oracle's
    two-pass reduction of the same pairs (§2.1), whatever the shift c."""
    rng = np.random.Generator(np.random.PCG64(300 + seed))
    n = int(rng.integers(3, 5000))
    s = (rng.normal(size=(n, 3)) * [20, 5, 1] + [40, -10, 3]).astype(np.float32)
    m = (s @ synth.rot_z(0.2).T + [1.0, 2.0, 0.5] + rng.normal(scale=0.1, size=s.shape)).astype(np.float32)
    d2 = rng.random(n).astype(np.float32)
    c = rng.normal(size=3) * 30
    got = kdnn.sums_to_dict(_ctypes_sums(_sums_from_pairs(s, m, d2.astype(np.float64), c)))
    red = oracle.reduce_pairs(s, m, d2)
    assert got["n"] == red["n"] == n
    np.testing.assert_allclose(got["mu_s"], red["mu_s"], rtol=1e-12, atol=1e-9)
    np.testing.assert_allclose(got["mu_m"], red["mu_m"], rtol=1e-12, atol=1e-9)
    assert np.linalg.norm(got["H"] - red["H"]) <= 1e-10 * np.linalg.norm(red["H"])
    assert got["E"] == pytest.approx(red["E"], rel=1e-12)
    assert got["mse"] == pytest.approx(red["E"] / n, rel=1e-12)


def test_moments_hand_example_and_empty(kdnn):
    """Unit tetrahedron corners matched to 2 s (H worked by hand: diagonal 3/2,
    off-diagonal -1/2), with the sums shifted by c = (1, -1, 2); n = 0 gives
    zero centroids and H."""
    s = np.array([[0, 0, 0], [1, 0, 0], [0, 1, 0], [0, 0, 1]], np.float64)
    got = kdnn.sums_to_dict(_ctypes_sums(_sums_from_pairs(s, 2 * s, [0, 1, 1, 1], [1.0, -1.0, 2.0])))
    np.testing.assert_allclose(got["mu_s"], [0.25] * 3, atol=1e-15)
    np.testing.assert_allclose(got["mu_m"], [0.5] * 3, atol=1e-15)
    H = np.full((3, 3), -0.5) + np.eye(3) * 2.0
    np.testing.assert_allclose(got["H"], H, atol=1e-14)
    assert got["E"] == 3.0 and got["mse"] == 0.75
    from kd_tree_nn_amd import _lib
    z = _lib.IcpSums()
    z.n, z.sum_d2 = 0, 0.0
    mo = _lib.IcpMoments()
    _lib.check(_lib.lib().kdnn_moments(ctypes.byref(z), ctypes.byref(mo)), "kdnn_moments")
    assert mo.n == 0 and list(mo.H) == [0.0] * 9 and mo.mse == 0.0
    assert _lib.lib().kdnn_moments(None, ctypes.byref(mo)) == _lib.KDNN_EINVAL


def _ctypes_sums(d):
    from kd_tree_nn_amd import _lib
    s = _lib.IcpSums()
    s.n = int(d["n"])
    s.c[:] = list(np.asarray(d["c"], np.float64))
    s.sum_s[:] = list(d["sum_s"])
    s.sum_m[:] = list(d["sum_m"])
    s.sum_sm[:] = list(np.asarray(d["sum_sm"]).ravel())
    s.sum_d2 = float(d["E"])
    return s


def test_noalloc_limits_consistent(kdnn):
    """The allocation-free registration's scratch holds the ICP workspace of
    its largest input; the binding's constants are the header's."""
    from kd_tree_nn_amd import _lib
    text = open(os.path.join(ROOT, "include", "kdnn.h")).read()
    mx = int(re.search(r"#define KDNN_NOALLOC_MAX_POINTS (\d+)", text).group(1))
    sh = int(re.search(r"#define KDNN_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text).group(1))
    sb = int(re.search(r"#define KDNN_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text).group(2))
    assert (mx, sh << sb) == (_lib.KDNN_NOALLOC_MAX_POINTS, _lib.KDNN_NOALLOC_SCRATCH_BYTES)
    L = _lib.lib()
    assert L.icp_workspace_bytes(mx) <= _lib.KDNN_NOALLOC_SCRATCH_BYTES
    # argument errors come back before any device work
    assert L.icp_align_noalloc(None, None, 10, None, None, 1, 0.0, None, None, None, None, None,
                               0, None, None) == _lib.KDNN_EINVAL
