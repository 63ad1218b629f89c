"""Pins for the oracle's transform, reduction, rigid solve, ICP loop and metrics
(O3-O7).  Expected values come from closed forms, exact special cases, hand
arithmetic and independent library routines -- never from the oracle itself.
"""

import numpy as np
import pytest

import oracle
import synth
from oracle.ref import solve_rigid


def _rand_rot(rng):
    return synth.rotation_about(synth.random_unit(rng), rng.uniform(0.1, 3.0))


# ---------------------------------------------------------------- O3 transform
def test_transform_identity_is_bit_exact():
    rng = np.random.Generator(np.random.PCG64(0))
    P = (rng.normal(size=(1000, 3)) * 30).astype(np.float32)
    out = oracle.transform(P, np.eye(3), np.zeros(3))
    np.testing.assert_array_equal(out.view(np.uint32), P.view(np.uint32))


def test_transform_signed_permutations_exact():
    """Entries in {0, +-1}: every output is an input coordinate, negated or not,
    plus an exactly representable shift."""
    rng = np.random.Generator(np.random.PCG64(1))
    P = rng.integers(-1000, 1000, (500, 3)).astype(np.float32)
    R = np.array([[0, -1, 0], [0, 0, 1], [-1, 0, 0]], np.float64)  # det = -1? no: check below
    R = R if np.linalg.det(R) > 0 else -R
    t = np.array([2.0, -3.0, 0.5])
    out = oracle.transform(P, R, t)
    expect = np.stack([R[0, 1] * P[:, 1] + t[0], R[1, 2] * P[:, 2] + t[1],
                       R[2, 0] * P[:, 0] + t[2]], 1).astype(np.float32)
    np.testing.assert_array_equal(out, expect)


def test_transform_matches_float64_matmul():
    """Single rounding of an fp64 evaluation: within 1 fp32 ulp of R@p + t."""
    rng = np.random.Generator(np.random.PCG64(2))
    P = (rng.normal(size=(20000, 3)) * 40).astype(np.float32)
    R = _rand_rot(rng)
    t = rng.normal(size=3) * 5
    out = oracle.transform(P, R, t)
    ref = P.astype(np.float64) @ R.T + t
    ulp = np.spacing(np.abs(ref).astype(np.float32))
    assert np.all(np.abs(out - ref) <= ulp)
    assert np.mean(out == ref.astype(np.float32)) > 0.999


def test_transform_known_rotation():
    R = synth.rot_z(np.pi / 6)
    out = oracle.transform(np.array([[2.0, 0.0, 1.0]], np.float32), R, [0.0, 0.0, 0.0])
    np.testing.assert_array_equal(out[0], np.array([np.sqrt(3.0), 1.0, 1.0], np.float32))


# ---------------------------------------------------------------- O4 reduction
def test_reduce_hand_example():
    """Unit tetrahedron corners, m = 2 s: mu_s = 1/4 (1,1,1); H worked by hand:
    diag = 3 * (1/16) + 9/16 = 3/4, off-diagonal = 2/16 - 6/16 = -1/4, doubled."""
    s = np.array([[0, 0, 0], [1, 0, 0], [0, 1, 0], [0, 0, 1]], np.float32)
    d2 = np.array([0.0, 1.0, 1.0, 1.0], np.float32)
    red = oracle.reduce_pairs(s, 2 * s, d2)
    assert red["n"] == 4
    np.testing.assert_array_equal(red["mu_s"], [0.25, 0.25, 0.25])
    np.testing.assert_array_equal(red["mu_m"], [0.5, 0.5, 0.5])
    H = 2 * np.array([[0.75, -0.25, -0.25], [-0.25, 0.75, -0.25], [-0.25, -0.25, 0.75]])
    np.testing.assert_allclose(red["H"], H, rtol=0, atol=1e-15)
    assert red["E"] == 3.0


def test_reduce_closed_forms():
    rng = np.random.Generator(np.random.PCG64(3))
    s = (rng.normal(size=(5000, 3)) * [3, 1, 0.2] + [10, -4, 2]).astype(np.float32)
    d2 = np.zeros(len(s), np.float32)
    red = oracle.reduce_pairs(s, s, d2)
    cov = np.cov(s.astype(np.float64).T, bias=True) * len(s)
    np.testing.assert_allclose(red["H"], cov, rtol=1e-12, atol=1e-9)
    np.testing.assert_allclose(red["H"], red["H"].T, rtol=0, atol=1e-9)
    assert np.all(np.linalg.eigvalsh(red["H"]) > 0)
    t0 = np.array([0.5, -2.0, 7.25])
    m = s.astype(np.float64) + t0
    red2 = oracle.reduce_pairs(s, m, d2)
    np.testing.assert_allclose(red2["mu_m"], red["mu_s"] + t0, rtol=1e-14, atol=1e-12)
    np.testing.assert_allclose(red2["H"], cov, rtol=1e-12, atol=1e-9)


def test_reduce_empty():
    red = oracle.reduce_pairs(np.zeros((0, 3)), np.zeros((0, 3)), np.zeros(0))
    assert red["n"] == 0 and red["E"] == 0.0


# ---------------------------------------------------------------- O5 rigid solve
@pytest.mark.parametrize("seed", range(5))
def test_horn_recovers_known_motion(seed):
    rng = np.random.Generator(np.random.PCG64(100 + seed))
    R0 = _rand_rot(rng)
    t0 = rng.normal(size=3) * 3
    s = rng.normal(size=(200, 3)) * [5, 2, 1]
    m = s @ R0.T + t0
    red = oracle.reduce_pairs(s, m, np.zeros(len(s)))
    R, t = solve_rigid(red)
    np.testing.assert_allclose(R, R0, atol=1e-12)
    np.testing.assert_allclose(t, t0, atol=1e-12)
    assert abs(np.linalg.det(R) - 1) < 1e-12


def test_horn_equals_svd_random():
    rng = np.random.Generator(np.random.PCG64(9))
    for _ in range(50):
        H = rng.normal(size=(3, 3))
        np.testing.assert_allclose(oracle.horn(H), oracle.kabsch_svd(H), atol=1e-10)


def test_horn_reflection_gives_proper_rotation():
    """Coplanar source, target mirrored through the plane: the best orthogonal
    map is a reflection; the rotation answer has det = +1 and leaves the plane."""
    rng = np.random.Generator(np.random.PCG64(11))
    s = np.concatenate([rng.normal(size=(100, 2)) * [3, 1], np.zeros((100, 1))], 1)
    m = s * [1, 1, -1] + rng.normal(scale=1e-3, size=s.shape) * [0, 0, 1]
    red = oracle.reduce_pairs(s, m, np.zeros(len(s)))
    R = oracle.horn(red["H"])
    assert abs(np.linalg.det(R) - 1) < 1e-12
    np.testing.assert_allclose(R, oracle.kabsch_svd(red["H"]), atol=1e-8)
    np.testing.assert_allclose(R @ R.T, np.eye(3), atol=1e-12)


def test_horn_half_turn():
    """180 degrees about z: quaternion scalar part 0."""
    R0 = synth.rot_z(np.pi)
    s = np.array([[1, 0, 0], [0, 2, 0], [0, 0, 3], [1, 1, 1]], np.float64)
    red = oracle.reduce_pairs(s, s @ R0.T, np.zeros(4))
    np.testing.assert_allclose(oracle.horn(red["H"]), R0, atol=1e-12)


# ---------------------------------------------------------------- O6 ICP
def test_icp_noise_free_recovers_truth():
    rng = np.random.Generator(np.random.PCG64(21))
    T = rng.random((3000, 3)).astype(np.float32)
    Rg = synth.rotation_about(synth.random_unit(rng), np.deg2rad(1.0))
    tg = np.array([0.01, -0.005, 0.0])
    S = (T.astype(np.float64) @ Rg.T + tg).astype(np.float32)
    res = oracle.icp(T, S, iters=30, nn="brute")
    np.testing.assert_allclose(res["R"], Rg.T, atol=1e-6)
    np.testing.assert_allclose(res["t"], -(Rg.T @ tg), atol=1e-6)
    assert res["E"][-1] < 1e-9


def test_icp_tiny_recovers_within_noise_and_E_nonincreasing():
    p = synth.tiny()
    res = oracle.icp(p.target, p.source, iters=p.iters, nn="brute")
    assert np.degrees(oracle.rot_err(res["R"], p.R_true)) < 0.1
    assert oracle.trans_err(res["t"], p.t_true) < 2e-3
    E = res["E"]
    assert np.all(E[1:] <= E[:-1] * (1 + 1e-6) + 1e-9), E
    assert E[0] > 10 * E[-1]


def test_icp_kd_and_brute_agree():
    p = synth.tiny()
    a = oracle.icp(p.target, p.source, iters=p.iters, nn="brute")
    b = oracle.icp(p.target, p.source, iters=p.iters, nn="kd", leaf_size=8)
    np.testing.assert_array_equal(a["E"], b["E"])
    np.testing.assert_array_equal(a["R"], b["R"])


def test_icp_convergence_rule_stops_early():
    p = synth.tiny()
    full = oracle.icp(p.target, p.source, iters=50, nn="brute")
    early = oracle.icp(p.target, p.source, iters=50, nn="brute", eps=1e-7)
    assert 3 <= early["iters"] < 50
    mse = full["E"] / full["n"]
    k = early["iters"] - 1
    assert abs(mse[k] - mse[k - 1]) < 1e-7 and abs(mse[k - 1] - mse[k - 2]) < 1e-7
    np.testing.assert_array_equal(early["E"], full["E"][:early["iters"]])


# ---------------------------------------------------------------- O7 metrics
def test_metrics():
    for ang in [0.0, 0.3, 1.0, 2.5, np.pi]:
        R = synth.rotation_about([1.0, 2.0, -0.5], ang)
        assert abs(oracle.rot_err(R, np.eye(3)) - ang) < 1e-7
    assert oracle.trans_err([3, 4, 0], [0, 0, 0]) == 5.0


def test_transform_fixed_association():
    """((R00 x + R01 y) + R02 z) + t0 summed left to right in fp64, then one cast.

    With x = y = z = 1, R0 = (1, 2^-53, 2^-53), t0 = 2^-24: left to right, each
    2^-53 is a tie that rounds back to 1, leaving 1 + 2^-24 -- a tie in fp32 that
    rounds to 1.  Grouping (R01 y + R02 z) first would give 1 + 2^-52 + 2^-24,
    which rounds up to 1 + 2^-23."""
    R = np.eye(3)
    R[0] = [1.0, 2.0 ** -53, 2.0 ** -53]
    out = oracle.transform(np.ones((1, 3), np.float32), R, [2.0 ** -24, 0.0, 0.0])
    assert out[0, 0] == np.float32(1.0)
