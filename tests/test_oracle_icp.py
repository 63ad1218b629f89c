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
    """The stop is at the FIRST iteration where the rule holds, never later."""
    p = synth.tiny()
    full = oracle.icp(p.target, p.source, iters=50, nn="brute")
    early = oracle.icp(p.target, p.source, iters=50, nn="brute", eps=1e-7)
    assert 3 <= early["iters"] < 50
    mse = full["E"] / full["n"]
    k = early["iters"] - 1
    assert abs(mse[k] - mse[k - 1]) < 1e-7 and abs(mse[k - 1] - mse[k - 2]) < 1e-7
    for j in range(2, k):   # no earlier iteration satisfies it
        assert not (abs(mse[j] - mse[j - 1]) < 1e-7 and abs(mse[j - 1] - mse[j - 2]) < 1e-7), j
    np.testing.assert_array_equal(early["E"], full["E"][:early["iters"]])


class _ScriptedTree:
    """Stands in for the oracle's KD-tree inside oracle.icp: every source point
    i is matched to target point i at a scripted squared distance, so the mean
    squared distance of iteration k is exactly script[k] (all values below are
    exact in fp32, and E / n is exact for n a power of two)."""

    def __init__(self, script):
        self.script = [np.float32(v) for v in script]
        self.k = 0

    def query(self, q):
        d = self.script[self.k]
        self.k += 1
        return np.arange(len(q), dtype=np.int32), np.full(len(q), d, np.float32)


# 8 non-coplanar points: source == target, so every solve is the identity
_CUBE = np.array([[x, y, z] for x in (0, 1) for y in (0, 2) for z in (0, 3)], np.float32)
_D = 2.0 ** -12      # a "small" change
_EPS = 2.0 ** -10    # eps of the scripted cases


def _scripted_icp(script, eps, iters=None):
    tree = _ScriptedTree(script)
    res = oracle.icp(_CUBE, _CUBE, iters or len(script), nn="kd", tree=tree, eps=eps)
    assert tree.k == res["iters"]
    np.testing.assert_array_equal(res["E"] / res["n"], np.asarray(script[:res["iters"]], np.float32))
    return res["iters"]


@pytest.mark.parametrize("script, expect", [
    # two small changes in a row at iterations 1 and 2: stop after iteration 2
    ([1.0, 1.0 - _D, 1.0 - 2 * _D, 0.5, 0.25, 0.125], 3),
    # a single small change (iteration 2), then a large one (3): no stop there;
    # two small changes at 4 and 5: stop after iteration 5 and not later
    ([1.0, 0.5, 0.5 - _D, 0.25, 0.25 - _D, 0.25 - 2 * _D, 0.25 - 3 * _D, 0.25 - 4 * _D], 6),
    # small, large, small, large ...: never two in a row, runs to the cap
    ([1.0, 1.0 - _D, 0.5, 0.5 - _D, 0.25, 0.25 - _D, 0.125, 0.125 - _D], 8),
    # a change of exactly eps is not "below eps" (strict): continues
    ([1.0, 1.0 - _EPS, 1.0 - 2 * _EPS, 1.0 - 2 * _EPS - _D, 1.0 - 2 * _EPS - 2 * _D, 0.5], 5),
    # the MSE rising counts by its magnitude too
    ([1.0, 0.5, 0.5 + _D, 0.5, 0.125], 4),
])
def test_icp_convergence_stop_on_scripted_mse(script, expect):
    """§4.6: stop once the MSE changed by less than eps on two consecutive
    iterations -- the literal iteration counts are worked out by hand."""
    assert _scripted_icp(script, _EPS) == expect


def test_icp_convergence_off_without_eps():
    script = [1.0, 1.0, 1.0, 1.0, 1.0, 1.0]
    assert _scripted_icp(script, 0.0) == 6
    assert _scripted_icp(script, _EPS) == 3


def test_mse_converged_hand_cases():
    """mse_converged over prefixes, as the loop calls it."""
    first = lambda m, eps: next((k for k in range(len(m))
                                 if oracle.mse_converged(m[:k + 1], [1] * (k + 1), eps)), None)
    assert first([1.0, 0.9, 0.89, 0.5, 0.49, 0.48, 0.47], 0.02) == 5
    assert first([1.0, 0.99, 0.98], 0.02) == 2
    assert first([1.0, 0.99, 0.5, 0.49, 0.2], 0.02) is None
    # MSE = E / n with n varying (rejection changes the pair count)
    assert oracle.mse_converged([10.0, 9.0, 8.0], [10, 9, 8], 1e-12)
    assert not oracle.mse_converged([10.0, 9.0, 8.0], [10, 10, 10], 0.05)


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
