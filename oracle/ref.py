"""ORACLE -- test infrastructure, not product code.

Plain CPU definitions of every step of the ICP correspondence path, written from
the CUDA-KDTree ICP article (pwwt.cn, "用 CUDA-KDTree 实现 ICP"), cited by
section.  Nearest-neighbour search is plain C (``oracle.c``, loaded with
ctypes); the rest is numpy in float64.  Nothing here is shared with, or
imported from, the library in ``kd_tree_nn_amd``.

Function                      follows                                 pinned by (tests/test_oracle_*.py)
----------------------------  --------------------------------------  -----------------------------------------------
brute_nn        (O1)          §3.2 per-query NN, fp32 distance        hand-built exact cases, scipy fp64 KD search
KDTree.query    (O2)          §2.2 tree search with plane pruning     bit equality with brute_nn on adversarial sets
transform       (O3)          §3.3 step 1 "apply current R, t"        identity / axis permutations exact, fp64 matmul
reduce_pairs    (O4)          §2.1 centroids, de-centring, H, and E   closed forms (m = s, m = s + t0), hand example
horn / kabsch   (O5)          §2.1 rigid solve from H                 known-motion recovery, Horn == SVD, det = +1
icp             (O6)          §2.1 loop, §3.3 main loop, §4.6 rule    known-motion recovery, E non-increasing
rot_err, trans_err (O7)       §6 regression metrics                   known rotation angles
max_dist_bound, residual_sq,  §4.4 correspondence rejection           hand values, inclusive bound, outlier recovery
reject_sigma (O8)
voxel_downsample (O9)         §4.3 voxel filter before the tree       hand voxels, dict-based grouping, idempotence
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIBPATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")


def _load():
    global _lib
    if _lib is not None:
        return _lib
    src = os.path.join(_HERE, "oracle.c")
    if (not os.path.exists(_LIBPATH)
            or os.path.getmtime(_LIBPATH) < os.path.getmtime(src)):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIBPATH)
    i64 = ctypes.c_int64
    lib.oracle_brute_nn.argtypes = [_f32p, i64, _f32p, i64, _i32p, _f32p]
    lib.oracle_brute_nn.restype = None
    lib.okd_build.argtypes = [_f32p, i64, ctypes.c_int32]
    lib.okd_build.restype = ctypes.c_void_p
    lib.okd_free.argtypes = [ctypes.c_void_p]
    lib.okd_free.restype = None
    lib.okd_node_count.argtypes = [ctypes.c_void_p]
    lib.okd_node_count.restype = i64
    lib.okd_query.argtypes = [ctypes.c_void_p, _f32p, i64, _i32p, _f32p, ctypes.c_void_p]
    lib.okd_query.restype = None
    lib.oracle_voxel.argtypes = [_f32p, i64, ctypes.c_double, _f32p, _i32p]
    lib.oracle_voxel.restype = i64
    _lib = lib
    return lib


def _pts(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    if a.ndim != 2 or a.shape[1] != 3:
        raise ValueError("points must have shape (n, 3)")
    return a


# ---------------------------------------------------------------------------
# O1 / O2: nearest neighbour
# ---------------------------------------------------------------------------
def brute_nn(target, queries):
    """Exact NN of every query by scanning all targets (§3.2; O(N) per query, §1).

    Returns ``(idx int32[m], d2 float32[m])``; d2 = (dx*dx + dy*dy) + dz*dz in
    fp32, lowest index on ties, (-1, +inf) when nothing is below +inf.
    """
    T, Q = _pts(target), _pts(queries)
    idx = np.empty(len(Q), np.int32)
    d2 = np.empty(len(Q), np.float32)
    _load().oracle_brute_nn(T, len(T), Q, len(Q), idx, d2)
    return idx, d2


class KDTree:
    """The oracle's own exact KD-tree (§2.2): an accelerator for big inputs.

    Round-robin split axis, middle-element split, box pruning, nearer side
    first.  ``query`` must equal :func:`brute_nn` bit for bit.
    """

    def __init__(self, target, leaf_size: int = 8):
        self.T = _pts(target)
        if len(self.T) == 0:
            raise ValueError("empty target")
        self._h = _load().okd_build(self.T, len(self.T), int(leaf_size))
        if not self._h:
            raise ValueError("okd_build failed")

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:
            _lib.okd_free(h)
            self._h = None

    @property
    def node_count(self) -> int:
        return int(_load().okd_node_count(self._h))

    def query(self, queries, return_visits: bool = False):
        Q = _pts(queries)
        idx = np.empty(len(Q), np.int32)
        d2 = np.empty(len(Q), np.float32)
        vis = np.empty(len(Q), np.int64) if return_visits else None
        _load().okd_query(self._h, Q, len(Q), idx, d2,
                          vis.ctypes.data if vis is not None else None)
        return (idx, d2, vis) if return_visits else (idx, d2)


# ---------------------------------------------------------------------------
# O3: rigid transform of the original source
# ---------------------------------------------------------------------------
def transform(points, R, t) -> np.ndarray:
    """q_r = fl32( ((R_r0*x + R_r1*y) + R_r2*z) + t_r ) in float64 (§3.3 step 1).

    The article applies the current R, t to the source each iteration, always
    starting from the original coordinates (§3.3, note under the main loop).
    Each product and sum is a separate float64 operation; one round-to-nearest
    cast to float32 at the end.
    """
    P = _pts(points).astype(np.float64)
    R = np.asarray(R, np.float64).reshape(3, 3)
    t = np.asarray(t, np.float64).reshape(3)
    x, y, z = P[:, 0], P[:, 1], P[:, 2]
    out = np.empty_like(P)
    for r in range(3):
        out[:, r] = ((R[r, 0] * x + R[r, 1] * y) + R[r, 2] * z) + t[r]
    return out.astype(np.float32)


# ---------------------------------------------------------------------------
# O4: correspondence reduction
# ---------------------------------------------------------------------------
def reduce_pairs(src, matched, d2) -> dict:
    """Centroids, cross-covariance H and squared-error sum E of the pairs (§2.1).

    s_i are *original* source points, m_i their matched target points (§3.3).
    mu_s = sum(s)/n, mu_m = sum(m)/n, H = sum (s_i - mu_s)(m_i - mu_m)^T (two
    passes, float64), E = sum d2_i (the fp32 distances, summed in float64) --
    the value of E(R, t) of §2.1 at the transform that produced the pairs.
    """
    s = np.asarray(src, np.float64).reshape(-1, 3)
    m = np.asarray(matched, np.float64).reshape(-1, 3)
    n = len(s)
    if n == 0:
        return {"n": 0, "mu_s": np.zeros(3), "mu_m": np.zeros(3),
                "H": np.zeros((3, 3)), "E": 0.0}
    mu_s = s.sum(0) / n
    mu_m = m.sum(0) / n
    H = (s - mu_s).T @ (m - mu_m)
    E = float(np.asarray(d2, np.float32).astype(np.float64).sum())
    return {"n": n, "mu_s": mu_s, "mu_m": mu_m, "H": H, "E": E}


# ---------------------------------------------------------------------------
# O5: rigid solve -- Horn's unit-quaternion closed form, SVD as a cross-check
# ---------------------------------------------------------------------------
def horn(H) -> np.ndarray:
    """Rotation R maximising tr(R H), i.e. minimising sum ||R s' - m'||^2.

    Horn (1987), "Closed-form solution of absolute orientation using unit
    quaternions": with S = H (S_ab = sum s'_a m'_b) the optimal quaternion is the
    eigenvector of the largest eigenvalue of the symmetric 4x4 matrix N below.
    The article solves the same minimisation by an SVD of H (§2.1).
    """
    S = np.asarray(H, np.float64).reshape(3, 3)
    Sxx, Sxy, Sxz = S[0]
    Syx, Syy, Syz = S[1]
    Szx, Szy, Szz = S[2]
    N = np.array([
        [Sxx + Syy + Szz, Syz - Szy, Szx - Sxz, Sxy - Syx],
        [Syz - Szy, Sxx - Syy - Szz, Sxy + Syx, Szx + Sxz],
        [Szx - Sxz, Sxy + Syx, -Sxx + Syy - Szz, Syz + Szy],
        [Sxy - Syx, Szx + Sxz, Syz + Szy, -Sxx - Syy + Szz],
    ])
    w, V = np.linalg.eigh(N)
    q0, qx, qy, qz = V[:, np.argmax(w)]
    return np.array([
        [q0 * q0 + qx * qx - qy * qy - qz * qz, 2 * (qx * qy - q0 * qz), 2 * (qx * qz + q0 * qy)],
        [2 * (qy * qx + q0 * qz), q0 * q0 - qx * qx + qy * qy - qz * qz, 2 * (qy * qz - q0 * qx)],
        [2 * (qz * qx - q0 * qy), 2 * (qz * qy + q0 * qx), q0 * q0 - qx * qx - qy * qy + qz * qz],
    ])


def kabsch_svd(H) -> np.ndarray:
    """The §2.1 SVD route with the reflection fix: R = V diag(1, 1, d) U^T."""
    U, _, Vt = np.linalg.svd(np.asarray(H, np.float64).reshape(3, 3))
    V = Vt.T
    d = 1.0 if np.linalg.det(V @ U.T) >= 0 else -1.0
    return V @ np.diag([1.0, 1.0, d]) @ U.T


def solve_rigid(red: dict, method: str = "horn"):
    """(R, t) with t = mu_m - R mu_s (§2.1: translation from the centroids)."""
    R = horn(red["H"]) if method == "horn" else kabsch_svd(red["H"])
    return R, red["mu_m"] - R @ red["mu_s"]


# ---------------------------------------------------------------------------
# O8: correspondence rejection (§4.4)
# ---------------------------------------------------------------------------
def max_dist_bound(max_dist) -> np.float32:
    """The fp32 squared-distance bound of a distance threshold (§4.4, first way).

    Pairs whose fp32 squared distance exceeds fl32(max_dist * max_dist) (the
    product in float64, one rounding) are dropped.  None, <= 0 or non-finite
    means no threshold (+inf).
    """
    if max_dist is None or not np.isfinite(max_dist) or max_dist <= 0:
        return np.float32(np.inf)
    md = float(max_dist)
    return np.float32(md * md)


def residual_sq(src, matched, R, t) -> np.ndarray:
    """r_i^2 = ||R s_i + t - m_i||^2 in float64 (§4.4, second way: residuals
    after the solve).

    Per axis e_a = (((R_a0 x + R_a1 y) + R_a2 z) + t_a) - m_a, every product and
    sum a separate float64 operation (the moved point is not rounded to
    float32), then r^2 = (e_0 e_0 + e_1 e_1) + e_2 e_2.
    """
    S = np.asarray(src, np.float32).reshape(-1, 3).astype(np.float64)
    M = np.asarray(matched, np.float32).reshape(-1, 3).astype(np.float64)
    R = np.asarray(R, np.float64).reshape(3, 3)
    t = np.asarray(t, np.float64).reshape(3)
    e = np.empty_like(S)
    for a in range(3):
        e[:, a] = (((R[a, 0] * S[:, 0] + R[a, 1] * S[:, 1]) + R[a, 2] * S[:, 2]) + t[a]) - M[:, a]
    return (e[:, 0] * e[:, 0] + e[:, 1] * e[:, 1]) + e[:, 2] * e[:, 2]


def reject_sigma(src, matched, R, t, k: float):
    """§4.4 residual rejection with the 3-sigma rule (k = 3).

    Residuals are taken under the first solve (R, t).  sigma^2 is the mean
    squared residual over the pairs (the residual vectors of a least-squares
    fit have zero mean, so this is their variance); a pair is kept iff
    r_i^2 <= (k * k) * sigma^2.  Returns (keep mask, sigma^2, threshold).
    """
    r2 = residual_sq(src, matched, R, t)
    n = len(r2)
    sigma2 = float(r2.sum()) / n if n else 0.0
    thr = (float(k) * float(k)) * sigma2
    return r2 <= thr, sigma2, thr


# ---------------------------------------------------------------------------
# O9: voxel-grid down-sampling (§4.3)
# ---------------------------------------------------------------------------
def voxel_downsample(points, leaf: float):
    """One point per occupied voxel of side ``leaf`` (§4.3 voxel filter).

    Voxel of p: floor(p_a / leaf) per axis in float64.  Each voxel yields the
    mean of its points (float64 sums in ascending point index, one cast to
    float32), listed by ascending linear key over the occupied voxels' grid
    (x fastest, z slowest).  Non-finite points are dropped.  Returns
    (centroids float32 (M, 3), counts int32 (M,)).  Plain C in ``oracle.c``.
    """
    P = _pts(points)
    if not (leaf > 0 and np.isfinite(leaf)):
        raise ValueError("leaf must be finite and > 0")
    out = np.empty((max(len(P), 1), 3), np.float32)
    cnt = np.empty(max(len(P), 1), np.int32)
    m = int(_load().oracle_voxel(P, len(P), float(leaf), out, cnt))
    return out[:m].copy(), cnt[:m].copy()


# ---------------------------------------------------------------------------
# O6: the ICP iteration
# ---------------------------------------------------------------------------
def mse_converged(E_hist, n_hist, eps: float) -> bool:
    """§4.6: the change of the mean squared pair distance stays below eps for
    two consecutive iterations."""
    if eps <= 0 or len(E_hist) < 3:
        return False
    mse = [e / max(n, 1) for e, n in zip(E_hist[-3:], n_hist[-3:])]
    return abs(mse[2] - mse[1]) < eps and abs(mse[1] - mse[0]) < eps


def icp(target, source, iters: int, R0=None, t0=None, leaf_size: int = 8,
        eps: float = 0.0, nn: str = "kd", tree: Optional[KDTree] = None,
        max_dist=None, reject_k: float = 0.0) -> dict:
    """ICP as the article describes it (§2.1, §3.3), with the optional
    correspondence rejection of §4.4.

    Each iteration k: q = transform(original source; R_k, t_k); find every
    q's nearest target point; drop pairs beyond ``max_dist``
    (:func:`max_dist_bound`); E_k = sum of the kept squared distances; solve
    the rigid motion mapping original source points onto their matches.  With
    ``reject_k`` > 0, the pairs are then filtered by :func:`reject_sigma`
    under that first solve and the motion is solved again from the pairs
    left (§4.4, the two ways combined).  Stops after ``iters`` iterations, or
    earlier under :func:`mse_converged`.  Source points whose query has no
    match (idx = -1, non-finite) are dropped from the pairs.
    """
    T = _pts(target)
    S = _pts(source)
    R = np.eye(3) if R0 is None else np.asarray(R0, np.float64).reshape(3, 3).copy()
    t = np.zeros(3) if t0 is None else np.asarray(t0, np.float64).reshape(3).copy()
    if nn == "kd" and tree is None:
        tree = KDTree(T, leaf_size)
    find = tree.query if nn == "kd" else (lambda q: brute_nn(T, q))
    tau = max_dist_bound(max_dist)
    E_hist, n_hist, Rt_hist, kept_hist = [], [], [], []
    done = 0
    for _ in range(iters):
        Rt_hist.append(np.concatenate([R.ravel(), t]))
        q = transform(S, R, t)
        idx, d2 = find(q)
        ok = (idx >= 0) & (d2 <= tau)
        Sp, Mp, dp = S[ok], T[idx[ok]], d2[ok]
        red = reduce_pairs(Sp, Mp, dp)
        E_hist.append(red["E"])
        n_hist.append(red["n"])
        R, t = solve_rigid(red)
        if reject_k > 0:
            keep, _, _ = reject_sigma(Sp, Mp, R, t, reject_k)
            R, t = solve_rigid(reduce_pairs(Sp[keep], Mp[keep], dp[keep]))
            kept_hist.append(int(keep.sum()))
        done += 1
        if mse_converged(E_hist, n_hist, eps):
            break
    return {"R": R, "t": t, "E": np.array(E_hist), "n": np.array(n_hist),
            "Rt_hist": np.array(Rt_hist), "iters": done, "kept": np.array(kept_hist)}


# ---------------------------------------------------------------------------
# O7: regression metrics
# ---------------------------------------------------------------------------
def rot_err(R, R_ref) -> float:
    """§6: arccos((tr(R^T R_ref) - 1) / 2), radians, clamped to [-1, 1]."""
    c = (np.trace(np.asarray(R).T @ np.asarray(R_ref)) - 1.0) / 2.0
    return float(np.arccos(np.clip(c, -1.0, 1.0)))


def trans_err(t, t_ref) -> float:
    """§6: ||t - t_ref||."""
    return float(np.linalg.norm(np.asarray(t, np.float64) - np.asarray(t_ref, np.float64)))
