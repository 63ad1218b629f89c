"""Seeded synthetic point clouds for the nearest-neighbour / ICP workloads.

This module is shared input plumbing: the CPU oracle (``oracle/``) and the HIP
library (``kd_tree_nn_amd``) both consume the arrays it returns, and neither
depends on the other.  It holds none of the method's arithmetic -- no
nearest-neighbour search, no transform as the method defines it, no
reduction and no rigid solve.  It only draws points (float64, numpy
``PCG64``) and applies the *generating* rigid motion with a numpy matmul before
the single cast to float32.

Sources of the workload shapes (the CUDA-KDTree ICP article, pwwt.cn
"用 CUDA-KDTree 实现 ICP", cited by section):

* §6 (simulation validation): a uniform target cloud, a known random rigid
  motion applied to it, Gaussian sensor noise; the errors are measured against
  the known motion.  ``tiny`` and ``recipe`` follow that recipe.
* §1 / §2.3: clouds of ~10^5 points per side are where the GPU search pays;
  ``scene`` is that size.  §4.3: 10^6-point inputs; ``stress`` is that size.
* §4.2 / §5.3: lidar-like, strongly non-uniform clouds; ``lidar_frames``
  ray-casts a procedural scene, ``skewed`` is a clustered cloud with far
  outliers (§4.4 talks about outliers dragging the solve).

Every array is C-contiguous float32 of shape (n, 3).  Rigid motions are given as
``(R_true, t_true)`` in float64 mapping *source* coordinates onto *target*
coordinates (``target ~ R_true @ source + t_true``), i.e. the transform ICP is
expected to recover.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

__all__ = [
    "Pair", "rng_streams", "rotation_about", "rot_z", "random_unit",
    "tiny", "scene", "stress", "lidar_frames", "lidar_pairs", "skewed",
    "recipe", "uniform_cloud", "CONFIGS",
]


@dataclass
class Pair:
    """A registration problem: target cloud, source cloud and the truth."""

    name: str
    target: np.ndarray
    source: np.ndarray
    leaf_size: int
    iters: int
    R_true: Optional[np.ndarray] = None
    t_true: Optional[np.ndarray] = None
    meta: dict = field(default_factory=dict)


def rng_streams(seed: int, k: int) -> List[np.random.Generator]:
    """``k`` independent PCG64 generators spawned from one seed."""
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(seed).spawn(k)]


def random_unit(rng: np.random.Generator) -> np.ndarray:
    """A direction drawn uniformly on the unit sphere."""
    while True:
        v = rng.normal(size=3)
        n = np.linalg.norm(v)
        if n > 1e-12:
            return v / n


def rotation_about(axis: np.ndarray, angle: float) -> np.ndarray:
    """Rotation matrix for ``angle`` radians about the unit ``axis`` (Rodrigues)."""
    a = np.asarray(axis, dtype=np.float64)
    a = a / np.linalg.norm(a)
    K = np.array([[0.0, -a[2], a[1]], [a[2], 0.0, -a[0]], [-a[1], a[0], 0.0]])
    return np.eye(3) + np.sin(angle) * K + (1.0 - np.cos(angle)) * (K @ K)


def rot_z(angle: float) -> np.ndarray:
    c, s = np.cos(angle), np.sin(angle)
    return np.array([[c, -s, 0.0], [s, c, 0.0], [0.0, 0.0, 1.0]])


def _f32(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))


def uniform_cloud(seed: int, n: int, lo: float, hi: float) -> np.ndarray:
    """``n`` points uniform in the cube [lo, hi)^3 (float32)."""
    (r,) = rng_streams(seed, 1)
    return _f32(lo + (hi - lo) * r.random((n, 3)))


# --------------------------------------------------------------------------
# Tiny: 1,024 uniform points, 5 degrees about a random axis + 0.02 shift
# --------------------------------------------------------------------------
def tiny(seed: int = 101, n: int = 1024) -> Pair:
    """Unit-cube cloud moved by a known small rigid motion plus N(0, 0.001^2) noise.

    The §6 simulation recipe at a size the brute-force oracle handles instantly.
    """
    r_pts, r_axis, r_tdir, r_noise = rng_streams(seed, 4)
    T = r_pts.random((n, 3))
    Rg = rotation_about(random_unit(r_axis), np.deg2rad(5.0))
    tg = 0.02 * random_unit(r_tdir)
    S = T @ Rg.T + tg + r_noise.normal(0.0, 0.001, size=(n, 3))
    return Pair("tiny", _f32(T), _f32(S), leaf_size=8, iters=20,
                R_true=Rg.T.copy(), t_true=-(Rg.T @ tg),
                meta={"R_gen": Rg, "t_gen": tg})


# --------------------------------------------------------------------------
# Page recipe: 200k uniform in [-25, 25]^3, 10 deg + 0.5 m, sigma 0.01
# --------------------------------------------------------------------------
def recipe(seed: int = 606, n: int = 200_000) -> Pair:
    """The §6 regression recipe at its stated size (noise sigma chosen as 0.01 m)."""
    r_pts, r_axis, r_tdir, r_noise = rng_streams(seed, 4)
    T = -25.0 + 50.0 * r_pts.random((n, 3))
    Rg = rotation_about(random_unit(r_axis), np.deg2rad(10.0))
    tg = 0.5 * random_unit(r_tdir)
    S = T @ Rg.T + tg + r_noise.normal(0.0, 0.01, size=(n, 3))
    return Pair("recipe", _f32(T), _f32(S), leaf_size=16, iters=30,
                R_true=Rg.T.copy(), t_true=-(Rg.T @ tg))


# --------------------------------------------------------------------------
# Scene: ground disk + 20 boxes + 10 spheres, density ~ 1/r^2, 100k per side
# --------------------------------------------------------------------------
def _scene_objects(rng: np.random.Generator):
    nb, ns = 20, 10
    rb = np.sqrt(rng.uniform(5.0 ** 2, 45.0 ** 2, nb))
    ab = rng.uniform(0.0, 2 * np.pi, nb)
    boxes = np.stack([rb * np.cos(ab), rb * np.sin(ab),
                      rng.uniform(1.0, 4.0, nb), rng.uniform(1.0, 4.0, nb),
                      rng.uniform(1.0, 3.0, nb), rng.uniform(0.0, 2 * np.pi, nb)], 1)
    rs = np.sqrt(rng.uniform(5.0 ** 2, 45.0 ** 2, ns))
    as_ = rng.uniform(0.0, 2 * np.pi, ns)
    spheres = np.stack([rs * np.cos(as_), rs * np.sin(as_), rng.uniform(0.5, 2.0, ns)], 1)
    return boxes, spheres


def _box_surface_points(rng, bx: np.ndarray) -> np.ndarray:
    """Area-uniform points on the 4 walls + roof of yawed boxes (one per row of bx)."""
    cx, cy, w, d, h, yaw = (bx[:, i] for i in range(6))
    m = len(bx)
    wall = 2.0 * (w + d) * h
    on_wall = rng.random(m) * (wall + w * d) < wall
    s = rng.random(m) * 2.0 * (w + d)
    z = np.where(on_wall, rng.random(m) * h, h)
    lx = np.empty(m)
    ly = np.empty(m)
    e0 = s < w
    e1 = (s >= w) & (s < w + d)
    e2 = (s >= w + d) & (s < 2 * w + d)
    e3 = s >= 2 * w + d
    lx[e0], ly[e0] = -w[e0] / 2 + s[e0], -d[e0] / 2
    lx[e1], ly[e1] = w[e1] / 2, -d[e1] / 2 + (s[e1] - w[e1])
    lx[e2], ly[e2] = w[e2] / 2 - (s[e2] - w[e2] - d[e2]), d[e2] / 2
    lx[e3], ly[e3] = -w[e3] / 2, d[e3] / 2 - (s[e3] - 2 * w[e3] - d[e3])
    roof = ~on_wall
    lx[roof] = (rng.random(roof.sum()) - 0.5) * w[roof]
    ly[roof] = (rng.random(roof.sum()) - 0.5) * d[roof]
    c, sn = np.cos(yaw), np.sin(yaw)
    return np.stack([cx + c * lx - sn * ly, cy + sn * lx + c * ly, z], 1)


def _scene_sample(rng, boxes, spheres, n: int, chunk: int = 2_000_000) -> np.ndarray:
    """Rejection-sample ``n`` surface points with acceptance (2 / max(r, 2))^2."""
    w, d, h = boxes[:, 2], boxes[:, 3], boxes[:, 4]
    areas = np.concatenate([[np.pi * 50.0 ** 2], 2 * (w + d) * h + w * d,
                            4 * np.pi * spheres[:, 2] ** 2])
    cum = np.cumsum(areas) / areas.sum()
    out, have = [], 0
    while have < n:
        k = np.minimum(np.searchsorted(cum, rng.random(chunk), side="right"), len(areas) - 1)
        P = np.empty((chunk, 3))
        g = k == 0
        rr = 50.0 * np.sqrt(rng.random(g.sum()))
        th = rng.uniform(0.0, 2 * np.pi, g.sum())
        P[g] = np.stack([rr * np.cos(th), rr * np.sin(th), np.zeros_like(rr)], 1)
        b = (k >= 1) & (k <= len(boxes))
        P[b] = _box_surface_points(rng, boxes[k[b] - 1])
        s = k > len(boxes)
        sp = spheres[k[s] - 1 - len(boxes)]
        v = rng.normal(size=(s.sum(), 3))
        v /= np.linalg.norm(v, axis=1, keepdims=True)
        P[s] = np.stack([sp[:, 0], sp[:, 1], sp[:, 2]], 1) + sp[:, 2:3] * v
        r = np.hypot(P[:, 0], P[:, 1])
        keep = rng.random(chunk) < (2.0 / np.maximum(r, 2.0)) ** 2
        out.append(P[keep])
        have += int(keep.sum())
    return np.concatenate(out)[:n]


def scene(seed: int = 202, n: int = 100_000) -> Pair:
    """Ground + boxes + spheres scene, ~1/r^2 density, independent resample as source.

    Source = an independent draw of the same surfaces, moved by a 10 degree yaw
    and a 0.5 m horizontal offset; both clouds carry N(0, 0.01^2) noise.
    """
    r_obj, r_tgt, r_src, r_ntgt, r_nsrc, r_phi = rng_streams(seed, 6)
    boxes, spheres = _scene_objects(r_obj)
    T = _scene_sample(r_tgt, boxes, spheres, n) + r_ntgt.normal(0.0, 0.01, (n, 3))
    P = _scene_sample(r_src, boxes, spheres, n) + r_nsrc.normal(0.0, 0.01, (n, 3))
    Rz = rot_z(np.deg2rad(10.0))
    phi = r_phi.uniform(0.0, 2 * np.pi)
    toff = 0.5 * np.array([np.cos(phi), np.sin(phi), 0.0])
    S = P @ Rz.T + toff
    return Pair("scene", _f32(T), _f32(S), leaf_size=16, iters=30,
                R_true=Rz.T.copy(), t_true=-(Rz.T @ toff),
                meta={"boxes": boxes, "spheres": spheres})


# --------------------------------------------------------------------------
# Query stress: 1M target + 1M queries uniform in a 100 m cube
# --------------------------------------------------------------------------
def stress(seed: int = 303, n: int = 1_000_000, m: int = 1_000_000) -> Pair:
    r_t, r_q = rng_streams(seed, 2)
    T = -50.0 + 100.0 * r_t.random((n, 3))
    Q = -50.0 + 100.0 * r_q.random((m, 3))
    return Pair("stress", _f32(T), _f32(Q), leaf_size=8, iters=0)


# --------------------------------------------------------------------------
# Skewed clusters: 32 anisotropic Gaussians + 10% far outliers among queries
# --------------------------------------------------------------------------
def _random_rotation(rng) -> np.ndarray:
    A = rng.normal(size=(3, 3))
    Q, Rr = np.linalg.qr(A)
    Q = Q * np.sign(np.diag(Rr))
    if np.linalg.det(Q) < 0:
        Q[:, 0] = -Q[:, 0]
    return Q


def skewed(seed: int = 505, n: int = 500_000, m: int = 500_000,
           outlier_frac: float = 0.10) -> Pair:
    """Clustered target; queries = fresh mixture draws + far outliers, shuffled.

    Outliers sit at a uniform direction, radius U[1000, 1100] m from the
    origin: ten times the 100 m extent of the cluster means.
    """
    r_mu, r_sig, r_rot, r_tc, r_tz, r_qc, r_qz, r_od, r_or, r_perm = rng_streams(seed, 10)
    K = 32
    mu = -50.0 + 100.0 * r_mu.random((K, 3))
    sig = np.exp(r_sig.uniform(np.log(0.05), np.log(2.0), (K, 3)))
    Qs = np.stack([_random_rotation(r_rot) for _ in range(K)])

    def draw(rc, rz, cnt):
        c = rc.integers(0, K, cnt)
        z = rz.normal(size=(cnt, 3)) * sig[c]
        return mu[c] + np.einsum("nij,nj->ni", Qs[c], z)

    T = draw(r_tc, r_tz, n)
    n_out = int(round(outlier_frac * m))
    inl = draw(r_qc, r_qz, m - n_out)
    v = r_od.normal(size=(n_out, 3))
    v /= np.linalg.norm(v, axis=1, keepdims=True)
    out = v * r_or.uniform(1000.0, 1100.0, (n_out, 1))
    Q = np.concatenate([inl, out])[r_perm.permutation(m)]
    return Pair("skewed", _f32(T), _f32(Q), leaf_size=8, iters=0,
                meta={"n_outliers": n_out})


# --------------------------------------------------------------------------
# LiDAR-like frames: 64 rings x 2048 azimuths ray-cast on a procedural scene
# --------------------------------------------------------------------------
_FACADES = ((0, 95.0), (0, -85.0), (1, 70.0), (1, -75.0))   # (axis, coordinate)
_FACADE_H = 25.0


def _lidar_scene(rng):
    nb = 60
    r = np.sqrt(rng.uniform(8.0 ** 2, 80.0 ** 2, nb))
    a = rng.uniform(0.0, 2 * np.pi, nb)
    return np.stack([r * np.cos(a), r * np.sin(a), rng.uniform(0.5, 6.0, nb),
                     rng.uniform(0.5, 6.0, nb), rng.uniform(0.5, 8.0, nb),
                     rng.uniform(0.0, 2 * np.pi, nb)], 1)


def _lidar_cast(boxes, origin, yaw, r_noise, rings=64, az=2048, max_range=120.0):
    el = np.deg2rad(np.linspace(-25.0, 3.0, rings))
    azv = 2 * np.pi * np.arange(az) / az
    E, A = np.meshgrid(el, azv, indexing="ij")
    ds = np.stack([np.cos(E) * np.cos(A), np.cos(E) * np.sin(A), np.sin(E)], -1).reshape(-1, 3)
    Rw = rot_z(yaw)
    dw = ds @ Rw.T
    t = np.full(len(dw), np.inf)
    with np.errstate(divide="ignore", invalid="ignore"):
        tg = np.where(dw[:, 2] < 0, -origin[2] / dw[:, 2], np.inf)
        t = np.minimum(t, tg)
        for ax, coord in _FACADES:
            tf = (coord - origin[ax]) / dw[:, ax]
            zf = origin[2] + tf * dw[:, 2]
            ok = (tf > 0) & (zf >= 0) & (zf <= _FACADE_H)
            t = np.minimum(t, np.where(ok, tf, np.inf))
        for cx, cy, w, d, h, byaw in boxes:
            c, s = np.cos(-byaw), np.sin(-byaw)
            ox, oy = origin[0] - cx, origin[1] - cy
            lox, loy, loz = c * ox - s * oy, s * ox + c * oy, origin[2]
            ldx = c * dw[:, 0] - s * dw[:, 1]
            ldy = s * dw[:, 0] + c * dw[:, 1]
            ldz = dw[:, 2]
            t0x, t1x = (-w / 2 - lox) / ldx, (w / 2 - lox) / ldx
            t0y, t1y = (-d / 2 - loy) / ldy, (d / 2 - loy) / ldy
            t0z, t1z = (0.0 - loz) / ldz, (h - loz) / ldz
            tn = np.maximum(np.maximum(np.minimum(t0x, t1x), np.minimum(t0y, t1y)),
                            np.minimum(t0z, t1z))
            tx = np.minimum(np.minimum(np.maximum(t0x, t1x), np.maximum(t0y, t1y)),
                            np.maximum(t0z, t1z))
            hit = (tn <= tx) & (tn > 0)
            t = np.minimum(t, np.where(hit, tn, np.inf))
    hit = t <= max_range
    tt = t[hit] + r_noise.normal(0.0, 0.02, hit.sum())
    pw = origin + tt[:, None] * dw[hit]
    return (pw - origin) @ Rw          # world -> sensor frame: Rw^T (p - o)


def lidar_frames(seed: int = 404, n_frames: int = 17):
    """17 scans along a path of 0.3 m forward + 2 degrees yaw per step.

    Returns ``(frames, poses)``: float32 clouds in each scan's own sensor frame
    (sensor 1.8 m above the ground) and the (origin, yaw) of every scan.
    """
    r_scene, r_noise = rng_streams(seed, 2)
    boxes = _lidar_scene(r_scene)
    noise_streams = [np.random.Generator(np.random.PCG64(s))
                     for s in r_noise.bit_generator.seed_seq.spawn(n_frames)]
    origin = np.array([0.0, 0.0, 1.8])
    yaw = 0.0
    frames, poses = [], []
    for k in range(n_frames):
        frames.append(_f32(_lidar_cast(boxes, origin, yaw, noise_streams[k])))
        poses.append((origin.copy(), yaw))
        origin = origin + 0.3 * np.array([np.cos(yaw), np.sin(yaw), 0.0])
        yaw += np.deg2rad(2.0)
    return frames, poses


def lidar_pairs(seed: int = 404, n_frames: int = 17, leaf_size: int = 16) -> List[Pair]:
    """Consecutive-scan pairs: target = scan k, source = scan k + 1."""
    frames, poses = lidar_frames(seed, n_frames)
    pairs = []
    for k in range(n_frames - 1):
        (o0, y0), (o1, y1) = poses[k], poses[k + 1]
        R = rot_z(y0).T @ rot_z(y1)
        t = rot_z(y0).T @ (o1 - o0)
        pairs.append(Pair(f"lidar{k}", frames[k], frames[k + 1], leaf_size=leaf_size,
                          iters=30, R_true=R, t_true=t))
    return pairs


CONFIGS = {
    "tiny": "1,024 uniform points in the unit cube, 5 deg + 0.02 motion, leaf 8, 20 iterations",
    "scene": "100k x 100k ground/boxes/spheres scene, 1/r^2 density, 10 deg yaw + 0.5 m, leaf 16, 30 iterations",
    "stress": "1M target x 1M queries uniform in a 100 m cube, one nn_query pass, leaf 8 and 16",
    "lidar": "64 x 2048 ray-cast scans, 16 consecutive pairs (0.3 m / 2 deg), 30 iterations each",
    "skewed": "500k clustered target, 500k queries with 10% far outliers, leaf 8 and 16",
}
