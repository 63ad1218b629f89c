"""kd_tree_nn_amd -- exact KD-tree nearest neighbours and ICP correspondences on MI355X.

A thin Python layer over libkdnn.so (C ABI: include/kdnn.h).  It only checks
and marshals arguments: every step of the search, the transform, the
reduction and the ICP loop runs in the library.  PyTorch provides device
memory (CUDA/HIP tensors) and the current stream.

    import kd_tree_nn_amd as kdnn
    tree = kdnn.Tree(target_points_cpu, leaf_size=16)      # built once, on the host
    idx, d2 = tree.query(q_gpu)                             # exact NN of every query
    res = tree.icp(src_gpu, max_iter=30)                    # ICP registration
"""

from __future__ import annotations

import ctypes
from typing import Optional

import numpy as np

from . import _lib
from ._lib import (  # noqa: F401
    KdnnError, KDNN_QUERY_NO_SORT, KDNN_QUERY_SORT, KDNN_ICP_REUSE_ORDER, KDNN_ICP_NO_SORT,
    KDNN_ICP_SORT, KDNN_ICP_HOST_LOOP, KDNN_ICP_DEVICE_LOOP, KDNN_SUMS_DOUBLES,
)

__all__ = ["Tree", "transform", "procrustes", "build_host", "layout", "sums_to_dict",
           "icp_batch", "icp_batch_workspace", "voxel_downsample", "KdnnError", "version",
           "gather_bench", "chase_bench"]


def _torch():
    import torch
    return torch


def version() -> int:
    return int(_lib.lib().kdnn_version())


def _host_points(points) -> np.ndarray:
    if hasattr(points, "detach"):
        if points.is_cuda:
            raise ValueError("target points must be host memory (build is on the CPU)")
        points = points.detach().numpy()
    a = np.ascontiguousarray(np.asarray(points, dtype=np.float32))
    if a.ndim != 2 or a.shape[1] != 3:
        raise ValueError("points must have shape (n, 3)")
    return a


def _dev_points(x, name):
    torch = _torch()
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if x.dtype != torch.float32 or x.dim() != 2 or x.shape[1] != 3:
        raise ValueError(f"{name} must be float32 of shape (n, 3)")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return x


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(None)


def _stream(stream=None) -> ctypes.c_void_p:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _mat(R, shape, name):
    a = np.ascontiguousarray(np.asarray(R, dtype=np.float64).reshape(shape))
    return a, a.ctypes.data_as(_lib.c_dp)


def _reject(max_dist, reject_k):
    """kdnn_icp_reject pointer, or NULL when neither rejection is asked for."""
    if max_dist is None and not reject_k:
        return None
    md = float("inf") if max_dist is None else float(max_dist)
    return ctypes.byref(_lib.IcpReject(md, float(reject_k or 0.0)))


def _params(leaf_size, max_depth, round_robin):
    return _lib.BuildParams(int(leaf_size), int(max_depth),
                            _lib.KDNN_BUILD_ROUND_ROBIN if round_robin else 0)


def sums_to_dict(s: "_lib.IcpSums") -> dict:
    """Correspondence sums plus the centroids, H and E the library derives from
    them (kdnn_moments); copies only."""
    m = _lib.IcpMoments()
    _lib.check(_lib.lib().kdnn_moments(ctypes.byref(s), ctypes.byref(m)), "kdnn_moments")
    n = int(s.n)
    out = {"n": n, "c": np.array(s.c[:]), "sum_s": np.array(s.sum_s[:]),
           "sum_m": np.array(s.sum_m[:]), "sum_sm": np.array(s.sum_sm[:]).reshape(3, 3),
           "E": float(s.sum_d2)}
    if n > 0:
        out["mu_s"] = np.array(m.mu_s[:])
        out["mu_m"] = np.array(m.mu_m[:])
        out["H"] = np.array(m.H[:]).reshape(3, 3)
        out["mse"] = float(m.mse)
    return out


class Tree:
    """KD-tree of a target cloud, built on the host and resident on the device."""

    def __init__(self, points, leaf_size: int = 16, max_depth: int = 0,
                 round_robin: bool = False):
        torch = _torch()
        pts = _host_points(points)
        self._h = ctypes.c_void_p(None)
        p = _params(leaf_size, max_depth, round_robin)
        h = ctypes.c_void_p()
        _lib.check(_lib.lib().kdtree_build(pts.ctypes.data, len(pts), ctypes.byref(p),
                                           ctypes.byref(h)), "kdtree_build")
        self._h = h
        self.n = len(pts)
        self.device = torch.device("cuda", torch.cuda.current_device())

    def close(self):
        if getattr(self, "_h", None):
            _lib.lib().kdtree_free(self._h)
            self._h = ctypes.c_void_p(None)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def info(self) -> dict:
        i = _lib.TreeInfo()
        _lib.check(_lib.lib().kdtree_info(self._h, ctypes.byref(i)), "kdtree_info")
        return {k: (list(getattr(i, k)) if k in ("bbox_min", "bbox_max", "center")
                    else getattr(i, k)) for k, _ in _lib.TreeInfo._fields_}

    # -------------------------------------------------------------- queries
    def query_workspace(self, m: int):
        torch = _torch()
        return torch.empty(int(_lib.lib().nn_query_workspace_bytes(m)), dtype=torch.uint8,
                           device=self.device)

    def query(self, q, sort=None, out=None, workspace=None, stream=None, lanes=None,
              budget=None, top_lds: bool = False, max_dist=None):
        """(idx int32[m], dist2 float32[m]) of the exact nearest target point.

        sort: Morton-order the queries (None = the library's choice by tree size).
        lanes: single pass with this many lanes per query (1, 2, 4, 8, 16);
        budget: two-pass schedule with this first-pass node budget;
        top_lds: single lane with the top tree levels staged in LDS.
        max_dist: only target points within this distance (else idx -1, +inf).
        """
        torch = _torch()
        q = _dev_points(q, "queries")
        m = q.shape[0]
        # buffers made here belong to the stream the search runs on, so the
        # caching allocator cannot hand them out again before it is done
        with torch.cuda.stream(stream if stream is not None else torch.cuda.current_stream()):
            idx, d2 = out if out is not None else (
                torch.empty(m, dtype=torch.int32, device=q.device),
                torch.empty(m, dtype=torch.float32, device=q.device))
            ws = None
            if m > 0:
                ws = workspace if workspace is not None else self.query_workspace(m)
        flags = (_lib.sort_flag(sort, KDNN_QUERY_SORT, KDNN_QUERY_NO_SORT)
                 | _lib.lanes_flag(lanes, budget, top_lds))
        wp, wn = _ptr(ws), ws.numel() if ws is not None else 0
        if max_dist is None:
            _lib.check(_lib.lib().nn_query(self._h, _ptr(q), m, _ptr(idx), _ptr(d2), flags,
                                           wp, wn, _stream(stream)), "nn_query")
        else:
            _lib.check(_lib.lib().nn_query_radius(self._h, _ptr(q), m, float(max_dist), _ptr(idx),
                                                  _ptr(d2), flags, wp, wn, _stream(stream)),
                       "nn_query_radius")
        return idx, d2

    def query_stats(self, q, sort=None, lanes=None, budget=None, top_lds: bool = False):
        """query() plus per-query counts of nodes loaded and leaf points scanned."""
        torch = _torch()
        q = _dev_points(q, "queries")
        m = q.shape[0]
        idx = torch.empty(m, dtype=torch.int32, device=q.device)
        d2 = torch.empty(m, dtype=torch.float32, device=q.device)
        cn = torch.empty(m, dtype=torch.int32, device=q.device)
        cp = torch.empty(m, dtype=torch.int32, device=q.device)
        ws = self.query_workspace(m) if m > 0 else None
        _lib.check(_lib.lib().nn_query_stats(
            self._h, _ptr(q), m, _ptr(idx), _ptr(d2), _ptr(cn), _ptr(cp),
            _lib.sort_flag(sort, KDNN_QUERY_SORT, KDNN_QUERY_NO_SORT)
            | _lib.lanes_flag(lanes, budget, top_lds), _ptr(ws), ws.numel() if ws is not None else 0, _stream()), "nn_query_stats")
        return idx, d2, cn, cp

    def replay_bench(self, q, icp: bool = False, sort=None, reps: int = 10, prev=None):
        """Replay ceiling of a search launch over the queries q
        (kdnn_replay_bench): each replay's kernel time in ms (numpy array of
        `reps`) and what was replayed (dict of kdnn_replay_info's fields).
        icp=True takes the fused ICP kernel's launch shape, else nn_query's;
        prev: the previous ICP iteration's queries (warm-started searches)."""
        torch = _torch()
        q = _dev_points(q, "queries")
        m = q.shape[0]
        if prev is not None:
            prev = _dev_points(prev, "prev")
            if prev.shape[0] != m:
                raise ValueError("prev must have as many points as q")
        flags = (_lib.KDNN_REPLAY_ICP if icp else 0) | _lib.sort_flag(
            sort, KDNN_QUERY_SORT, KDNN_QUERY_NO_SORT)
        nbytes = int(_lib.lib().kdnn_replay_workspace_bytes(self._h, m, flags))
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
        ms = (ctypes.c_float * int(reps))()
        info = _lib.ReplayInfo()
        _lib.check(_lib.lib().kdnn_replay_bench(self._h, _ptr(q), _ptr(prev), m, flags, int(reps),
                                                _ptr(ws), nbytes, ms, ctypes.byref(info),
                                                _stream()), "kdnn_replay_bench")
        out = {f: getattr(info, f) for f, _ in _lib.ReplayInfo._fields_}
        return np.array(ms[:], dtype=np.float64), out

    # ------------------------------------------------------------------ ICP
    def icp_workspace(self, n: int):
        torch = _torch()
        return torch.empty(int(_lib.lib().icp_workspace_bytes(n)), dtype=torch.uint8,
                           device=self.device)

    def correspond_reduce(self, src, R=None, t=None, return_pairs: bool = False,
                          flags: int = 0, workspace=None, stream=None, max_dist=None,
                          reject_k: float = 0.0) -> dict:
        """Sums of one ICP correspondence step at (R, t); optionally the pairs.

        max_dist drops pairs farther than it; reject_k > 0 also keeps the
        matches in the workspace for a following :meth:`reject_reduce`.
        """
        torch = _torch()
        src = _dev_points(src, "src")
        n = src.shape[0]
        Ra, Rp = _mat(np.eye(3) if R is None else R, (3, 3), "R")
        ta, tp = _mat(np.zeros(3) if t is None else t, (3,), "t")
        ws = workspace if workspace is not None else self.icp_workspace(n)
        idx = d2 = None
        if return_pairs:
            idx = torch.empty(n, dtype=torch.int32, device=src.device)
            d2 = torch.empty(n, dtype=torch.float32, device=src.device)
        s = _lib.IcpSums()
        _lib.check(_lib.lib().icp_correspond_reduce(
            self._h, _ptr(src), n, Rp, tp, ctypes.byref(s), _ptr(idx), _ptr(d2), int(flags),
            _reject(max_dist, reject_k), _ptr(ws), ws.numel(), _stream(stream)),
            "icp_correspond_reduce")
        out = sums_to_dict(s)
        if return_pairs:
            out["idx"], out["d2"] = idx, d2
        return out

    def correspond_reduce_async(self, src, R, t, sums_out, workspace, flags: int = 0,
                                idx=None, d2=None, stream=None, max_dist=None,
                                reject_k: float = 0.0):
        """Enqueue one correspondence step; KDNN_SUMS_DOUBLES float64 sums go to sums_out."""
        torch = _torch()
        src = _dev_points(src, "src")
        if sums_out.dtype != torch.float64 or sums_out.numel() < KDNN_SUMS_DOUBLES:
            raise ValueError("sums_out must be float64 with >= 17 elements")
        Ra, Rp = _mat(R, (3, 3), "R")
        ta, tp = _mat(t, (3,), "t")
        _lib.check(_lib.lib().icp_correspond_reduce_async(
            self._h, _ptr(src), src.shape[0], Rp, tp, _ptr(sums_out), _ptr(idx), _ptr(d2),
            int(flags), _reject(max_dist, reject_k), _ptr(workspace), workspace.numel(),
            _stream(stream)), "icp_correspond_reduce_async")

    def reject_reduce(self, src, R, t, reject_k: float, workspace, return_kept: bool = False,
                      stream=None) -> dict:
        """Residual rejection of the matches a previous :meth:`correspond_reduce`
        (with reject_k > 0, same workspace) kept: sums of the pairs whose
        residual under (R, t) is within reject_k sigma, plus sigma^2."""
        torch = _torch()
        src = _dev_points(src, "src")
        n = src.shape[0]
        Ra, Rp = _mat(R, (3, 3), "R")
        ta, tp = _mat(t, (3,), "t")
        kept = torch.empty(n, dtype=torch.uint8, device=src.device) if return_kept else None
        s = _lib.IcpSums()
        sigma2 = ctypes.c_double(0.0)
        _lib.check(_lib.lib().icp_reject_reduce(
            self._h, _ptr(src), n, Rp, tp, float(reject_k), ctypes.byref(s),
            ctypes.byref(sigma2), _ptr(kept), _ptr(workspace), workspace.numel(),
            _stream(stream)), "icp_reject_reduce")
        out = sums_to_dict(s)
        out["sigma2"] = sigma2.value
        if return_kept:
            out["kept"] = kept
        return out

    def icp(self, src, R0=None, t0=None, max_iter: int = 30, eps: float = 0.0,
            workspace=None, stream=None, lanes=None, sort=None, budget=None,
            top_lds: bool = False, max_dist=None, reject_k: float = 0.0,
            device_loop: Optional[bool] = None) -> dict:
        """ICP registration of the source (device, original coordinates) onto the
        tree; max_dist / reject_k: correspondence rejection (kdnn_icp_reject).
        device_loop: None or False = a host solve per iteration (the default;
        KDNN_ICP_HOST_LOOP); True = the iterations stay on the device
        (KDNN_ICP_DEVICE_LOOP)."""
        src = _dev_points(src, "src")
        n = src.shape[0]
        R0a = None if R0 is None else _mat(R0, (3, 3), "R0")
        t0a = None if t0 is None else _mat(t0, (3,), "t0")
        R = np.zeros(9)
        t = np.zeros(3)
        E = np.zeros(max(max_iter, 1))
        Rt = np.zeros((max(max_iter, 1), 12))
        it = ctypes.c_int32(0)
        ws = workspace if workspace is not None else self.icp_workspace(n)
        _lib.check(_lib.lib().icp_align(
            self._h, _ptr(src), n,
            R0a[1] if R0a else None, t0a[1] if t0a else None, int(max_iter), float(eps),
            R.ctypes.data_as(_lib.c_dp), t.ctypes.data_as(_lib.c_dp),
            E.ctypes.data_as(_lib.c_dp), Rt.ctypes.data_as(_lib.c_dp), ctypes.byref(it),
            _lib.sort_flag(sort, KDNN_ICP_SORT, KDNN_ICP_NO_SORT)
            | _lib.lanes_flag(lanes, budget, top_lds)
            | _lib.loop_flag(device_loop), _reject(max_dist, reject_k),
            _ptr(ws), ws.numel(), _stream(stream)), "icp_align")
        k = it.value
        return {"R": R.reshape(3, 3), "t": t, "E": E[:k], "Rt_hist": Rt[:k], "iters": k}


def transform(x, R, t, out=None, stream=None):
    """out = fl32(R x + t) per point, fp64 inside (in place when out is x)."""
    torch = _torch()
    x = _dev_points(x, "points")
    if out is None:
        out = torch.empty_like(x)
    else:
        out = _dev_points(out, "out")
    Ra, Rp = _mat(R, (3, 3), "R")
    ta, tp = _mat(t, (3,), "t")
    _lib.check(_lib.lib().transform_points(_ptr(x), _ptr(out), x.shape[0], Rp, tp,
                                           _stream(stream)), "transform_points")
    return out


def icp_batch_workspace(sources_n, device=None):
    """Device workspace for :func:`icp_batch` over pairs of these sizes."""
    torch = _torch()
    n = np.ascontiguousarray(np.asarray(sources_n, np.int64))
    nb = int(_lib.lib().icp_batch_workspace_bytes(len(n), n.ctypes.data_as(
        ctypes.POINTER(_lib.c_i64))))
    return torch.empty(nb, dtype=torch.uint8, device=device or "cuda")


def icp_batch(trees, sources, R0=None, t0=None, max_iter: int = 30, eps: float = 0.0,
              workspace=None, stream=None, max_dist=None,
              device_loop: Optional[bool] = None) -> list:
    """Register sources[p] onto trees[p] for every p together (icp_align_batch).

    Returns one dict per pair: R, t, E (per iteration), iters and status
    (0 = OK; a degenerate pair keeps its last good transform).  device_loop:
    None or True = the iterations stay on the device (the default;
    KDNN_ICP_DEVICE_LOOP); False = a host solve per iteration
    (KDNN_ICP_HOST_LOOP).
    """
    B = len(trees)
    if B != len(sources) or B < 1:
        raise ValueError("trees and sources must be non-empty and of equal length")
    srcs = [_dev_points(x, "src") for x in sources]
    n = np.ascontiguousarray([x.shape[0] for x in srcs], dtype=np.int64)
    th = (ctypes.c_void_p * B)(*[tr._h.value for tr in trees])
    sp = (ctypes.c_void_p * B)(*[x.data_ptr() for x in srcs])
    R0a = None if R0 is None else np.ascontiguousarray(np.asarray(R0, np.float64).reshape(B, 9))
    t0a = None if t0 is None else np.ascontiguousarray(np.asarray(t0, np.float64).reshape(B, 3))
    R = np.zeros((B, 9))
    t = np.zeros((B, 3))
    E = np.zeros((B, max(max_iter, 1)))
    it = np.zeros(B, np.int32)
    st = np.zeros(B, np.int32)
    ws = workspace if workspace is not None else icp_batch_workspace(n, srcs[0].device)
    status = _lib.lib().icp_align_batch(
        B, th, sp, n.ctypes.data_as(ctypes.POINTER(_lib.c_i64)),
        R0a.ctypes.data_as(_lib.c_dp) if R0a is not None else None,
        t0a.ctypes.data_as(_lib.c_dp) if t0a is not None else None,
        int(max_iter), float(eps), R.ctypes.data_as(_lib.c_dp), t.ctypes.data_as(_lib.c_dp),
        E.ctypes.data_as(_lib.c_dp), it.ctypes.data_as(ctypes.POINTER(_lib.c_i32)),
        st.ctypes.data_as(ctypes.POINTER(_lib.c_i32)),
        _lib.loop_flag(device_loop), _reject(max_dist, 0.0),
        _ptr(ws), ws.numel(), _stream(stream))
    if status not in (_lib.KDNN_OK, _lib.KDNN_EDEGENERATE):
        _lib.check(status, "icp_align_batch")
    return [{"R": R[p].reshape(3, 3), "t": t[p], "E": E[p, :it[p]], "iters": int(it[p]),
             "status": int(st[p])} for p in range(B)]


def voxel_downsample(points, leaf: float, return_counts: bool = False, workspace=None,
                     stream=None):
    """One point per occupied voxel of side ``leaf`` (the mean of its points),
    ordered by linear voxel key; device in, device out (voxel_downsample)."""
    torch = _torch()
    x = _dev_points(points, "points")
    n = x.shape[0]
    out = torch.empty((max(n, 1), 3), dtype=torch.float32, device=x.device)
    cnt = torch.empty(max(n, 1), dtype=torch.int32, device=x.device) if return_counts else None
    ws = workspace
    if ws is None and n > 0:
        ws = torch.empty(int(_lib.lib().voxel_downsample_workspace_bytes(n)), dtype=torch.uint8,
                         device=x.device)
    m = ctypes.c_int64(0)
    _lib.check(_lib.lib().voxel_downsample(
        _ptr(x), n, float(leaf), _ptr(out), ctypes.byref(m), _ptr(cnt), _ptr(ws),
        ws.numel() if ws is not None else 0, _stream(stream)), "voxel_downsample")
    k = m.value
    return (out[:k], cnt[:k]) if return_counts else out[:k]


def procrustes(sums) -> tuple:
    """Host rigid solve from correspondence sums (an IcpSums or a dict from sums_to_dict)."""
    if isinstance(sums, dict):
        s = _lib.IcpSums()
        s.n = int(sums["n"])
        s.c[:] = list(np.asarray(sums["c"], np.float64))
        s.sum_s[:] = list(np.asarray(sums["sum_s"], np.float64))
        s.sum_m[:] = list(np.asarray(sums["sum_m"], np.float64))
        s.sum_sm[:] = list(np.asarray(sums["sum_sm"], np.float64).ravel())
        s.sum_d2 = float(sums.get("E", 0.0))
        sums = s
    R = np.zeros(9)
    t = np.zeros(3)
    _lib.check(_lib.lib().kdnn_procrustes(ctypes.byref(sums), R.ctypes.data_as(_lib.c_dp),
                                          t.ctypes.data_as(_lib.c_dp)), "kdnn_procrustes")
    return R.reshape(3, 3), t


KDNN_TIMING_MAX = 65536


def timing_begin(cap: int) -> None:
    """Time the search kernel of this thread's next `cap` correspondence launches."""
    _lib.check(_lib.lib().kdnn_timing_begin(int(cap)), "kdnn_timing_begin")


def timing_end() -> np.ndarray:
    """Wait for the timed launches; their search-kernel durations in ms (float32)."""
    cnt = _lib.c_i32()
    ms = np.zeros(KDNN_TIMING_MAX, np.float32)
    _lib.check(_lib.lib().kdnn_timing_end(ms.ctypes.data_as(_lib.c_fp),
                                          KDNN_TIMING_MAX, ctypes.byref(cnt)), "kdnn_timing_end")
    return ms[:cnt.value].copy()


def gather_bench(buf, words: int, lanes: int, rounds: int, seed: int = 1, stream=None) -> float:
    """Random-gather micro-benchmark (kdnn_gather_bench): `lanes` lanes each read
    `rounds` records of `words` 16-byte words at pseudo-random indices of the
    device buffer `buf` (its bytes are taken as n_records * words * 16).
    Returns the kernel time in ms; useful bytes = lanes * rounds * words * 16."""
    torch = _torch()
    if not (hasattr(buf, "is_cuda") and buf.is_cuda and buf.is_contiguous()):
        raise ValueError("buf must be a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size()
    n_rec = nbytes // (16 * int(words))
    sink = torch.zeros(1, dtype=torch.int32, device=buf.device)
    ms = ctypes.c_float()
    _lib.check(_lib.lib().kdnn_gather_bench(_ptr(buf), n_rec, int(words), int(lanes), int(rounds),
                                            int(seed) & 0xFFFFFFFF, _ptr(sink), ctypes.byref(ms),
                                            _stream(stream)), "kdnn_gather_bench")
    return float(ms.value)


def chase_bench(next_idx, waves: int, steps: int, stream=None) -> float:
    """Dependent-load micro-benchmark (kdnn_chase_bench).  `next_idx`: a device
    int32 tensor of n_records * 16 words (64-byte records) whose word 16 k holds
    the record after record k.  Returns the kernel time in ms (ms / steps per hop)."""
    torch = _torch()
    if not (hasattr(next_idx, "is_cuda") and next_idx.is_cuda and next_idx.is_contiguous()
            and next_idx.dtype == torch.int32 and next_idx.numel() % 16 == 0):
        raise ValueError("next_idx must be a contiguous int32 device tensor of 16-word records")
    sink = torch.zeros(1, dtype=torch.int32, device=next_idx.device)
    ms = ctypes.c_float()
    _lib.check(_lib.lib().kdnn_chase_bench(_ptr(next_idx), next_idx.numel() // 16, int(waves),
                                           int(steps), _ptr(sink), ctypes.byref(ms),
                                           _stream(stream)), "kdnn_chase_bench")
    return float(ms.value)


def layout(n: int, leaf_size: int = 16, max_depth: int = 0, round_robin: bool = False):
    """(depth D, node slots 2^(D+1)) of the tree kdtree_build would make."""
    p = _params(leaf_size, max_depth, round_robin)
    d = ctypes.c_int32()
    s = ctypes.c_int64()
    _lib.check(_lib.lib().kdtree_layout(int(n), ctypes.byref(p), ctypes.byref(d),
                                        ctypes.byref(s)), "kdtree_layout")
    return d.value, s.value


def build_host(points, leaf_size: int = 16, max_depth: int = 0, round_robin: bool = False) -> dict:
    """Host-only build (no device): the node records and leaf-ordered points."""
    pts = _host_points(points)
    D, slots = layout(len(pts), leaf_size, max_depth, round_robin)
    nodes = np.zeros((slots, 8), np.float32)
    pout = np.zeros((len(pts), 4), np.float32)
    p = _params(leaf_size, max_depth, round_robin)
    _lib.check(_lib.lib().kdtree_build_host(pts.ctypes.data, len(pts), ctypes.byref(p),
                                            nodes.ctypes.data, pout.ctypes.data),
               "kdtree_build_host")
    return {"depth": D, "nodes": nodes, "points": pout}
