"""ctypes declarations of libkdnn.so (the C ABI in include/kdnn.h)."""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIBPATH = os.path.join(HERE, "libkdnn.so")

c_i32, c_i64, c_u32, c_sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t
c_vp, c_dp, c_fp = ctypes.c_void_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_float)

KDNN_OK, KDNN_EINVAL, KDNN_ENOMEM, KDNN_EDEVICE, KDNN_ENONFINITE, KDNN_EDEGENERATE = range(6)
STATUS_NAMES = {0: "OK", 1: "EINVAL", 2: "ENOMEM", 3: "EDEVICE", 4: "ENONFINITE", 5: "EDEGENERATE"}
KDNN_BUILD_ROUND_ROBIN = 1
KDNN_QUERY_NO_SORT = 1
KDNN_QUERY_SORT = 2
KDNN_ICP_REUSE_ORDER = 1
KDNN_ICP_NO_SORT = 2
KDNN_ICP_SORT = 4
KDNN_ICP_HOST_LOOP = 8
KDNN_ICP_DEVICE_LOOP = 16
KDNN_SUMS_DOUBLES = 17
KDNN_REPLAY_ICP = 4
KDNN_REPLAY_CAP = 512
KDNN_NOALLOC_MAX_POINTS = 262144
KDNN_NOALLOC_SCRATCH_BYTES = 12 << 20
KDNN_LANES_SHIFT = 8
KDNN_BUDGET_SHIFT = 16
KDNN_TOP_LDS = 1 << 24


def lanes_flag(lanes=None, budget=None, top_lds=False):
    """Schedule flags: KDNN_LANES(g) (single pass, g lanes per query),
    KDNN_BUDGET(b) (two passes, first-pass budget b), KDNN_TOP_LDS; all
    unset = the library's automatic choice."""
    return (((int(lanes or 0) & 0x1f) << KDNN_LANES_SHIFT)
            | ((int(budget or 0) & 0xff) << KDNN_BUDGET_SHIFT)
            | (KDNN_TOP_LDS if top_lds else 0))


def sort_flag(sort, on, off):
    """Ordering flag: None = the library's automatic choice, True/False forced."""
    return 0 if sort is None else (on if sort else off)


class BuildParams(ctypes.Structure):
    _fields_ = [("leaf_size", c_i32), ("max_depth", c_i32), ("flags", c_u32)]


class TreeInfo(ctypes.Structure):
    _fields_ = [("n", c_i64), ("depth", c_i32), ("leaf_size", c_i32), ("node_slots", c_i64),
                ("leaves", c_i64), ("min_leaf", c_i32), ("max_leaf", c_i32),
                ("bbox_min", ctypes.c_float * 3), ("bbox_max", ctypes.c_float * 3),
                ("center", ctypes.c_double * 3), ("build_ms", ctypes.c_double),
                ("upload_ms", ctypes.c_double), ("device_bytes", c_i64),
                ("l2_bytes", c_i64), ("auto_sort", c_i32),
                ("auto_sort_icp", c_i32)]


class IcpReject(ctypes.Structure):
    _fields_ = [("max_dist", ctypes.c_double), ("reject_k", ctypes.c_double)]


class IcpSums(ctypes.Structure):
    _fields_ = [("n", c_i64), ("c", ctypes.c_double * 3), ("sum_s", ctypes.c_double * 3),
                ("sum_m", ctypes.c_double * 3), ("sum_sm", ctypes.c_double * 9),
                ("sum_d2", ctypes.c_double)]


class IcpMoments(ctypes.Structure):
    _fields_ = [("n", c_i64), ("mu_s", ctypes.c_double * 3), ("mu_m", ctypes.c_double * 3),
                ("H", ctypes.c_double * 9), ("E", ctypes.c_double), ("mse", ctypes.c_double)]


class ReplayInfo(ctypes.Structure):
    _fields_ = [("visits", c_i64), ("bytes", c_i64), ("node_records", c_i64),
                ("leaf_points", c_i64), ("truncated", c_i64), ("blocks", c_i64),
                ("queries_per_wave", c_i32), ("spread", c_i32)]


def loop_flag(device_loop):
    """ICP loop flag: None = the entry point's default, True = iterations on the
    device (KDNN_ICP_DEVICE_LOOP), False = a host solve per iteration."""
    return 0 if device_loop is None else (KDNN_ICP_DEVICE_LOOP if device_loop else KDNN_ICP_HOST_LOOP)


# name -> (restype, argtypes)
SIGNATURES = {
    "kdtree_build": (c_i32, [c_vp, c_i64, ctypes.POINTER(BuildParams), ctypes.POINTER(c_vp)]),
    "kdtree_free": (None, [c_vp]),
    "kdtree_info": (c_i32, [c_vp, ctypes.POINTER(TreeInfo)]),
    "kdtree_layout": (c_i32, [c_i64, ctypes.POINTER(BuildParams), ctypes.POINTER(c_i32),
                              ctypes.POINTER(c_i64)]),
    "kdtree_build_host": (c_i32, [c_vp, c_i64, ctypes.POINTER(BuildParams), c_vp, c_vp]),
    "nn_query_workspace_bytes": (c_sz, [c_i64]),
    "nn_query": (c_i32, [c_vp, c_vp, c_i64, c_vp, c_vp, c_u32, c_vp, c_sz, c_vp]),
    "nn_query_radius": (c_i32, [c_vp, c_vp, c_i64, ctypes.c_double, c_vp, c_vp, c_u32, c_vp, c_sz,
                                c_vp]),
    "nn_query_stats": (c_i32, [c_vp, c_vp, c_i64, c_vp, c_vp, c_vp, c_vp, c_u32, c_vp, c_sz, c_vp]),
    "transform_points": (c_i32, [c_vp, c_vp, c_i64, c_dp, c_dp, c_vp]),
    "icp_workspace_bytes": (c_sz, [c_i64]),
    "icp_correspond_reduce": (c_i32, [c_vp, c_vp, c_i64, c_dp, c_dp, ctypes.POINTER(IcpSums),
                                      c_vp, c_vp, c_u32, ctypes.POINTER(IcpReject), c_vp, c_sz,
                                      c_vp]),
    "icp_correspond_reduce_async": (c_i32, [c_vp, c_vp, c_i64, c_dp, c_dp, c_vp, c_vp, c_vp,
                                            c_u32, ctypes.POINTER(IcpReject), c_vp, c_sz, c_vp]),
    "icp_reject_reduce": (c_i32, [c_vp, c_vp, c_i64, c_dp, c_dp, ctypes.c_double,
                                  ctypes.POINTER(IcpSums), c_dp, c_vp, c_vp, c_sz, c_vp]),
    "kdnn_procrustes": (c_i32, [ctypes.POINTER(IcpSums), c_dp, c_dp]),
    "kdnn_moments": (c_i32, [ctypes.POINTER(IcpSums), ctypes.POINTER(IcpMoments)]),
    "icp_align": (c_i32, [c_vp, c_vp, c_i64, c_dp, c_dp, c_i32, ctypes.c_double, c_dp, c_dp,
                          c_dp, c_dp, ctypes.POINTER(c_i32), c_u32, ctypes.POINTER(IcpReject),
                          c_vp, c_sz, c_vp]),
    "icp_align_noalloc": (c_i32, [c_vp, c_vp, c_i64, c_dp, c_dp, c_i32, ctypes.c_double, c_dp,
                                  c_dp, c_dp, c_dp, ctypes.POINTER(c_i32), c_u32,
                                  ctypes.POINTER(IcpReject), c_vp]),
    "icp_batch_workspace_bytes": (c_sz, [c_i32, ctypes.POINTER(c_i64)]),
    "icp_align_batch": (c_i32, [c_i32, c_vp, c_vp, ctypes.POINTER(c_i64), c_dp, c_dp, c_i32,
                                ctypes.c_double, c_dp, c_dp, c_dp, ctypes.POINTER(c_i32),
                                ctypes.POINTER(c_i32), c_u32, ctypes.POINTER(IcpReject), c_vp,
                                c_sz, c_vp]),
    "voxel_downsample_workspace_bytes": (c_sz, [c_i64]),
    "voxel_downsample": (c_i32, [c_vp, c_i64, ctypes.c_double, c_vp, ctypes.POINTER(c_i64), c_vp,
                                 c_vp, c_sz, c_vp]),
    "kdnn_timing_begin": (c_i32, [c_i32]),
    "kdnn_gather_bench": (c_i32, [c_vp, c_i64, c_i32, c_i64, c_i32, c_u32, c_vp, c_fp, c_vp]),
    "kdnn_chase_bench": (c_i32, [c_vp, c_i64, c_i32, c_i32, c_vp, c_fp, c_vp]),
    "kdnn_timing_end": (c_i32, [c_fp, c_i32, ctypes.POINTER(c_i32)]),
    "kdnn_replay_workspace_bytes": (c_sz, [c_vp, c_i64, c_u32]),
    "kdnn_replay_bench": (c_i32, [c_vp, c_vp, c_vp, c_i64, c_u32, c_i32, c_vp, c_sz, c_fp,
                                  ctypes.POINTER(ReplayInfo), c_vp]),
    "kdnn_last_error": (ctypes.c_char_p, []),
    "kdnn_version": (c_i32, []),
}

_lib = None


class KdnnError(RuntimeError):
    def __init__(self, status, where, msg):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {msg}")


def lib():
    """Load libkdnn.so; fail loudly if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBPATH):
            raise RuntimeError(f"{LIBPATH} is missing: build it with "
                               "`python -m kd_tree_nn_amd.build`")
        L = ctypes.CDLL(LIBPATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def check(status, where):
    if status != KDNN_OK:
        msg = lib().kdnn_last_error()
        raise KdnnError(status, where, msg.decode() if msg else "")
