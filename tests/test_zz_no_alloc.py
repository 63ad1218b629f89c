"""GPU: icp_align_noalloc (the registration for callers that cannot allocate,
workspace in a library-owned device array) against icp_align with a caller
workspace, through the C ABI: two calls in a row on the shared scratch, the
second with a smaller input, each bit-identical to the allocating call."""

import ctypes
import sys

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import kd_tree_nn_amd as kdnn
    from kd_tree_nn_amd import _lib
    _lib.lib()
    return torch, kdnn, _lib


def _run(_lib, fn, tree, src, n, iters, flags, ws=None, reject=None, eps=0.0):
    R, t = np.zeros(9), np.zeros(3)
    E, Rt = np.zeros(iters), np.zeros((iters, 12))
    it = ctypes.c_int32(-1)
    args = [tree._h, ctypes.c_void_p(src.data_ptr()), n, None, None, iters, eps,
            R.ctypes.data_as(_lib.c_dp), t.ctypes.data_as(_lib.c_dp),
            E.ctypes.data_as(_lib.c_dp), Rt.ctypes.data_as(_lib.c_dp), ctypes.byref(it), flags,
            ctypes.byref(reject) if reject is not None else None]
    if ws is not None:
        args += [ctypes.c_void_p(ws.data_ptr()), ws.numel()]
    args.append(None)
    st = getattr(_lib.lib(), fn)(*args)
    assert st == _lib.KDNN_OK, (fn, st, _lib.lib().kdnn_last_error())
    k = it.value
    return R, t, E[:k], Rt[:k], k


def _same(a, b, what):
    for x, y, name in zip(a, b, ("R", "t", "E", "Rt_hist", "iters")):
        np.testing.assert_array_equal(x, y, err_msg=f"{what}: {name}")


@pytest.mark.parametrize("flags_name", ["host_loop", "device_loop", "device_loop_sorted",
                                        "host_loop_sorted_reject"])
def test_noalloc_matches_icp_align_twice(env, flags_name):
    torch, kdnn, _lib = env
    flags = {"host_loop": 0, "device_loop": _lib.KDNN_ICP_DEVICE_LOOP,
             "device_loop_sorted": _lib.KDNN_ICP_DEVICE_LOOP | _lib.KDNN_ICP_SORT,
             "host_loop_sorted_reject": _lib.KDNN_ICP_SORT}[flags_name]
    reject = _lib.IcpReject(1.0, 3.0) if flags_name.endswith("reject") else None
    sc, tn = synth.scene(), synth.tiny()
    for name, p, leaf in (("scene 100k", sc, 16), ("tiny 1024 (smaller, second)", tn, 8)):
        say("noalloc", flags_name, name)
        tree = kdnn.Tree(p.target, leaf)
        src = torch.from_numpy(np.ascontiguousarray(p.source)).cuda()
        n = len(p.source)
        ws = tree.icp_workspace(n)
        ref = _run(_lib, "icp_align", tree, src, n, p.iters, flags, ws=ws, reject=reject)
        got = _run(_lib, "icp_align_noalloc", tree, src, n, p.iters, flags, reject=reject)
        assert got[4] == p.iters
        _same(got, ref, f"{flags_name} {name}")


def test_noalloc_limit_and_eps(env):
    torch, kdnn, _lib = env
    p = synth.tiny()
    tree = kdnn.Tree(p.target, 8)
    src = torch.from_numpy(np.ascontiguousarray(p.source)).cuda()
    say("noalloc eps stop")
    ws = tree.icp_workspace(len(p.source))
    ref = _run(_lib, "icp_align", tree, src, len(p.source), 50, 0, ws=ws, eps=1e-7)
    got = _run(_lib, "icp_align_noalloc", tree, src, len(p.source), 50, 0, eps=1e-7)
    assert 3 <= got[4] < 50
    _same(got, ref, "eps 1e-7")
    say("noalloc beyond the limit")
    big = _lib.KDNN_NOALLOC_MAX_POINTS + 1
    R, t = np.zeros(9), np.zeros(3)
    st = _lib.lib().icp_align_noalloc(tree._h, ctypes.c_void_p(src.data_ptr()), big, None, None,
                                      5, 0.0, R.ctypes.data_as(_lib.c_dp),
                                      t.ctypes.data_as(_lib.c_dp), None, None, None, 0, None, None)
    assert st == _lib.KDNN_EINVAL and b"exceeds" in _lib.lib().kdnn_last_error()
