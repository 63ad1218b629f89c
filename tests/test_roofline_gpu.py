"""Roofline micro-benchmarks through the C ABI (kdnn_gather_bench,
kdnn_chase_bench): they run, time something, and reject bad arguments on the
host before any launch."""

import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


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


def test_gather_bench_shapes(torch, kdnn):
    buf = torch.zeros(1 << 18, dtype=torch.float32, device="cuda")  # 1 MiB
    for words in (1, 3, 16):
        say("gather bench, words", words)
        ms = kdnn.gather_bench(buf, words, lanes=256 * 64, rounds=8, seed=words)
        assert ms > 0.0


def test_chase_bench_chain_and_garbage(torch, kdnn):
    n = 4096
    rng = np.random.Generator(np.random.PCG64(5))
    perm = rng.permutation(n).astype(np.int32)
    nxt = np.zeros((n, 16), np.int32)
    nxt[perm, 0] = np.roll(perm, -1)              # one random cycle through all records
    say("chase bench, cycle of", n)
    ms = kdnn.chase_bench(torch.from_numpy(nxt.ravel()).cuda(), waves=1, steps=256)
    assert ms > 0.0
    # indices past the end are read as the last record: still in bounds
    junk = torch.full((n * 16,), -1, dtype=torch.int32, device="cuda")
    say("chase bench, out-of-range indices")
    assert kdnn.chase_bench(junk, waves=2, steps=64) > 0.0


def test_bench_argument_checks(torch, kdnn):
    from kd_tree_nn_amd import _lib
    L = _lib.lib()
    buf = torch.zeros(1 << 12, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    import ctypes
    ms = ctypes.c_float()
    p, s = buf.data_ptr(), sink.data_ptr()
    say("bench argument checks")
    bad = [(p, 64, 2, 256, 4), (p, 64, 3, 100, 4), (p, 64, 3, 256, 3), (p, 0, 1, 256, 4),
           (p + 4, 64, 1, 256, 4)]
    for a in bad:
        assert L.kdnn_gather_bench(a[0], a[1], a[2], a[3], a[4], 1, s, ctypes.byref(ms), None) \
            == _lib.KDNN_EINVAL, a
    assert L.kdnn_chase_bench(p + 16, 16, 1, 1, s, ctypes.byref(ms), None) == _lib.KDNN_EINVAL
    assert L.kdnn_chase_bench(p, 16, 0, 1, s, ctypes.byref(ms), None) == _lib.KDNN_EINVAL
    assert L.kdnn_chase_bench(p, 16, 1, 1, None, ctypes.byref(ms), None) == _lib.KDNN_EINVAL
