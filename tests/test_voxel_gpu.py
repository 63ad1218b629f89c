"""GPU parity of voxel-grid down-sampling (CUDA-KDTree ICP article, §4.3)
against the oracle: centroids (bits) and counts identical, same order."""

import numpy as np
import pytest

import oracle
import synth
from tests.test_parity_gpu import dev, kdnn, lidar, say, scene, torch  # noqa: F401

pytestmark = pytest.mark.gpu


def check_voxels(kdnn, torch, P, leaf, what):
    say("voxel", what, len(P), leaf)
    ec, en = oracle.voxel_downsample(P, leaf)
    c, n = kdnn.voxel_downsample(dev(torch, P), leaf, return_counts=True)
    c = c.cpu().numpy()
    n = n.cpu().numpy()
    assert len(c) == len(ec), (what, len(c), len(ec))
    bad = np.nonzero(np.any(c.view(np.uint32) != ec.view(np.uint32), axis=1) | (n != en))[0]
    assert len(bad) == 0, (what, bad[:5], c[bad[:5]], ec[bad[:5]], n[bad[:5]], en[bad[:5]])
    return c


def test_hand_and_edge_cases(torch, kdnn):
    P = np.array([[0.5, 0.5, 0.5], [0.25, 0.75, 0.5], [1.0, 0.0, 0.0], [-0.5, 0.0, 0.0],
                  [np.float32(0.7), 0, 0]], np.float32)
    check_voxels(kdnn, torch, P, 1.0, "hand")
    check_voxels(kdnn, torch, P, 0.1, "hand fine")
    check_voxels(kdnn, torch, P[:1], 0.3, "one point")
    out = kdnn.voxel_downsample(torch.empty((0, 3), dtype=torch.float32, device="cuda"), 0.5)
    assert out.shape[0] == 0
    bad = np.full((100, 3), np.nan, np.float32)
    assert kdnn.voxel_downsample(dev(torch, bad), 0.5).shape[0] == 0
    with pytest.raises(kdnn.KdnnError, match="EINVAL"):
        kdnn.voxel_downsample(dev(torch, [[0, 0, 0], [100, 100, 100]]), 1e-4)   # 10^18 cells
    for leaf in (0.0, -1.0, np.inf, np.nan):
        with pytest.raises(kdnn.KdnnError, match="EINVAL"):
            kdnn.voxel_downsample(dev(torch, P), leaf)


@pytest.mark.parametrize("seed,leaf", [(1, 0.1), (2, 0.37), (3, 1.0), (4, 0.013), (5, 1e3)])
def test_random_clouds_with_boundaries(torch, kdnn, seed, leaf):
    rng = np.random.Generator(np.random.PCG64(seed))
    scale = min(1.0, leaf / 0.1)        # keep the grid under 2^32 cells
    P = (rng.normal(size=(50_003, 3)) * np.array([20.0, 10.0, 2.0]) * scale).astype(np.float32)
    P[::7] = np.round(P[::7] / np.float32(leaf)) * np.float32(leaf)   # on or near boundaries
    P[::1001] = P[3]                                                   # many duplicates
    P[11] = [np.nan, 1, 1]
    P[12] = [1, -np.inf, 1]
    check_voxels(kdnn, torch, P, leaf, f"random seed {seed}")


def test_workloads(torch, kdnn):
    sc = scene()
    for leaf in (0.05, 0.1, 0.5):
        check_voxels(kdnn, torch, sc.target, leaf, "scene target")
    check_voxels(kdnn, torch, lidar()[0].target, 0.2, "lidar frame")
    st = synth.stress()
    check_voxels(kdnn, torch, st.target, 2.0, "stress 1M")


def test_idempotent_on_gpu(torch, kdnn):
    sc = scene()
    c = kdnn.voxel_downsample(dev(torch, sc.target), 0.3)
    c2, n2 = kdnn.voxel_downsample(c.contiguous(), 0.3, return_counts=True)
    assert torch.equal(c.view(torch.int32), c2.view(torch.int32))
    assert bool((n2 == 1).all())


def test_large_voxels(torch, kdnn):
    """Voxels of more points than one lane sums (a wave sums them, in windows
    of 256 points): 8 LiDAR frames at 0.5 m and 1 m (up to ~1,800 and ~6,100
    points per voxel), and voxels of 64, 65, 255-257, 513 and 5,000 points."""
    P = np.concatenate([p.source for p in lidar()[:8]]).astype(np.float32)
    for leaf in (0.5, 1.0):
        c = check_voxels(kdnn, torch, P, leaf, f"8 lidar frames, leaf {leaf}")
        assert len(c) > 0
    rng = np.random.Generator(np.random.PCG64(11))
    sizes = [64, 65, 255, 256, 257, 513, 5000]
    parts = [rng.uniform(0.05, 0.95, (m, 3)) + [4.0 * k, 0.0, 0.0] for k, m in enumerate(sizes)]
    parts.append(rng.uniform(-60.0, 60.0, (30_000, 3)))
    Q = np.concatenate(parts).astype(np.float32)
    Q = Q[rng.permutation(len(Q))]
    _, en = oracle.voxel_downsample(Q, 1.0)
    assert set(sizes) <= set(en.tolist())
    check_voxels(kdnn, torch, Q, 1.0, "voxels at the one-lane and window limits")


def test_errors_then_a_good_call(torch, kdnn):
    """The grid's range checks run on the device: each error is reported after
    the call, and the next call on the same workspace is unaffected."""
    P = np.array([[0.5, 0.5, 0.5], [0.25, 0.75, 0.5], [1.0, 0.0, 0.0], [-0.5, 0.0, 0.0]],
                 np.float32)
    ec, en = oracle.voxel_downsample(P, 1.0)
    ws = torch.empty(int(kdnn._lib.lib().voxel_downsample_workspace_bytes(len(P))),
                     dtype=torch.uint8, device="cuda")
    for bad, leaf, what in [([[1e30, 0, 0], [0, 0, 0]], 1e-10, "too small for the coordinates"),
                            ([[0, 0, 0], [100, 100, 100]], 1e-4, "2\\^32 cells")]:
        with pytest.raises(kdnn.KdnnError, match=what):
            kdnn.voxel_downsample(dev(torch, bad), leaf, workspace=ws)
        c, n = kdnn.voxel_downsample(dev(torch, P), 1.0, return_counts=True, workspace=ws)
        assert np.array_equal(c.cpu().numpy().view(np.uint32), ec.view(np.uint32))
        assert np.array_equal(n.cpu().numpy(), en)
