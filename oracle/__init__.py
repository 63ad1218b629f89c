"""ORACLE -- test infrastructure, not product code.

A plain, slow CPU implementation of what the nearest-neighbour / ICP path
computes.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may import it; the library in ``kd_tree_nn_amd`` never does, and
the two share no code.  Floating point follows the article's fp32 distance and
fp64 solve (see ``ref.py`` for each function's citation and its pins).
"""

from .ref import (  # noqa: F401
    brute_nn, KDTree, transform, reduce_pairs, horn, kabsch_svd, icp,
    rot_err, trans_err, mse_converged, max_dist_bound, residual_sq, reject_sigma, solve_rigid,
    voxel_downsample,
)
