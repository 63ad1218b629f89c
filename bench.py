#!/usr/bin/env python3
"""NN queries/s and ICP iterations/s at 100k x 100k points on one MI355X.

Workload (seeded, synthetic): the Scene pair -- 100k-point target sampled on a
ground disk, 20 boxes and 10 spheres (density ~ 1/r^2, 1 cm noise); source = an
independent 100k resample moved by 10 degrees of yaw and 0.5 m; leaf 16.

One step = one ICP registration of 30 iterations (transform, exact NN of all
100k source points, fp64 reduction, host SVD, per iteration) with the tree
already built and both clouds resident in device memory.  The tree build and
upload are timed separately.  value = NN queries/s over the timed steps
(30 x 100k queries per step); icp_iters_per_s is the same clock.

Also reported: the fused correspondence kernel's duration (HIP events around
each launch on the launch stream) and its roofline against algorithmic bytes
counted by the instrumented traversal; standalone nn_query rates with and
without the Morton ordering; and the CPU oracle on the host (one thread).

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NN queries/sec and ICP iterations/sec at 100k×100k points, 1 MI355X"
HBM_PEAK_GBS = 8000.0


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--kernel-reps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world})", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import kd_tree_nn_amd as kdnn
    import synth

    assert torch.cuda.is_available(), "bench needs a HIP device"
    torch.cuda.set_device(0)
    ITERS = 30

    log("generating Scene workload")
    p = synth.scene()
    n = len(p.source)
    log("building tree")
    t0 = time.perf_counter()
    tree = kdnn.Tree(p.target, p.leaf_size)
    build_wall_ms = (time.perf_counter() - t0) * 1e3
    info = tree.info
    src = torch.from_numpy(p.source).cuda()
    ws = tree.icp_workspace(n)
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- headline
    log(f"warmup {args.warmup} registrations")
    for _ in range(args.warmup):
        g = tree.icp(src, max_iter=ITERS, workspace=ws)
    torch.cuda.synchronize()
    log(f"timing {args.steps} registrations x {ITERS} iterations")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        g = tree.icp(src, max_iter=ITERS, workspace=ws)
    torch.cuda.synchronize()
    T = time.perf_counter() - t0
    assert g["iters"] == ITERS
    value = args.steps * ITERS * n / T
    iters_per_s = args.steps * ITERS / T
    log(f"{value / 1e9:.3f} G queries/s, {iters_per_s:.0f} ICP iterations/s")

    # ------------------------------------------- fused kernel: events per launch
    Rt = g["Rt_hist"]
    stream = torch.cuda.current_stream()
    sums = torch.zeros(kdnn.KDNN_SUMS_DOUBLES, dtype=torch.float64, device="cuda")
    tree.correspond_reduce_async(src, Rt[0, :9], Rt[0, 9:], sums, ws)   # computes the order
    evs = []
    for _ in range(args.kernel_reps):
        for k in range(ITERS):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            tree.correspond_reduce_async(src, Rt[k, :9], Rt[k, 9:], sums, ws,
                                         flags=kdnn.KDNN_ICP_REUSE_ORDER)
            e1.record(stream)
            evs.append((e0, e1))
    torch.cuda.synchronize()
    kern_ms = np.array([a.elapsed_time(b) for a, b in evs])
    kern_avg_ms = float(kern_ms.mean())
    log(f"fused kernel: mean {kern_avg_ms * 1e3:.1f} us, median {np.median(kern_ms) * 1e3:.1f} us")

    # algorithmic bytes of one launch, per iteration's transform
    nodes_tot, pts_tot = [], []
    for k in range(ITERS):
        q = kdnn.transform(src, Rt[k, :9], Rt[k, 9:])
        _, _, cn, cp = tree.query_stats(q)
        nodes_tot.append(int(cn.sum()))
        pts_tot.append(int(cp.sum()))
    nodes_avg = float(np.mean(nodes_tot)) / n
    pts_avg = float(np.mean(pts_tot)) / n
    n_blocks = min((n + 255) // 256, 4096)
    per_query = 32 * nodes_avg + 16 * pts_avg + 12 + 4
    bytes_launch = n * per_query + n_blocks * 17 * 8 * 2 + 17 * 8
    achieved = bytes_launch / (kern_avg_ms * 1e-3) / 1e9
    descent_lb = 32 * (info["depth"] + 1) + 16 * (n / 2 ** info["depth"]) + 16

    # ------------------------------------------------------ standalone nn_query
    def time_query(q, sort, reps=20):
        qws = tree.query_workspace(len(q))
        out = (torch.empty(len(q), dtype=torch.int32, device="cuda"),
               torch.empty(len(q), dtype=torch.float32, device="cuda"))
        tree.query(q, sort=sort, out=out, workspace=qws)
        ts = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            tree.query(q, sort=sort, out=out, workspace=qws)
            e1.record(stream)
            ts.append((e0, e1))
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ts]))

    q0 = src
    qc = kdnn.transform(src, g["R"], g["t"])
    nnq = {}
    for name, q in (("iteration0", q0), ("converged", qc)):
        for sort in (True, False):
            ms = time_query(q, sort)
            nnq[f"{name}_{'morton' if sort else 'unsorted'}"] = {
                "ms": round(ms, 4), "queries_per_s": round(len(q) / (ms * 1e-3))}
    log("nn_query:", nnq)

    result = {
        "metric": METRIC,
        "value": round(value),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(T / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 distances, f64 transform+reduction",
        "data": "synthetic",
        "config": {
            "workload": "scene-100k-icp30",
            "target_points": len(p.target), "source_points": n, "leaf_size": p.leaf_size,
            "icp_iterations_per_step": ITERS, "tree_depth": info["depth"],
            "step": "one 30-iteration ICP registration, tree and clouds resident",
        },
        "icp_iters_per_s": round(iters_per_s, 1),
        "icp_iter_us": round(T / (args.steps * ITERS) * 1e6, 2),
        "build": {"host_build_ms": round(info["build_ms"], 3),
                  "upload_ms": round(info["upload_ms"], 3),
                  "wall_ms": round(build_wall_ms, 3),
                  "registration_incl_build_ms": round(build_wall_ms + T / args.steps * 1e3, 3)},
        "fused_kernel": {"name": "icp_fused_kernel", "mean_us": round(kern_avg_ms * 1e3, 2),
                         "median_us": round(float(np.median(kern_ms)) * 1e3, 2),
                         "launches": len(kern_ms),
                         "queries_per_s": round(n / (kern_avg_ms * 1e-3))},
        "nn_query": nnq,
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
            "kernel": "icp_fused_kernel",
            "bytes_per_launch": round(bytes_launch),
            "bytes_per_query": round(per_query, 1),
            "nodes_per_query": round(nodes_avg, 2), "points_per_query": round(pts_avg, 2),
            "single_descent_bytes_per_query": round(descent_lb, 1),
            "note": "working set (~2 MB) is L2-resident; algorithmic gather bytes vs HBM peak",
        },
    }

    if not args.no_cpu_baseline:
        import oracle
        log("cpu baseline: oracle ICP, 30 iterations, 1 thread")
        t0 = time.perf_counter()
        o = oracle.icp(p.target, p.source, ITERS, leaf_size=p.leaf_size)
        Tc = time.perf_counter() - t0
        result["cpu_baseline"] = {
            "value": round(ITERS * n / Tc), "unit": "queries/s", "cores": 1, "kind": "oracle",
            "sample": "one full Scene registration (30 ICP iterations x 100k queries) with the "
                      "oracle's C KD-tree search and numpy fp64 reduction/Horn solve, "
                      f"{Tc:.2f} s wall",
            "icp_iters_per_s": round(ITERS / Tc, 2),
            "R_diff_vs_gpu": float(np.linalg.norm(o["R"] - g["R"])),
        }
        log(f"cpu baseline {ITERS * n / Tc / 1e6:.2f} M queries/s")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
