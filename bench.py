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
each launch, on the stream it is launched on) and its roofline against the
algorithmic bytes counted by the instrumented traversal; HBM traffic from the
committed rocprofv3 counter summary when it was taken on the current kernel
source; standalone nn_query rates with and without the Morton ordering; and
the CPU oracle on the host (one thread, a bounded sample).

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --profile-pass    # short run for rocprofv3 counter passes
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
KERNEL_SRC = os.path.join(ROOT, "kd_tree_nn_amd", "csrc", "kernels.hip")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "icp_fused_kernel_scene100k_traffic.txt")
COPY_MIB = 512


def kernel_source_hash():
    """SHA-256 (first 16 hex digits) of the kernel source's code: comments and
    whitespace are dropped first, so an edited comment does not invalidate a
    counter summary taken on the same code."""
    import hashlib
    import re
    with open(KERNEL_SRC) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)   # block comments
    src = re.sub(r"//[^\n]*", " ", src)                 # line comments
    code = " ".join(src.split())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def committed_traffic():
    """HBM bytes per fused launch from the counter summary, or None when the
    summary is missing or was taken on another kernel source."""
    try:
        with open(TRAFFIC_SUMMARY) as f:
            kv = dict(line.split("=", 1) for line in f.read().splitlines()
                      if "=" in line and not line.startswith(("#", " ")))
    except OSError:
        return None, "no counter summary"
    if kv.get("kernels_hip_sha256_16", "").strip() != kernel_source_hash():
        return None, "counter summary predates the current kernel source"
    return float(kv["traffic_bytes_per_launch"]), TRAFFIC_SUMMARY[len(ROOT) + 1:]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


TRACE_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/trace -o bench "
             "-- python3 -u bench.py --steps 5 --warmup 1 --no-cpu-baseline --headline-only")
PMC_CMD = ("timeout -s KILL 120 rocprofv3 --pmc {c} --output-format csv -d gpurun_out/pmc_{d} "
           "-o pmc -- python3 -u bench.py --profile-pass")


def summarize(trace_dir, fetch_dir, write_dir):
    """Write the short rocprofv3 summaries under profiles/ from the CSV output of
    the trace run and the two counter passes (commands in TRACE_CMD, PMC_CMD)."""
    import csv

    import numpy as np

    def rows(path):
        with open(path) as f:
            return list(csv.DictReader(f))

    def agent(d):
        try:
            for r in rows(os.path.join(d, [f for f in os.listdir(d) if f.endswith("agent_info.csv")][0])):
                if r.get("Agent_Type", "").upper() == "GPU":
                    return (f'{r.get("Name", "?")}, {r.get("Cu_Count", "?")} CUs, '
                            f'{r.get("Num_Xcc", "?")} XCDs, {r.get("Max_Engine_Clk_Fcompute", "?")} MHz')
        except (OSError, IndexError):
            pass
        return "?"

    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    stats = rows(os.path.join(trace_dir, "bench_kernel_stats.csv"))
    out = [f"# rocprofv3 kernel statistics: bench.py on the Scene 100k x 100k ICP workload",
           f"# command: {TRACE_CMD}",
           f"# device: {agent(trace_dir)}",
           f"# kernels.hip code sha256[:16] (comments, whitespace dropped): {kernel_source_hash()}",
           "",
           f"{'kernel':64s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'time%':>6s}"]
    for r in stats[:14]:
        out.append(f"{r['Name'][:64]:64s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} "
                   f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} "
                   f"{float(r['Percentage']):6.2f}")
    with open(os.path.join(ROOT, "profiles", "icp_fused_kernel_scene100k_trace.txt"), "w") as f:
        f.write("\n".join(out) + "\n")

    def counter(d):
        per = {}
        for r in rows(os.path.join(d, "pmc_counter_collection.csv")):
            per.setdefault(r["Kernel_Name"], []).append((int(r["Grid_Size"]), float(r["Counter_Value"])))
        return per

    copy_kib = COPY_MIB * 1024
    res = {}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = counter(d)
        fused = [v for k, vs in per.items() if "icp_fused_kernel" in k for _, v in vs]
        copies = [v for k, vs in per.items() if "copyBuffer" in k for _, v in vs
                  if v > 0.25 * copy_kib]
        factor = copy_kib / float(np.mean(copies))
        res[name] = (float(np.mean(fused)), len(fused), copies, factor)
    traffic = sum(v * 1024 * fac for v, _, _, fac in res.values())
    out = ["# HBM traffic of icp_fused_kernel<1> on the Scene 100k x 100k ICP workload",
           "# two rocprofv3 counter passes, each over the same short program:",
           "#   " + PMC_CMD.format(c="FETCH_SIZE", d="fetch"),
           "#   " + PMC_CMD.format(c="WRITE_SIZE", d="write"),
           f"# device: {agent(fetch_dir)}",
           "# calibration: three device copies of a known size in the same program;",
           "# factor = copied KiB / counter KiB of those dispatches",
           ""]
    for name, (avg, cnt, copies, fac) in res.items():
        out.append(f"# {name}: fused kernel {avg:.1f} KiB/dispatch over {cnt} dispatches; "
                   f"{COPY_MIB} MiB copies read {', '.join(f'{c:.1f}' for c in copies)} KiB "
                   f"-> factor {fac:.5f}")
    out += ["",
            f"fetch_bytes_per_launch={res['FETCH_SIZE'][0] * 1024 * res['FETCH_SIZE'][3]:.0f}",
            f"write_bytes_per_launch={res['WRITE_SIZE'][0] * 1024 * res['WRITE_SIZE'][3]:.0f}",
            f"traffic_bytes_per_launch={traffic:.0f}",
            f"kernels_hip_sha256_16={kernel_source_hash()}"]
    with open(TRAFFIC_SUMMARY, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


PMC_SETS = {
    "sq1": "SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_INST_ANY SQ_ACTIVE_INST_VALU "
           "SQ_INSTS_VALU SQ_INSTS_VMEM_RD SQ_INST_LEVEL_VMEM",
    "mem": "TCC_HIT_sum TCC_MISS_sum TCC_REQ_sum TCP_PENDING_STALL_CYCLES_sum "
           "TCP_READ_TAGCONFLICT_STALL_CYCLES_sum TCP_TCC_READ_REQ_sum "
           "TCP_TOTAL_CACHE_ACCESSES_sum TA_TA_BUSY_sum TA_ADDR_STALLED_BY_TC_CYCLES_sum "
           "GRBM_GUI_ACTIVE",
    "sq2": "SQ_THREAD_CYCLES_VALU SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_VMEM SQ_INST_CYCLES_VMEM_RD "
           "SQ_WAIT_ANY SQ_CYCLES SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT",
}


def summarize_counters(root):
    """profiles/ summary of the three counter passes (PMC_SETS) over
    `bench.py --profile-pass`, per dispatch of the fused kernel."""
    import csv

    import numpy as np
    val = {}
    for name in PMC_SETS:
        per = {}
        with open(os.path.join(root, f"pmc_{name}", "pmc_counter_collection.csv")) as f:
            for r in csv.DictReader(f):
                if "icp_fused_kernel" in r["Kernel_Name"]:
                    per.setdefault(r["Counter_Name"], {}).setdefault(r["Dispatch_Id"], 0.0)
                    per[r["Counter_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
        for c, d in per.items():
            val[c] = float(np.mean(list(d.values())))
    waves = val["SQ_WAVES"]
    derived = [
        ("L2 hit rate", val["TCC_HIT_sum"] / max(val["TCC_REQ_sum"], 1)),
        ("L1 hit rate (1 - L1->L2 reads / L1 accesses)",
         1 - val["TCP_TCC_READ_REQ_sum"] / max(val["TCP_TOTAL_CACHE_ACCESSES_sum"], 1)),
        ("VALU lane utilisation (thread-cycles / (64 x VALU cycles))",
         val["SQ_THREAD_CYCLES_VALU"] / max(64 * val["SQ_ACTIVE_INST_VALU"], 1)),
        ("VALU instructions per wave", val["SQ_INSTS_VALU"] / waves),
        ("vector-memory read instructions per wave", val["SQ_INSTS_VMEM_RD"] / waves),
        ("LDS instructions per wave", val["SQ_INSTS_LDS"] / waves),
        ("LDS bank conflicts per dispatch", val["SQ_LDS_BANK_CONFLICT"]),
        ("address unit busy (TA busy / (CUs x GPU-active cycles per XCD))",
         val["TA_TA_BUSY_sum"] / (256 * val["GRBM_GUI_ACTIVE"] / 8)),
    ]
    out = ["# rocprofv3 counters of icp_fused_kernel<1>, Scene 100k x 100k, mean per dispatch",
           "# three passes, each: timeout -s KILL 120 rocprofv3 --pmc <set> --output-format csv "
           "-d gpurun_out/pmc_<name> -o pmc -- python3 -u bench.py --profile-pass",
           f"# kernels.hip code sha256[:16] (comments, whitespace dropped): {kernel_source_hash()}", ""]
    for name, cs in PMC_SETS.items():
        out.append(f"# set {name}: {cs}")
    out.append("")
    for c in sorted(val):
        out.append(f"{c:44s} {val[c]:14.6g}")
    out.append("")
    for k, v in derived:
        out.append(f"{k:64s} {v:10.4g}")
    with open(os.path.join(ROOT, "profiles", "icp_fused_kernel_scene100k_counters.txt"), "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


def roofline_micro(torch, kdnn, work_bytes, n, nodes_avg, pts_avg, kern_ms):
    """The library's micro-benchmarks at three working-set sizes: the fused
    kernel's own (box array + points + index map: one XCD's L2), 64 MiB (the
    Infinity Cache) and 512 MiB (HBM).  Random-gather GB/s for records of 16 B
    (a point), 48 B (a child-pair box load) and 256 B (a leaf chunk), 2^20
    lanes x 16 records, best of three seeds; dependent-load latency per hop
    for 64 lanes chasing a random cycle of 64-byte records.  Then the fused
    kernel's floor at its own level: its box-pair, leaf and per-point bytes
    each at the L2 rate for that record shape."""
    sizes = {"l2_working_set": int(work_bytes), "infinity_cache": 64 << 20, "hbm": 512 << 20}
    lanes, rounds = 1 << 20, 16
    out = {}
    for lvl, size in sizes.items():
        size -= size % 4096
        buf = torch.empty(size // 4, dtype=torch.int32, device="cuda")
        e = {"mib": round(size / 2 ** 20, 2)}
        for words in (1, 3, 16):
            kdnn.gather_bench(buf, words, lanes, rounds)
            ms = min(kdnn.gather_bench(buf, words, lanes, rounds, seed=s_) for s_ in (1, 2, 3))
            e[f"gather_gbs_{16 * words}B"] = round(lanes * rounds * words * 16 / (ms * 1e-3) / 1e9, 1)
        nrec = size // 64
        perm = torch.randperm(nrec, device="cuda", dtype=torch.int64)
        nxt = torch.zeros(nrec * 16, dtype=torch.int32, device="cuda")
        nxt[perm * 16] = torch.roll(perm, -1).to(torch.int32)
        steps = 4000
        kdnn.chase_bench(nxt, 1, 200)
        e["latency_ns"] = round(kdnn.chase_bench(nxt, 1, steps) * 1e6 / steps, 1)
        out[lvl] = e
        del buf, perm, nxt
    l2 = out["l2_working_set"]
    t_min = n * (24 * nodes_avg / l2["gather_gbs_48B"] + 16 * pts_avg / l2["gather_gbs_256B"]
                 + 32 / l2["gather_gbs_16B"]) / 1e9
    out["fused_kernel_at_l2"] = {
        "floor_us": round(t_min * 1e6, 2), "measured_us": round(kern_ms * 1e3, 2),
        "frac": round(t_min / (kern_ms * 1e-3), 4),
        "note": "floor = box-pair bytes at the 48 B rate + leaf bytes at the 256 B rate + "
                "source/match bytes at the 16 B rate, all for this working set"}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--kernel-reps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the rejection, leaf/axis sweep, LiDAR batch and voxel sections "
                         "(the kernel trace of the Scene workload alone)")
    ap.add_argument("--profile-pass", action="store_true",
                    help="only: 30 fused launches of the Scene ICP iterations, then a "
                         f"{COPY_MIB} MiB device copy (calibration for HBM counters)")
    ap.add_argument("--summarize", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write the profiles/ summaries from rocprofv3 CSV output and exit")
    ap.add_argument("--summarize-counters", metavar="OUT_DIR",
                    help="write the profiles/ counter summary from gpurun_out/pmc_<set> and exit")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.summarize:
        summarize(*args.summarize)
        return
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
    stream = torch.cuda.current_stream()
    sums = torch.zeros(kdnn.KDNN_SUMS_DOUBLES, dtype=torch.float64, device="cuda")

    if args.profile_pass:
        g = tree.icp(src, max_iter=ITERS, workspace=ws)
        Rt = g["Rt_hist"]
        for k in range(ITERS):
            tree.correspond_reduce_async(src, Rt[k, :9], Rt[k, 9:], sums, ws)
        a = torch.empty(COPY_MIB << 18, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        a.fill_(1.0)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log("profile pass done: icp", ITERS, "iterations +", ITERS, "fused launches +",
            f"3 copies of {COPY_MIB} MiB")
        return

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
    # the same registrations with the iterations kept on the device
    for _ in range(max(args.warmup, 1)):
        gh = tree.icp(src, max_iter=ITERS, workspace=ws, device_loop=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        gh = tree.icp(src, max_iter=ITERS, workspace=ws, device_loop=True)
    torch.cuda.synchronize()
    T_host = time.perf_counter() - t0
    assert gh["iters"] == ITERS
    log(f"device loop: {args.steps * ITERS / T_host:.0f} ICP iterations/s")

    rej, sweep, lid, vox = None, None, None, None
    if not args.headline_only:
        # ---------------------------------- the same registration with rejection
        # (article §4.4: max_dist fused into the search, then 3-sigma residual
        # rejection and a second solve per iteration)
        REJ = {"max_dist": 1.0, "reject_k": 3.0}
        for _ in range(2):
            tree.icp(src, max_iter=ITERS, workspace=ws, **REJ)
        torch.cuda.synchronize()
        rsteps = max(args.steps // 2, 1)
        t0 = time.perf_counter()
        for _ in range(rsteps):
            gr = tree.icp(src, max_iter=ITERS, workspace=ws, **REJ)
        torch.cuda.synchronize()
        Tr = time.perf_counter() - t0
        rej = {"max_dist_m": REJ["max_dist"], "reject_k": REJ["reject_k"], "steps": rsteps,
               "icp_iters_per_s": round(rsteps * ITERS / Tr, 1),
               "icp_iter_us": round(Tr / (rsteps * ITERS) * 1e6, 2),
               "queries_per_s": round(rsteps * ITERS * n / Tr)}
        log(f"with rejection: {rej['icp_iters_per_s']:.0f} ICP iterations/s")

        # ------------------ builder variants: leaf size and split-axis rule sweep
        # (article §4.1 leaf table, §4.2 max-variance vs round-robin axis)
        log("leaf / axis sweep on the Scene target")
        q_it0 = src
        sweep = []
        for rr in (False, True):
            for leaf in (1, 4, 8, 16, 32, 64):
                tr = kdnn.Tree(p.target, leaf, round_robin=rr)
                inf_ = tr.info
                out_ = (torch.empty(n, dtype=torch.int32, device="cuda"),
                        torch.empty(n, dtype=torch.float32, device="cuda"))
                qw = tr.query_workspace(n)
                tr.query(q_it0, out=out_, workspace=qw)
                ts = []
                for _ in range(10):
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    tr.query(q_it0, out=out_, workspace=qw)
                    e1.record(stream)
                    ts.append((e0, e1))
                _, _, cn_, cp_ = tr.query_stats(q_it0)
                torch.cuda.synchronize()
                iw = tr.icp_workspace(n)
                tr.icp(src, max_iter=ITERS, workspace=iw)
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for _ in range(3):
                    tr.icp(src, max_iter=ITERS, workspace=iw)
                torch.cuda.synchronize()
                icp_us = (time.perf_counter() - t0) / (3 * ITERS) * 1e6
                sweep.append({
                    "axis": "round_robin" if rr else "max_variance", "leaf": leaf,
                    "depth": inf_["depth"], "host_build_ms": round(inf_["build_ms"], 2),
                    "device_mb": round(inf_["device_bytes"] / 2**20, 2),
                    "nn_query_us": round(float(np.median([a.elapsed_time(b) for a, b in ts])) * 1e3, 1),
                    "nodes_per_query": round(float(cn_.float().mean()), 2),
                    "points_per_query": round(float(cp_.float().mean()), 2),
                    "icp_iter_us": round(icp_us, 1)})
                del tr
        log("sweep:", [(r["axis"][0], r["leaf"], r["nn_query_us"]) for r in sweep])

        # ----------------------- LiDAR frame pairs: batched vs one after another
        # (article §3.4: consecutive frames in flight together)
        log("LiDAR: 16 frame pairs, 30 iterations each")
        lp = synth.lidar_pairs()
        ltrees = [kdnn.Tree(q.target, q.leaf_size) for q in lp]
        lsrc = [torch.from_numpy(np.ascontiguousarray(q.source)).cuda() for q in lp]
        bws = kdnn.icp_batch_workspace([len(x) for x in lsrc])
        lws = [t_.icp_workspace(len(x)) for t_, x in zip(ltrees, lsrc)]

        def run_batch():
            return kdnn.icp_batch(ltrees, lsrc, max_iter=ITERS, workspace=bws)

        def run_seq():
            return [t_.icp(x, max_iter=ITERS, workspace=w_, sort=False)
                    for t_, x, w_ in zip(ltrees, lsrc, lws)]

        lid = {"pairs": len(lp), "points_per_frame": int(np.mean([len(x) for x in lsrc])),
               "iterations": ITERS}
        for name, fn in (("batched", run_batch), ("sequential", run_seq)):
            fn()
            torch.cuda.synchronize()
            reps = 5
            t0 = time.perf_counter()
            for _ in range(reps):
                fn()
            torch.cuda.synchronize()
            T_ = (time.perf_counter() - t0) / reps
            q_ = sum(len(x) for x in lsrc) * ITERS
            lid[name] = {"ms_per_16_pairs": round(T_ * 1e3, 3), "pairs_per_s": round(len(lp) / T_, 1),
                         "icp_iters_per_s": round(len(lp) * ITERS / T_, 1),
                         "queries_per_s": round(q_ / T_)}
        lid["speedup"] = round(lid["sequential"]["ms_per_16_pairs"] / lid["batched"]["ms_per_16_pairs"], 2)
        log(f"LiDAR batched {lid['batched']['pairs_per_s']} pairs/s, "
            f"sequential {lid['sequential']['pairs_per_s']} pairs/s")

        # ------------------------------- voxel-grid down-sampling (article §4.3)
        # ~1M points: the first 8 LiDAR frames stacked (each in its own sensor
        # frame), filtered at 0.2 m (the article's outdoor range 0.2-0.5 m)
        vox_in = torch.cat(lsrc[:8]).contiguous()
        vws = torch.empty(int(kdnn._lib.lib().voxel_downsample_workspace_bytes(len(vox_in))),
                          dtype=torch.uint8, device="cuda")
        vox = {"input_points": int(len(vox_in)), "leaf_m": 0.2}
        vout = kdnn.voxel_downsample(vox_in, 0.2, workspace=vws)
        torch.cuda.synchronize()
        reps = 10
        t0 = time.perf_counter()
        for _ in range(reps):
            vout = kdnn.voxel_downsample(vox_in, 0.2, workspace=vws)
        torch.cuda.synchronize()
        Tv = (time.perf_counter() - t0) / reps
        vox.update({"voxels": int(len(vout)), "ms": round(Tv * 1e3, 3),
                    "points_per_s": round(len(vox_in) / Tv),
                    "note": "wall time of the synchronous call (two host round trips included)"})
        log(f"voxel filter: {vox['input_points']} -> {vox['voxels']} in {vox['ms']} ms")

    # ------------------------------------------- fused kernel: events per launch
    # The library launches on torch's current stream.  Its timing facility
    # records a HIP event pair around the search kernel of each launch; torch
    # events around each call time the whole call (search kernel + the
    # one-group reduction).  A spin kernel queued ahead of every 30 launches
    # keeps the GPU from running dry while the host enqueues them, so that the
    # events time the kernels and not the host.
    Rt = g["Rt_hist"]
    tree.correspond_reduce_async(src, Rt[0, :9], Rt[0, 9:], sums, ws)   # order, if any
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1 << 20)
    c0.record(stream)
    torch.cuda._sleep(1 << 24)
    c1.record(stream)
    torch.cuda.synchronize()
    spin_cycles = int((1 << 24) * 25.0 / max(c0.elapsed_time(c1), 1e-3))   # ~25 ms
    Rts = [(Rt[k, :9].copy(), Rt[k, 9:].copy()) for k in range(ITERS)]
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.kernel_reps * ITERS)]
    # pass 1: whole calls (torch events); pass 2: the search kernel alone
    # (library events, which add their own markers between the two kernels)
    for r in range(args.kernel_reps):
        torch.cuda._sleep(spin_cycles)
        for k in range(ITERS):
            e0, e1 = evs[r * ITERS + k]
            e0.record(stream)
            tree.correspond_reduce_async(src, Rts[k][0], Rts[k][1], sums, ws,
                                         flags=kdnn.KDNN_ICP_REUSE_ORDER)
            e1.record(stream)
    torch.cuda.synchronize()
    call_ms = np.array([a.elapsed_time(b) for a, b in evs])
    kdnn.timing_begin(args.kernel_reps * ITERS)
    for r in range(args.kernel_reps):
        torch.cuda._sleep(spin_cycles)
        for k in range(ITERS):
            tree.correspond_reduce_async(src, Rts[k][0], Rts[k][1], sums, ws,
                                         flags=kdnn.KDNN_ICP_REUSE_ORDER)
    torch.cuda.synchronize()
    kern_ms = kdnn.timing_end().astype(np.float64)
    assert len(kern_ms) == args.kernel_reps * ITERS
    kern_avg_ms = float(kern_ms.mean())
    log(f"fused kernel: mean {kern_avg_ms * 1e3:.1f} us, median {np.median(kern_ms) * 1e3:.1f} us;"
        f" whole call mean {call_ms.mean() * 1e3:.1f} us")

    # host rigid solve alone (what each iteration does between two launches)
    sd = tree.correspond_reduce(src, Rt[0, :9], Rt[0, 9:], workspace=ws)
    t0 = time.perf_counter()
    for _ in range(200):
        kdnn.procrustes(sd)
    solve_us = (time.perf_counter() - t0) / 200 * 1e6

    # algorithmic bytes of one launch, per iteration's transform
    nodes_tot, pts_tot = [], []
    for k in range(ITERS):
        q = kdnn.transform(src, Rt[k, :9], Rt[k, 9:])
        _, _, cn, cp = tree.query_stats(q)
        nodes_tot.append(int(cn.sum()))
        pts_tot.append(int(cp.sum()))
    nodes_avg = float(np.mean(nodes_tot)) / n
    pts_avg = float(np.mean(pts_tot)) / n
    # per source point: the box of every node record the search reads (24 B),
    # every leaf point scanned (16 B: x, y, z, original index), the source point
    # (12 B), its matched target point and that point's slot (16 + 4 B), and its
    # slot in the traversal order when ordered (4 B).  The 136 B of partial sums
    # each work-group writes are left out (< 0.1%).
    per_query = (24 * nodes_avg + 16 * pts_avg + 12 + 20
                 + (4 if info["auto_sort_icp"] else 0))
    bytes_launch = n * per_query
    achieved = bytes_launch / (kern_avg_ms * 1e-3) / 1e9
    # one descent to a leaf and nothing else: the root box, both children's
    # boxes at each of D levels, one leaf's points, the source and its match
    descent_lb = 24 * (2 * info["depth"] + 1) + 16 * (n / 2 ** info["depth"]) + 32

    # ------------------------------------------------------ standalone nn_query
    def time_query(tr, q, sort, reps=100, warm=10):
        """Device time of nn_query (events on the launch stream): median, p25, p75 in ms."""
        qws = tr.query_workspace(len(q))
        out = (torch.empty(len(q), dtype=torch.int32, device="cuda"),
               torch.empty(len(q), dtype=torch.float32, device="cuda"))
        for _ in range(warm):
            tr.query(q, sort=sort, out=out, workspace=qws)
        evs_ = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(reps)]
        torch.cuda._sleep(spin_cycles)
        for e0, e1 in evs_:
            e0.record(stream)
            tr.query(q, sort=sort, out=out, workspace=qws)
            e1.record(stream)
        torch.cuda.synchronize()
        t_ = np.array([a.elapsed_time(b) for a, b in evs_])
        return float(np.median(t_)), float(np.percentile(t_, 25)), float(np.percentile(t_, 75))

    def nn_entry(m_, ms):
        return {"ms": round(ms[0], 4), "p25_ms": round(ms[1], 4), "p75_ms": round(ms[2], 4),
                "queries_per_s": round(m_ / (ms[0] * 1e-3))}

    q0 = src
    qc = kdnn.transform(src, g["R"], g["t"])
    nnq = {"automatic_order": "morton" if info["auto_sort"] else "unsorted",
           "runs": "median and quartiles of 100 launches after 10 warm-ups"}
    for name, q in (("iteration0", q0), ("converged", qc)):
        for sort in (True, False):
            nnq[f"{name}_{'morton' if sort else 'unsorted'}"] = nn_entry(
                len(q), time_query(tree, q, sort))
    log("nn_query:", nnq)

    # the other query workloads (one nn_query pass each, the library's automatic order)
    other = {}
    if not args.headline_only:
        for wname, gen, leaf in (("stress_1M_leaf8", synth.stress, 8),
                                 ("stress_1M_leaf16", synth.stress, 16),
                                 ("skewed_500k_leaf8", synth.skewed, 8),
                                 ("skewed_500k_leaf16", synth.skewed, 16)):
            pw = gen()
            tw = kdnn.Tree(pw.target, leaf)
            qw = torch.from_numpy(np.ascontiguousarray(pw.source)).cuda()
            other[wname] = dict(nn_entry(len(qw), time_query(tw, qw, None, reps=20, warm=3)),
                                automatic_order="morton" if tw.info["auto_sort"] else "unsorted",
                                build_ms=round(tw.info["build_ms"], 1))
            del tw, qw
        log("other workloads:", other)
    micro = None
    if not args.headline_only:
        work = 24 * 2 ** (info["depth"] + 1) + 16 * (len(p.target) + 16) + 4 * len(p.target)
        micro = roofline_micro(torch, kdnn, work, n, nodes_avg, pts_avg, kern_avg_ms)
        log("roofline micro-benchmarks:", micro)
    traffic, traffic_src = committed_traffic()

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
        "icp_with_rejection": rej,
        "lidar_pairs": lid,
        "leaf_axis_sweep": sweep,
        "voxel_downsample": vox,
        "icp_iter_us": round(T / (args.steps * ITERS) * 1e6, 2),
        "build": {"host_build_ms": round(info["build_ms"], 3),
                  "upload_ms": round(info["upload_ms"], 3),
                  "wall_ms": round(build_wall_ms, 3),
                  "registration_incl_build_ms": round(build_wall_ms + T / args.steps * 1e3, 3)},
        "fused_kernel": {"name": "icp_fused_kernel", "mean_us": round(kern_avg_ms * 1e3, 2),
                         "median_us": round(float(np.median(kern_ms)) * 1e3, 2),
                         "p25_us": round(float(np.percentile(kern_ms, 25)) * 1e3, 2),
                         "p75_us": round(float(np.percentile(kern_ms, 75)) * 1e3, 2),
                         "launches": len(kern_ms),
                         "queries_per_s": round(n / (kern_avg_ms * 1e-3)),
                         "timing": "event pair stamped by the search kernel's dispatch "
                                   "(library timing facility, hipExtLaunchKernel)"},
        "icp_host_loop": {"icp_iters_per_s": round(args.steps * ITERS / T_host, 1),
                          "icp_iter_us": round(T_host / (args.steps * ITERS) * 1e6, 2),
                          "queries_per_s": round(args.steps * ITERS * n / T_host),
                          "R_diff_vs_device_loop": float(np.linalg.norm(gh["R"] - g["R"]))},
        "icp_iteration_breakdown_us": {
            "iteration": round(T / (args.steps * ITERS) * 1e6, 2),
            "of_which_fused_kernel": round(kern_avg_ms * 1e3, 2),
            "device_loop_rest": round(T / (args.steps * ITERS) * 1e6 - kern_avg_ms * 1e3, 2),
            "host_loop_iteration": round(T_host / (args.steps * ITERS) * 1e6, 2),
            "host_loop_correspondence_call_events": round(float(call_ms.mean()) * 1e3, 2),
            "host_solve_through_python": round(solve_us, 2),
            "note": "device loop (the headline): per iteration the fused kernel, then one "
                    "work-group that sums the partials, solves and leaves the next transform "
                    "on the device; device_loop_rest = that step kernel and the two launch "
                    "gaps.  Host loop: host_loop_correspondence_call_events = the search "
                    "kernel, the one-group reduction into pinned memory and the gap between "
                    "them; the rest of its iteration is the readback wait, host solve and "
                    "next launch.  host_solve_through_python times kdnn_procrustes called "
                    "from Python (ctypes marshalling included): an upper bound of the C++ call"},
        "nn_query": nnq,
        "other_workloads_nn_query": other,
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None if traffic is None else round(traffic),
            "traffic_source": traffic_src,
            "kernel": "icp_fused_kernel<1>",
            "kernels_hip_sha256_16": kernel_source_hash(),
            "bytes_per_launch": round(bytes_launch),
            "bytes_per_query": round(per_query, 1),
            "nodes_per_query": round(nodes_avg, 2), "points_per_query": round(pts_avg, 2),
            "single_descent_bytes_per_query": round(descent_lb, 1),
            "tree_device_bytes": info["device_bytes"], "l2_bytes": info["l2_bytes"],
            "note": "the tree fits one XCD's L2: algorithmic gather bytes vs HBM peak; "
                    "traffic = HBM bytes the counters saw per launch",
            "measured_levels": micro,
        },
    }

    if not args.no_cpu_baseline:
        import oracle
        log("cpu baseline: oracle ICP registrations (30 iterations each), 1 thread, >= 10 s")
        regs, Tc = 0, 0.0
        while Tc < 10.0 and regs < 6:
            t0 = time.perf_counter()
            o = oracle.icp(p.target, p.source, ITERS, leaf_size=p.leaf_size)
            Tc += time.perf_counter() - t0
            regs += 1
        result["cpu_baseline"] = {
            "value": round(regs * ITERS * n / Tc), "unit": "queries/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{regs} full Scene registrations (30 ICP iterations x 100k queries each) "
                      "with the oracle's C KD-tree search and numpy fp64 reduction/Horn "
                      f"solve, {Tc:.2f} s wall",
            "icp_iters_per_s": round(regs * ITERS / Tc, 2),
            "R_diff_vs_gpu": float(np.linalg.norm(o["R"] - g["R"])),
        }
        log(f"cpu baseline {regs * ITERS * n / Tc / 1e6:.2f} M queries/s")
        # context: the oracle's KD-tree query of one iteration's queries on every
        # host core (threads over query chunks; the C query holds no global
        # state and ctypes releases the GIL), and its brute force on a sample
        import concurrent.futures as cf
        threads = max(1, min(16, len(os.sched_getaffinity(0))))
        otree = oracle.KDTree(p.target, p.leaf_size)
        chunks = np.array_split(p.source, threads * 4)
        t0 = time.perf_counter()
        otree.query(p.source)
        Tq1 = time.perf_counter() - t0
        with cf.ThreadPoolExecutor(threads) as ex:
            list(ex.map(otree.query, chunks[:threads]))  # warm
            t0 = time.perf_counter()
            list(ex.map(otree.query, chunks))
            Tq = time.perf_counter() - t0
        ns = 2000
        t0 = time.perf_counter()
        oracle.brute_nn(p.target, p.source[:ns])
        Tb = time.perf_counter() - t0
        result["cpu_context"] = {
            "oracle_kd_nn_queries_per_s_all_cores": round(n / Tq),
            "threads": threads,
            "oracle_kd_nn_queries_per_s_1_thread": round(n / Tq1),
            "brute_force_pairs_per_s_1_thread": round(ns * len(p.target) / Tb),
            "brute_force_one_scene_iteration_s": round(Tb * n / ns, 1),
            "note": "context only: the oracle's own KD search of one Scene iteration's "
                    "100k queries split over host threads; brute force timed on 2,000 "
                    "queries and scaled to 100k x 100k pairs"}
        log(f"cpu context: {n / Tq / 1e6:.2f} M queries/s on {threads} threads, brute force "
            f"{Tb * n / ns:.1f} s per Scene iteration")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
