#!/usr/bin/env python3
"""NN queries/s and ICP iterations/s at 100k x 100k points on one MI355X.

Workload (seeded, synthetic): the Scene pair -- 100k-point target sampled on a
ground disk, 20 boxes and 10 spheres (density ~ 1/r^2, 1 cm noise); source = an
independent 100k resample moved by 10 degrees of yaw and 0.5 m; leaf 16.

One step = one ICP registration of 30 iterations as the library runs it by
default: per iteration the fused kernel (transform, exact NN of all 100k
source points, fp64 reduction to 17 sums), a 136-byte readback, the SVD solve
with the det sign fix and the convergence check on the host -- with the tree
already built and both clouds resident in device memory.  value = NN
queries/s over the timed steps (30 x 100k queries per step); icp_iters_per_s
is the same clock.  The same registrations with the iterations kept on the
device (KDNN_ICP_DEVICE_LOOP) are reported beside it.

Also reported: the fused kernel's duration (the library's event pair stamped
by the kernel's own dispatch, on the stream it is launched on) and its
roofline -- the algorithmic bytes of the search (node records, leaf points,
index, query, source and match, counted by the instrumented traversal) against
the random-gather ceiling of the memory level holding the tree, measured by
the library's micro-benchmark, with the 8 TB/s HBM peak as context; HBM
traffic from the committed rocprofv3 counter summary when it was taken on the
current kernel source; the other workloads' nn_query rooflines; the CPU
oracle on the host cores.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--only SECTION]
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
ITERS = 30
QUERY_WORKLOADS = ("stress_1M_leaf8", "stress_1M_leaf16", "skewed_500k_leaf8",
                   "skewed_500k_leaf16")
SECTIONS = ("scene", "reject", "sweep", "lidar", "voxel", "recipe") + QUERY_WORKLOADS


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


def pct(a):
    import numpy as np
    a = np.asarray(a, dtype=np.float64)
    return {"median": float(np.median(a)), "p25": float(np.percentile(a, 25)),
            "p75": float(np.percentile(a, 75)), "mean": float(a.mean()), "n": int(len(a))}


# --------------------------------------------------------------- profiles/
TRACE_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/trace_{only} "
             "-o bench -- python3 -u bench.py --steps 20 --warmup 3 --no-cpu-baseline "
             "--only {only} --json-out gpurun_out/trace_{only}/bench.json")
PMC_CMD = ("timeout -s KILL 120 rocprofv3 --pmc {c} --output-format csv -d gpurun_out/pmc_{d} "
           "-o pmc -- python3 -u bench.py --profile-pass")


def _rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _agent(d):
    try:
        for r in _rows(os.path.join(d, [f for f in os.listdir(d) if f.endswith("agent_info.csv")][0])):
            if r.get("Agent_Type", "").upper() == "GPU":
                return (f'{r.get("Name", "?")}, {r.get("Cu_Count", "?")} CUs, '
                        f'{r.get("Num_Xcc", "?")} XCDs, {r.get("Max_Engine_Clk_Fcompute", "?")} MHz')
    except (OSError, IndexError):
        pass
    return "?"


def summarize_trace(trace_dir, only, out_name):
    """profiles/<out_name>: rocprofv3 kernel statistics of `bench.py --only
    <only>` (TRACE_CMD) and that same run's bench line, from which its
    roofline figures are computed."""
    stats = _rows(os.path.join(trace_dir, "bench_kernel_stats.csv"))
    out = [f"# rocprofv3 kernel statistics of bench.py --only {only}",
           f"# command: {TRACE_CMD.format(only=only)}",
           f"# device: {_agent(trace_dir)}",
           f"# kernels.hip code sha256[:16] (comments, whitespace dropped): {kernel_source_hash()}",
           "",
           "# (torch's spin_kernel, which bench.py queues ahead of timed regions so that the",
           "#  host's launches run ahead of the device, is left out; time% is of the rest)",
           "",
           f"{'kernel':72s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'time%':>6s}"]
    stats = [r for r in stats if "spin_kernel" not in r["Name"]]
    total = sum(float(r["TotalDurationNs"]) for r in stats) or 1.0
    for r in stats[:24]:
        r["Percentage"] = 100.0 * float(r["TotalDurationNs"]) / total
        out.append(f"{r['Name'][:72]:72s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} "
                   f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} "
                   f"{float(r['Percentage']):6.2f}")
    # the bench's event-timed batches: the dispatches queued behind a spin
    # kernel, up to the next spin kernel or the first idle gap of 200 us (the
    # batch's closing synchronisation) -- the launches whose event pairs give
    # the bench line's kernel times (under the profiler those events read higher)
    try:
        trace = sorted(_rows(os.path.join(trace_dir, "bench_kernel_trace.csv")),
                       key=lambda r: int(r["Start_Timestamp"]))
        per, last_end = {}, None
        for r in trace:
            t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
            if "spin_kernel" in r["Kernel_Name"]:
                last_end = t1
                continue
            if last_end is not None and t0 - last_end < 200000:
                per.setdefault(r["Kernel_Name"], []).append((t1 - t0) / 1e3)
                last_end = t1
            else:
                last_end = None
        if per:
            out += ["", "# dispatches queued behind a spin kernel (the event-timed batches):",
                    f"{'kernel':72s} {'calls':>6s} {'avg_us':>9s} {'median':>9s}"]
            for name, ds in sorted(per.items(), key=lambda kv: -sum(kv[1]))[:8]:
                ds = sorted(ds)
                out.append(f"{name[:72]:72s} {len(ds):6d} {sum(ds) / len(ds):9.2f} "
                           f"{ds[len(ds) // 2]:9.2f}")
        # the fused launches of ICP registrations (runs of fused launches with
        # only their reductions or step kernels between them, not behind a
        # spin kernel, cut at every loop start): iteration 0 searches from the
        # root, iterations 1.. start at the leaf of the previous match
        runs, cur, spun = [], [], False
        for r in trace:
            name = r["Kernel_Name"]
            d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            if "icp_fused_kernel" in name:
                cur.append(d)
            elif "reduce_partials" in name or "icp_loop_step" in name:
                continue
            else:
                if cur and not spun:
                    runs.append(cur)
                cur, spun = [], "spin_kernel" in name
        if cur and not spun:
            runs.append(cur)
        it0 = [x for run in runs if len(run) % ITERS == 0 for x in run[0::ITERS]]
        warm = [x for run in runs if len(run) % ITERS == 0
                for j, x in enumerate(run) if j % ITERS]
        if it0 and warm:
            out += ["", f"# icp_fused_kernel inside {len(it0)} ICP registrations of {ITERS} "
                        "iterations (runs of fused launches with only their reductions or "
                        "step kernels between them):",
                    f"iteration 0 (no start leaf: point location): {len(it0)} launches, avg "
                    f"{sum(it0) / len(it0):.2f} us",
                    f"iterations 1..{ITERS - 1} (warm start): {len(warm)} launches, avg "
                    f"{sum(warm) / len(warm):.2f} us, median {sorted(warm)[len(warm) // 2]:.2f} us"]
    except (OSError, KeyError, ValueError):
        pass
    try:
        with open(os.path.join(trace_dir, "bench.json")) as f:
            line = json.load(f)
        out += ["", "# the same run's bench line:", json.dumps(line, indent=1, sort_keys=True)]
    except OSError:
        pass
    with open(os.path.join(ROOT, "profiles", out_name), "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out[:34]))


PROFILE_REGS = 2  # registrations in the profile pass


def fused_dispatch_groups(rows):
    """Dispatch ids of the profile pass's fused launches, in order: (warm --
    the registrations' iterations after the first, iteration 0s, cold entry
    point launches)."""
    ids = sorted({int(r["Dispatch_Id"]) for r in rows if "icp_fused_kernel" in r["Kernel_Name"]})
    reg = ids[:PROFILE_REGS * ITERS]
    warm = {d for j, d in enumerate(reg) if j % ITERS}
    first = {d for j, d in enumerate(reg) if j % ITERS == 0}
    return warm, first, set(ids[PROFILE_REGS * ITERS:])


def summarize(fetch_dir, write_dir):
    """profiles/ traffic summary of the fused kernel from the two counter
    passes (PMC_CMD, FETCH_SIZE then WRITE_SIZE), each scaled by what the same
    counter reads for device copies of a known size in the same program."""
    import numpy as np

    copy_kib = COPY_MIB * 1024
    res, cold = {}, {}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _rows(os.path.join(d, "pmc_counter_collection.csv"))
        warm_ids, _, cold_ids = fused_dispatch_groups(rows)
        per = {}
        for r in rows:
            if "icp_fused_kernel" in r["Kernel_Name"]:
                per[int(r["Dispatch_Id"])] = per.get(int(r["Dispatch_Id"]), 0.0) + \
                    float(r["Counter_Value"])
        fused = [v for k, v in per.items() if k in warm_ids]
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]
                  and float(r["Counter_Value"]) > 0.25 * copy_kib]
        factor = copy_kib / float(np.mean(copies))
        res[name] = (float(np.mean(fused)), len(fused), copies, factor)
        cold[name] = float(np.mean([v for k, v in per.items() if k in cold_ids])) * 1024 * factor
    traffic = sum(v * 1024 * fac for v, _, _, fac in res.values())
    out = ["# HBM traffic of icp_fused_kernel<1> on the Scene 100k x 100k ICP workload, as the",
           f"# ICP loop runs it: the warm-started launches (iterations 1..{ITERS - 1}) of "
           f"{PROFILE_REGS} registrations",
           "# two rocprofv3 counter passes, each over the same short program:",
           "#   " + PMC_CMD.format(c="FETCH_SIZE", d="fetch"),
           "#   " + PMC_CMD.format(c="WRITE_SIZE", d="write"),
           f"# device: {_agent(fetch_dir)}",
           "# calibration: three device copies of a known size in the same program;",
           "# factor = copied KiB / counter KiB of those dispatches",
           ""]
    for name, (avg, cnt, copies, fac) in res.items():
        out.append(f"# {name}: warm fused kernel {avg:.1f} KiB/dispatch over {cnt} dispatches; "
                   f"{COPY_MIB} MiB copies read {', '.join(f'{c:.1f}' for c in copies)} KiB "
                   f"-> factor {fac:.5f}")
    out += ["",
            f"fetch_bytes_per_launch={res['FETCH_SIZE'][0] * 1024 * res['FETCH_SIZE'][3]:.0f}",
            f"write_bytes_per_launch={res['WRITE_SIZE'][0] * 1024 * res['WRITE_SIZE'][3]:.0f}",
            f"traffic_bytes_per_launch={traffic:.0f}",
            f"kernels_hip_sha256_16={kernel_source_hash()}",
            "",
            "# context: the cold entry point (icp_correspond_reduce_async, no start leaf: point "
            f"location, then the walk): fetch {cold['FETCH_SIZE']:.0f}, write "
            f"{cold['WRITE_SIZE']:.0f} bytes per launch"]
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


def summarize_counters(root, kernel="icp_fused_kernel", out_name=None, title=None, cmd=None):
    """profiles/ summary of the three counter passes (PMC_SETS) over
    `bench.py --profile-pass` (or the command given), per dispatch of the
    kernels whose name contains `kernel`."""
    import numpy as np
    val = {}
    for name in PMC_SETS:
        per = {}
        rows = _rows(os.path.join(root, f"pmc_{name}", "pmc_counter_collection.csv"))
        # the profile pass: the warm-started launches of its registrations only
        keep = fused_dispatch_groups(rows)[0] if cmd is None else None
        for r in rows:
            if kernel in r["Kernel_Name"] and (keep is None or int(r["Dispatch_Id"]) in keep):
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
    cmd = cmd or "python3 -u bench.py --profile-pass"
    out = [f"# rocprofv3 counters of {title or 'icp_fused_kernel<1>, Scene 100k x 100k, warm-started launches of the ICP loop'}, "
           "mean per dispatch",
           "# three passes, each: timeout -s KILL 120 rocprofv3 --pmc <set> --output-format csv "
           f"-d {root}/pmc_<name> -o pmc -- {cmd}",
           f"# kernels.hip code sha256[:16] (comments, whitespace dropped): {kernel_source_hash()}", ""]
    for name, cs in PMC_SETS.items():
        out.append(f"# set {name}: {cs}")
    out.append("")
    for c in sorted(val):
        out.append(f"{c:44s} {val[c]:14.6g}")
    out.append("")
    for k, v in derived:
        out.append(f"{k:64s} {v:10.4g}")
    with open(os.path.join(ROOT, "profiles", out_name or "icp_fused_kernel_scene100k_counters.txt"),
              "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


# ------------------------------------------------------------ measurement
class Gpu:
    """torch, the library, the launch stream and a calibrated spin length."""

    def __init__(self):
        import torch

        import kd_tree_nn_amd as kdnn
        assert torch.cuda.is_available(), "bench needs a HIP device"
        torch.cuda.set_device(0)
        self.torch, self.kdnn = torch, kdnn
        self.stream = torch.cuda.current_stream()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1 << 20)
        c0.record(self.stream)
        torch.cuda._sleep(1 << 24)
        c1.record(self.stream)
        torch.cuda.synchronize()
        # a spin kernel of ~25 ms queued before a batch of launches keeps the GPU
        # from running dry while the host enqueues them
        self.spin = int((1 << 24) * 25.0 / max(c0.elapsed_time(c1), 1e-3))

    def dev(self, a):
        import numpy as np
        return self.torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()

    def events(self, k):
        E = self.torch.cuda.Event
        return [(E(enable_timing=True), E(enable_timing=True)) for _ in range(k)]


def gather_ceilings(g, size_bytes):
    """The library's micro-benchmarks at one working-set size: random-gather
    GB/s for records of 16 B (a point), 48 B (a child-pair box run) and 256 B
    (a leaf chunk), 2^20 lanes x 16 records, best of three seeds; and the
    dependent-load latency of 64 lanes chasing a random cycle of 64-B records."""
    torch, kdnn = g.torch, g.kdnn
    size = max(int(size_bytes) - int(size_bytes) % 4096, 1 << 16)
    lanes, rounds = 1 << 20, 16
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
    return e


def level_of(bytes_, l2_bytes):
    return "l2" if bytes_ <= l2_bytes else ("infinity_cache" if bytes_ <= (256 << 20) else "hbm")


def search_roofline(n, nodes_avg, pts_avg, per_query_fixed, kern_s, ceil, level, what,
                    replay_s, replay_info):
    """Roofline of one search launch of n queries.

    Algorithmic bytes per query, as the path's byte model counts them: 32 B
    per node record visited, 12 B per leaf point scanned, plus the fixed
    per-query bytes (index read, query, and -- fused -- original source and
    matched point, or -- nn_query -- the two outputs).

    Peak: the replay ceiling (kdnn_replay_bench) -- the time the memory system
    takes to deliver exactly the records this launch's queries visit, in the
    launch's own work-groups, waves and XCDs, step by step across each wave's
    queries, with the dependencies removed -- plus the fixed bytes at the
    measured 16-B random-gather rate; peak = bytes / that time and frac =
    achieved / peak = that time / kernel time.  A uniform random gather over
    the working set (`random_gather`, context) misses what the tree's hot top
    levels and neighbouring queries get from L1 and L2, and under-rates
    launches whose queries share records (its fraction exceeds 1 there)."""
    b_nodes, b_pts = 32.0 * nodes_avg, 12.0 * pts_avg
    per_query = b_nodes + b_pts + per_query_fixed
    bytes_launch = n * per_query
    achieved = bytes_launch / kern_s / 1e9
    t_fixed = n * per_query_fixed / ceil["gather_gbs_16B"] / 1e9
    t_gather = n * (b_nodes / ceil["gather_gbs_48B"] + b_pts / ceil["gather_gbs_256B"]) / 1e9 \
        + t_fixed
    t_floor = replay_s + t_fixed
    peak = bytes_launch / t_floor / 1e9
    g_peak = bytes_launch / t_gather / 1e9
    ri = replay_info
    return {
        "bound": level, "achieved": round(achieved, 1), "peak": round(peak, 1), "unit": "GB/s",
        "frac": round(achieved / peak, 4),
        "peak_source": "replay of the launch's own record stream without dependencies "
                       "(kdnn_replay_bench) + fixed bytes at the 16-B random-gather rate",
        "hbm_context": {"peak": HBM_PEAK_GBS, "frac": round(achieved / HBM_PEAK_GBS, 4)},
        "bytes_per_launch": round(bytes_launch), "bytes_per_query": round(per_query, 2),
        "nodes_per_query": round(nodes_avg, 3), "points_per_query": round(pts_avg, 3),
        "fixed_bytes_per_query": per_query_fixed,
        "kernel_us": round(kern_s * 1e6, 3), "floor_us": round(t_floor * 1e6, 3),
        "replay": {"us": round(replay_s * 1e6, 3), "bytes_loaded": ri["bytes"],
                   "gbs_loaded": round(ri["bytes"] / replay_s / 1e9, 1),
                   "visits": ri["visits"], "truncated_queries": ri["truncated"],
                   "launch": {"blocks": ri["blocks"], "queries_per_wave": ri["queries_per_wave"],
                              "spread": bool(ri["spread"])}},
        "random_gather": {"peak": round(g_peak, 1), "frac": round(achieved / g_peak, 4),
                          "floor_us": round(t_gather * 1e6, 3), "ceilings": ceil},
        "byte_model": f"{what}: 32 B x node records + 12 B x leaf points + "
                      f"{per_query_fixed} B per query; node and point counts from the "
                      "instrumented single-lane traversal of the same queries",
    }


def replay_time(tree, q, icp, reps, prev=None):
    """Median replay time (s) of the launch over queries q (warm-started from
    the previous iteration's queries `prev` when given), and what it replayed."""
    import numpy as np
    ms, info = tree.replay_bench(q, icp=icp, reps=reps, prev=prev)
    return float(np.median(ms)) * 1e-3, info


def time_fused(g, tree, src, ws, Rts, reps):
    """The fused kernel at every iteration's transform, `reps` times: its own
    duration (the library's event pair stamped by the search kernel's
    dispatch) and the whole call (torch events: search + one-group reduction)."""
    import numpy as np
    kdnn, torch = g.kdnn, g.torch
    sums = torch.zeros(kdnn.KDNN_SUMS_DOUBLES, dtype=torch.float64, device="cuda")
    tree.correspond_reduce_async(src, Rts[0][0], Rts[0][1], sums, ws)   # order, if any
    evs = g.events(reps * len(Rts))
    for r in range(reps):
        torch.cuda._sleep(g.spin)
        for k, (R, t) in enumerate(Rts):
            e0, e1 = evs[r * len(Rts) + k]
            e0.record(g.stream)
            tree.correspond_reduce_async(src, R, t, sums, ws, flags=kdnn.KDNN_ICP_REUSE_ORDER)
            e1.record(g.stream)
    torch.cuda.synchronize()
    call_ms = np.array([a.elapsed_time(b) for a, b in evs])
    kdnn.timing_begin(reps * len(Rts))
    for r in range(reps):
        torch.cuda._sleep(g.spin)
        for R, t in Rts:
            tree.correspond_reduce_async(src, R, t, sums, ws, flags=kdnn.KDNN_ICP_REUSE_ORDER)
    torch.cuda.synchronize()
    kern_ms = kdnn.timing_end().astype(np.float64)
    assert len(kern_ms) == reps * len(Rts)
    return kern_ms, call_ms


def time_query(g, tr, q, sort, reps=100, warm=10):
    """nn_query: whole calls (torch events on the launch stream: the Morton
    ordering, when applied, and the search) and the search kernel alone (the
    library's event pair), ms."""
    import numpy as np
    torch, kdnn = g.torch, g.kdnn
    qws = tr.query_workspace(len(q))
    out = (torch.empty(len(q), dtype=torch.int32, device="cuda"),
           torch.empty(len(q), dtype=torch.float32, device="cuda"))
    for _ in range(warm):
        tr.query(q, sort=sort, out=out, workspace=qws)
    evs = g.events(reps)
    torch.cuda._sleep(g.spin)
    for e0, e1 in evs:
        e0.record(g.stream)
        tr.query(q, sort=sort, out=out, workspace=qws)
        e1.record(g.stream)
    torch.cuda.synchronize()
    call = np.array([a.elapsed_time(b) for a, b in evs])
    kdnn.timing_begin(reps)
    torch.cuda._sleep(g.spin)
    for _ in range(reps):
        tr.query(q, sort=sort, out=out, workspace=qws)
    torch.cuda.synchronize()
    kern = kdnn.timing_end().astype(np.float64)
    return call, kern


def query_counts(tr, q):
    _, _, cn, cp = tr.query_stats(q)
    return float(cn.double().mean()), float(cp.double().mean())


def timed_steps(g, fn, steps):
    """`steps` calls of fn, each timed on the host (every registration
    synchronises), bracketed by device synchronisations: (total s, per-step s)."""
    import numpy as np
    g.torch.cuda.synchronize()
    per = []
    r = None
    t0 = time.perf_counter()
    for _ in range(steps):
        a = time.perf_counter()
        r = fn()
        per.append(time.perf_counter() - a)
    g.torch.cuda.synchronize()
    return time.perf_counter() - t0, np.array(per), r


def ms_stats(per_s):
    return {k: round(v * 1e3, 4) for k, v in pct(per_s).items() if k != "n"}


# ------------------------------------------------------------------ scene
def bench_scene(g, args, result):
    import numpy as np
    kdnn, torch = g.kdnn, g.torch
    import synth
    log("generating Scene workload")
    p = synth.scene()
    n = len(p.source)
    log("building tree")
    t0 = time.perf_counter()
    tree = kdnn.Tree(p.target, p.leaf_size)
    build_wall_ms = (time.perf_counter() - t0) * 1e3
    # a second build of the same tree: its upload excludes the runtime's
    # one-time start-up, which the first device allocation pays
    tree2 = kdnn.Tree(p.target, p.leaf_size)
    info, info2 = tree.info, tree2.info
    del tree2
    src = g.dev(p.source)
    ws = tree.icp_workspace(n)
    torch.cuda.synchronize()

    log(f"warmup {args.warmup} registrations")
    for _ in range(args.warmup):
        tree.icp(src, max_iter=ITERS, workspace=ws)
    log(f"timing {args.steps} registrations x {ITERS} iterations (host solve per iteration)")
    T, per, r = timed_steps(g, lambda: tree.icp(src, max_iter=ITERS, workspace=ws), args.steps)
    assert r["iters"] == ITERS
    value = args.steps * ITERS * n / T
    log(f"{value / 1e9:.3f} G queries/s, {args.steps * ITERS / T:.0f} ICP iterations/s")
    for _ in range(max(args.warmup, 1)):
        tree.icp(src, max_iter=ITERS, workspace=ws, device_loop=True)
    Td, perd, rd = timed_steps(
        g, lambda: tree.icp(src, max_iter=ITERS, workspace=ws, device_loop=True), args.steps)
    assert rd["iters"] == ITERS
    log(f"device loop: {args.steps * ITERS / Td:.0f} ICP iterations/s")

    Rt = r["Rt_hist"]
    Rts = [(Rt[k, :9].copy(), Rt[k, 9:].copy()) for k in range(ITERS)]
    kern_ms, call_ms = time_fused(g, tree, src, ws, Rts, args.kernel_reps)
    kern_s = float(kern_ms.mean()) * 1e-3
    log(f"fused kernel: mean {kern_s * 1e6:.1f} us, median {np.median(kern_ms) * 1e3:.1f} us; "
        f"whole call mean {call_ms.mean() * 1e3:.1f} us")

    # host SVD solve alone, through the C ABI from Python (an upper bound)
    sd = tree.correspond_reduce(src, Rt[0, :9], Rt[0, 9:], workspace=ws)
    t0 = time.perf_counter()
    for _ in range(500):
        kdnn.procrustes(sd)
    solve_us = (time.perf_counter() - t0) / 500 * 1e6

    # the fused kernel as the ICP loop runs it: the library's event pairs around
    # every fused launch of `kernel_reps` registrations.  Iteration 0 starts
    # each search at the leaf holding its query (point location); iterations
    # 1..29 start at the leaf of each point's previous match (warm start).
    kdnn.timing_begin(ITERS * args.kernel_reps)
    for _ in range(args.kernel_reps):
        tree.icp(src, max_iter=ITERS, workspace=ws)
    torch.cuda.synchronize()
    loop_ms = kdnn.timing_end().astype(np.float64).reshape(args.kernel_reps, ITERS)
    warm_s = float(loop_ms[:, 1:].mean()) * 1e-3
    log(f"fused kernel in the ICP loop: iteration 0 {loop_ms[:, 0].mean() * 1e3:.1f} us, "
        f"iterations 1..{ITERS - 1} {warm_s * 1e6:.1f} us")

    # node records and leaf points per query and the replay ceiling, both for
    # the instrumented single-lane search of each iteration's queries in the
    # fused kernel's launch shape: warm-started from the previous iteration's
    # queries (iterations 1..29; node records then include two for the start
    # leaf's 64-byte plane record), and with no start leaf (all 30, the cold
    # entry point above: point location, then the walk)
    qs = [kdnn.transform(src, R, t) for R, t in Rts]
    wcnt, wrep, ccnt, crep = [], [], [], []
    for k in range(ITERS):
        ccnt.append(query_counts(tree, qs[k]))
        rs, rinfo_c = replay_time(tree, qs[k], True, 5)
        crep.append(rs)
        if k > 0:
            rs, rinfo_w = replay_time(tree, qs[k], True, 5, prev=qs[k - 1])
            wrep.append(rs)
            wcnt.append((rinfo_w["node_records"] / n, rinfo_w["leaf_points"] / n))
    work = 24 * 2 ** (info["depth"] + 1) + 16 * (len(p.target) + 16) + 4 * len(p.target)
    ceil = gather_ceilings(g, work)
    level = level_of(work, info["l2_bytes"])
    # fused: index read 4 + query 12 + original source 12 + matched point 12
    # (+ the warm start's leaf read and write, 4 + 4)
    roof = search_roofline(n, float(np.mean([c[0] for c in wcnt])),
                           float(np.mean([c[1] for c in wcnt])), 4 + 12 + 12 + 12 + 8, warm_s,
                           ceil, level, "fused correspondence kernel, warm-started",
                           float(np.mean(wrep)), rinfo_w)
    roof["replay"]["note"] = (f"mean over iterations 1..{ITERS - 1} of the median of 5 replays "
                              "each, every search starting at the leaf of its query's match in "
                              "the previous iteration; bytes and launch of the last")
    cold = search_roofline(n, float(np.mean([c[0] for c in ccnt])),
                           float(np.mean([c[1] for c in ccnt])), 4 + 12 + 12 + 12, kern_s, ceil,
                           level, "fused correspondence kernel, no start leaf (point location, then the walk)",
                           float(np.mean(crep)), rinfo_c)
    traffic, traffic_src = committed_traffic()
    roof.update({
        "traffic": None if traffic is None else round(traffic),
        "traffic_source": traffic_src,
        "kernel": "icp_fused_kernel<1, 16>",
        "kernel_time_source": "mean of the library's dispatch-stamped event pairs over the "
                              f"warm-started launches (iterations 1..{ITERS - 1}) of "
                              f"{args.kernel_reps} registrations",
        "kernel_us_iteration0": round(float(loop_ms[:, 0].mean()) * 1e3, 3),
        "kernels_hip_sha256_16": kernel_source_hash(),
        "working_set_bytes": work,
        "single_descent_bytes_per_query": round(32 * (info["depth"] + 1)
                                                + 12 * (n / 2 ** info["depth"]) + 40, 1),
        "cold_start": {k: cold[k] for k in ("achieved", "peak", "frac", "kernel_us", "floor_us",
                                            "bytes_per_query", "nodes_per_query",
                                            "points_per_query", "replay", "random_gather",
                                            "byte_model")},
    })
    roof["cold_start"]["kernel_time_source"] = (
        f"icp_correspond_reduce_async at the 30 iterations' transforms x {args.kernel_reps}, "
        "the library's event pairs (no warm start)")
    log(f"roofline: {roof['achieved']} of {roof['peak']} GB/s at {roof['bound']} "
        f"-> frac {roof['frac']}")

    # standalone nn_query on the iteration-0 and the converged queries
    nnq = {"automatic_order": "morton" if info["auto_sort"] else "unsorted",
           "runs": "median and quartiles of 100 launches after 10 warm-ups"}
    qc = kdnn.transform(src, r["R"], r["t"])
    for name, q in (("iteration0", src), ("converged", qc)):
        for sort in (True, False):
            call, kern = time_query(g, tree, q, sort)
            c = pct(call)
            km = float(np.median(kern))
            nnq[f"{name}_{'morton' if sort else 'unsorted'}"] = {
                "call_us": round(c["median"] * 1e3, 2), "call_p25_us": round(c["p25"] * 1e3, 2),
                "call_p75_us": round(c["p75"] * 1e3, 2), "search_kernel_us": round(km * 1e3, 2),
                "order_us": round((c["median"] - km) * 1e3, 2) if sort else 0.0,
                "queries_per_s": round(len(q) / (c["median"] * 1e-3))}
    log("nn_query:", nnq)

    result.update({
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
        "dtype": "f32 distances, f64 transform+reduction+solve",
        "data": "synthetic",
        "config": {
            "workload": "scene-100k-icp30",
            "target_points": len(p.target), "source_points": n, "leaf_size": p.leaf_size,
            "icp_iterations_per_step": ITERS, "tree_depth": info["depth"],
            "step": "one 30-iteration ICP registration (icp_align default: host SVD solve "
                    "and convergence check per iteration), tree and clouds resident",
        },
        "icp_iters_per_s": round(args.steps * ITERS / T, 1),
        "icp_iter_us": round(T / (args.steps * ITERS) * 1e6, 2),
        "registration_ms": ms_stats(per),
        "icp_device_loop": {
            "icp_iters_per_s": round(args.steps * ITERS / Td, 1),
            "icp_iter_us": round(Td / (args.steps * ITERS) * 1e6, 2),
            "queries_per_s": round(args.steps * ITERS * n / Td),
            "registration_ms": ms_stats(perd),
            "speedup_vs_host_solve": round(T / Td, 3),
            "R_diff_vs_host_loop": float(np.linalg.norm(rd["R"] - r["R"])),
            "note": "KDNN_ICP_DEVICE_LOOP: the iterations stay on the device (a one-group "
                    "kernel reduces, solves with Horn's quaternion form and applies the "
                    "convergence rule); the host enqueues all 30 and waits once"},
        "build": {"host_build_ms": round(info["build_ms"], 3),
                  "upload_ms_first_tree": round(info["upload_ms"], 3),
                  "upload_ms": round(info2["upload_ms"], 3),
                  "wall_ms": round(build_wall_ms, 3),
                  "note": "upload_ms: a second build of the same tree (the first device "
                          "allocation also pays the runtime's start-up)"},
        "fused_kernel": {"name": "icp_fused_kernel<1, 16>",
                         "in_icp_loop": {
                             "iteration0_mean_us": round(float(loop_ms[:, 0].mean()) * 1e3, 3),
                             **{f"warm_{k}_us": round(v * 1e3, 3)
                                for k, v in pct(loop_ms[:, 1:].ravel()).items() if k != "n"},
                             "launches": int(loop_ms.size),
                             "note": "every fused launch of the host-loop registrations; "
                                     "iterations after the first start each search at the "
                                     "leaf of its point's previous match"},
                         "cold_entry_point": {
                             **{f"{k}_us": round(v * 1e3, 3) for k, v in pct(kern_ms).items()
                                if k != "n"},
                             "launches": len(kern_ms),
                             "queries_per_s": round(n / kern_s),
                             "call_mean_us": round(float(call_ms.mean()) * 1e3, 2),
                             "note": "icp_correspond_reduce_async at the 30 iterations' "
                                     "transforms: no start leaf (point location, then the walk)"},
                         "timing": "event pair stamped by the search kernel's dispatch "
                                   "(library timing facility, hipExtLaunchKernel)"},
        "icp_iteration_breakdown_us": {
            "host_loop_iteration": round(T / (args.steps * ITERS) * 1e6, 2),
            "device_loop_iteration": round(Td / (args.steps * ITERS) * 1e6, 2),
            "fused_kernel_in_loop_warm": round(warm_s * 1e6, 2),
            "fused_kernel": round(kern_s * 1e6, 2),
            "correspondence_call_events": round(float(call_ms.mean()) * 1e3, 2),
            "host_svd_solve_through_python": round(solve_us, 2),
            "note": "host loop: the search kernel, the one-group reduction into pinned "
                    "memory (correspondence_call_events covers both and the gap between "
                    "them), then the host's wait, SVD solve and next launch; device loop: the "
                    "search kernel and a one-group step kernel per iteration"},
        "nn_query": nnq,
        "roofline": roof,
    })
    return p, tree, src, ws, r


def bench_reject(g, p, tree, src, ws, args):
    """Scene ICP with max_dist 1 m fused into the search and the 3-sigma
    residual rejection with a second solve per iteration (article §4.4)."""
    rej = {"max_dist_m": 1.0, "reject_k": 3.0}
    for name, kw in (("host_loop", {}), ("device_loop", {"device_loop": True})):
        for _ in range(2):
            tree.icp(src, max_iter=ITERS, workspace=ws, max_dist=1.0, reject_k=3.0, **kw)
        steps = max(args.steps // 2, 1)
        Tr, _, _ = timed_steps(g, lambda: tree.icp(src, max_iter=ITERS, workspace=ws,
                                                   max_dist=1.0, reject_k=3.0, **kw), steps)
        rej[name] = {"steps": steps, "icp_iters_per_s": round(steps * ITERS / Tr, 1),
                     "icp_iter_us": round(Tr / (steps * ITERS) * 1e6, 2),
                     "queries_per_s": round(steps * ITERS * len(p.source) / Tr)}
    log("with rejection:", rej)
    return rej


def bench_sweep(g, p, src):
    """Builder variants: leaf size and split-axis rule (article §4.1, §4.2)."""
    import numpy as np
    kdnn = g.kdnn
    n = len(p.source)
    sweep = []
    for rr in (False, True):
        for leaf in (1, 4, 8, 16, 32, 64):
            tr = kdnn.Tree(p.target, leaf, round_robin=rr)
            inf_ = tr.info
            call, _ = time_query(g, tr, src, None, reps=10, warm=2)
            cn, cp = query_counts(tr, src)
            iw = tr.icp_workspace(n)
            tr.icp(src, max_iter=ITERS, workspace=iw)
            Ti, _, _ = timed_steps(g, lambda: tr.icp(src, max_iter=ITERS, workspace=iw), 3)
            sweep.append({
                "axis": "round_robin" if rr else "max_variance", "leaf": leaf,
                "depth": inf_["depth"], "host_build_ms": round(inf_["build_ms"], 2),
                "device_mb": round(inf_["device_bytes"] / 2 ** 20, 2),
                "nn_query_us": round(float(np.median(call)) * 1e3, 1),
                "nodes_per_query": round(cn, 2), "points_per_query": round(cp, 2),
                "icp_iter_us": round(Ti / (3 * ITERS) * 1e6, 1)})
            del tr
    log("sweep:", [(s["axis"][0], s["leaf"], s["nn_query_us"]) for s in sweep])
    return sweep


def bench_lidar(g):
    """16 LiDAR frame pairs x 30 iterations: batched (device loop, the default;
    and a host solve per iteration) vs one registration after another."""
    import numpy as np
    kdnn = g.kdnn
    import synth
    log("LiDAR: 16 frame pairs, 30 iterations each")
    lp = synth.lidar_pairs()
    ltrees = [kdnn.Tree(q.target, q.leaf_size) for q in lp]
    lsrc = [g.dev(q.source) for q in lp]
    bws = kdnn.icp_batch_workspace([len(x) for x in lsrc])
    lws = [t_.icp_workspace(len(x)) for t_, x in zip(ltrees, lsrc)]
    runs = {
        "batched": lambda: kdnn.icp_batch(ltrees, lsrc, max_iter=ITERS, workspace=bws),
        "batched_host_solve": lambda: kdnn.icp_batch(ltrees, lsrc, max_iter=ITERS, workspace=bws,
                                                     device_loop=False),
        "sequential": lambda: [t_.icp(x, max_iter=ITERS, workspace=w_, sort=False)
                               for t_, x, w_ in zip(ltrees, lsrc, lws)],
        "sequential_device_loop": lambda: [t_.icp(x, max_iter=ITERS, workspace=w_, sort=False,
                                                  device_loop=True)
                                           for t_, x, w_ in zip(ltrees, lsrc, lws)],
    }
    lid = {"pairs": len(lp), "points_per_frame": int(np.mean([len(x) for x in lsrc])),
           "iterations": ITERS}
    q_ = sum(len(x) for x in lsrc) * ITERS
    for name, fn in runs.items():
        fn()
        _, per, _ = timed_steps(g, fn, 5)
        med = float(np.median(per))
        lid[name] = {"ms_per_16_pairs": round(med * 1e3, 3), "pairs_per_s": round(len(lp) / med, 1),
                     "icp_iters_per_s": round(len(lp) * ITERS / med, 1),
                     "queries_per_s": round(q_ / med), "runs": "median of 5"}
    lid["speedup_batched_vs_sequential"] = round(lid["sequential"]["ms_per_16_pairs"]
                                                 / lid["batched"]["ms_per_16_pairs"], 2)
    log("LiDAR:", {k: v["ms_per_16_pairs"] for k, v in lid.items() if isinstance(v, dict)})
    return lid, lp, lsrc


def bench_voxel(g, lsrc):
    """Voxel-grid down-sampling (article §4.3): the first 8 LiDAR frames stacked
    (~1.05M points, each in its own sensor frame), 0.2 m voxels; the same cloud
    at 1 m beside it (voxels of up to ~6,000 points)."""
    import numpy as np
    kdnn, torch = g.kdnn, g.torch
    vox_in = torch.cat(lsrc[:8]).contiguous()
    vws = torch.empty(int(kdnn._lib.lib().voxel_downsample_workspace_bytes(len(vox_in))),
                      dtype=torch.uint8, device="cuda")

    def timed(leaf):
        vout = kdnn.voxel_downsample(vox_in, leaf, workspace=vws)
        evs = g.events(20)
        walls = []
        for e0, e1 in evs:
            torch.cuda.synchronize()
            a = time.perf_counter()
            e0.record(g.stream)
            vout = kdnn.voxel_downsample(vox_in, leaf, workspace=vws)
            e1.record(g.stream)
            torch.cuda.synchronize()
            walls.append(time.perf_counter() - a)
        span = np.array([a.elapsed_time(b) for a, b in evs])
        return len(vout), float(np.median(walls)), float(np.median(span)) * 1e-3

    m, wall, t = timed(0.2)
    n = len(vox_in)
    # the filter's minimum traffic: every point read once, every voxel written
    # once (centroid 12 B + count 4 B)
    b_min = 12 * n + 16 * m
    m1, wall1, t1 = timed(1.0)
    vox = {"input_points": int(n), "leaf_m": 0.2, "voxels": int(m),
           "wall_ms": round(wall * 1e3, 4),
           "device_span_ms": round(t * 1e3, 4),
           "points_per_s": round(n / wall),
           "hbm_roofline": {"bound": "hbm", "bytes_min": b_min,
                            "achieved": round(b_min / t / 1e9, 1), "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": round(b_min / t / 1e9 / HBM_PEAK_GBS, 5)},
           "leaf_1m": {"voxels": int(m1), "wall_ms": round(wall1 * 1e3, 4),
                       "device_span_ms": round(t1 * 1e3, 4)},
           "note": "median of 20 calls; device_span = events around the synchronous call (its "
                   "kernels, launched at once, and the read-back of the voxel count at the "
                   "end); bytes_min = one read of every point and one write per voxel"}
    log(f"voxel filter: {n} -> {m} in {vox['wall_ms']} ms wall, {vox['device_span_ms']} ms span; "
        f"1 m: {m1} in {vox['leaf_1m']['device_span_ms']} ms span")
    return vox


def bench_recipe(g):
    """The article's regression recipe (§6): 200k points uniform in [-25, 25]^3,
    10 degrees about a random axis + 0.5 m, N(0, 0.01^2) noise, 30 iterations --
    the whole registration's time (the article expects under 200 ms for its GPU
    version) and the §6 error metrics of the result."""
    import numpy as np
    kdnn = g.kdnn
    import oracle
    import synth
    p = synth.recipe()
    t0 = time.perf_counter()
    tree = kdnn.Tree(p.target, p.leaf_size)
    build_ms = (time.perf_counter() - t0) * 1e3
    src = g.dev(p.source)
    ws = tree.icp_workspace(len(p.source))
    out = {"points": len(p.source), "iterations": p.iters, "host_build_ms": round(build_ms, 2)}
    for name, kw in (("host_loop", {}), ("device_loop", {"device_loop": True})):
        tree.icp(src, max_iter=p.iters, workspace=ws, **kw)
        _, per, r = timed_steps(g, lambda: tree.icp(src, max_iter=p.iters, workspace=ws, **kw), 5)
        med = float(np.median(per))
        out[name] = {"ms_per_registration": round(med * 1e3, 3),
                     "icp_iters_per_s": round(p.iters / med, 1),
                     "rot_err_deg": round(float(np.degrees(oracle.rot_err(r["R"], p.R_true))), 4),
                     "trans_err_m": round(oracle.trans_err(r["t"], p.t_true), 5),
                     "runs": "median of 5"}
    out["note"] = ("registration time excludes the tree build (host_build_ms); plain "
                   "point-to-point ICP on this uniform cloud is still approaching the truth "
                   "after 30 iterations")
    log("recipe:", out)
    return out, p


def bench_query_workload(g, name):
    """One nn_query pass of a Stress or Skewed configuration in the library's
    automatic order, with its roofline at the level holding its tree."""
    import numpy as np
    kdnn = g.kdnn
    import synth
    gen, leaf = {"stress_1M_leaf8": (synth.stress, 8), "stress_1M_leaf16": (synth.stress, 16),
                 "skewed_500k_leaf8": (synth.skewed, 8),
                 "skewed_500k_leaf16": (synth.skewed, 16)}[name]
    pw = gen()
    tw = kdnn.Tree(pw.target, leaf)
    inf_ = tw.info
    qw = g.dev(pw.source)
    m = len(qw)
    call, kern = time_query(g, tw, qw, None, reps=20, warm=3)
    cn, cp = query_counts(tw, qw)
    sorted_ = bool(inf_["auto_sort"])
    work = 24 * 2 ** (inf_["depth"] + 1) + 16 * (len(pw.target) + 16)
    ceil = gather_ceilings(g, work)
    km = float(np.median(kern))
    # index read 4 + query 12 + outputs 8 (+ the traversal-order slot 4 when ordered)
    rs, rinfo = replay_time(tw, qw, False, 20)
    roof = search_roofline(m, cn, cp, 4 + 12 + 8 + (4 if sorted_ else 0), km * 1e-3, ceil,
                           level_of(work, inf_["l2_bytes"]), "nn_query search kernel", rs, rinfo)
    roof["replay"]["note"] = "median of 20 replays in nn_query's launch shape and order"
    c = pct(call)
    out = {"queries": m, "target_points": len(pw.target), "leaf": leaf, "depth": inf_["depth"],
           "automatic_order": "morton" if sorted_ else "unsorted",
           "call_us": round(c["median"] * 1e3, 2), "call_p25_us": round(c["p25"] * 1e3, 2),
           "call_p75_us": round(c["p75"] * 1e3, 2), "search_kernel_us": round(km * 1e3, 2),
           "order_us": round((c["median"] - km) * 1e3, 2) if sorted_ else 0.0,
           "queries_per_s": round(m / (c["median"] * 1e-3)),
           "host_build_ms": round(inf_["build_ms"], 1),
           "working_set_bytes": work, "roofline": roof,
           "runs": "median and quartiles of 20 calls after 3 warm-ups"}
    log(name, {k: out[k] for k in ("call_us", "search_kernel_us")}, "frac", roof["frac"])
    return out, pw


# -------------------------------------------------------------- CPU oracle
def cpu_threads():
    """Host threads for the oracle: the CPUs this process may run on, capped
    by OMP_NUM_THREADS when the environment sets it (the host's share)."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    return max(1, min(n, int(cap))) if cap.isdigit() else n


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "?"


class ThreadedSearch:
    """The oracle's KD search of a query set split into chunks over host threads
    (the C query keeps no global state; ctypes releases the GIL)."""

    def __init__(self, tree, pool, threads):
        self.tree, self.pool, self.k = tree, pool, threads

    def query(self, q):
        import numpy as np
        parts = list(self.pool.map(self.tree.query, np.array_split(q, self.k * 4)))
        return np.concatenate([a for a, _ in parts]), np.concatenate([b for _, b in parts])


def cpu_baseline(scene_p, workloads, lidar_pairs, recipe_p=None):
    """The oracle, as it stands, on the host: the first two of the article's
    three baselines (§6: brute force, CPU KD-tree; the GPU is the third)."""
    import concurrent.futures as cf

    import numpy as np

    import oracle
    import synth
    th = cpu_threads()
    n = len(scene_p.source)
    res = {}
    with cf.ThreadPoolExecutor(th) as pool:
        otree = oracle.KDTree(scene_p.target, scene_p.leaf_size)
        par = ThreadedSearch(otree, pool, th)
        log(f"cpu: oracle Scene ICP, 1 thread and {th} threads")
        t1 = []
        for _ in range(3):
            t0 = time.perf_counter()
            oracle.icp(scene_p.target, scene_p.source, ITERS, tree=otree)
            t1.append(time.perf_counter() - t0)
        tn = []
        o = None
        for _ in range(3):
            t0 = time.perf_counter()
            o = oracle.icp(scene_p.target, scene_p.source, ITERS, tree=par)
            tn.append(time.perf_counter() - t0)
        m1, mn = float(np.median(t1)), float(np.median(tn))
        res["scene_icp"] = {"threads": th, "s_per_registration_all_threads": round(mn, 3),
                            "s_per_registration_1_thread": round(m1, 3),
                            "queries_per_s_all_threads": round(ITERS * n / mn),
                            "queries_per_s_1_thread": round(ITERS * n / m1),
                            "icp_iters_per_s_all_threads": round(ITERS / mn, 2),
                            "icp_iters_per_s_1_thread": round(ITERS / m1, 2),
                            "runs": "median of 3 registrations each"}
        log("cpu: brute force")
        tiny = synth.tiny()
        tb = []
        for _ in range(10):
            t0 = time.perf_counter()
            oracle.icp(tiny.target, tiny.source, tiny.iters, nn="brute")
            tb.append(time.perf_counter() - t0)
        res["tiny_brute_force_icp"] = {"iterations": tiny.iters, "s": round(float(np.median(tb)), 4),
                                       "threads": 1, "runs": "median of 10"}
        T_ = scene_p.target
        tsb = []
        for _ in range(3):
            t0 = time.perf_counter()
            list(pool.map(lambda c: oracle.brute_nn(T_, c), np.array_split(scene_p.source, th * 4)))
            tsb.append(time.perf_counter() - t0)
        t0 = time.perf_counter()
        oracle.brute_nn(T_, scene_p.source[:5000])
        t_one = (time.perf_counter() - t0) * n / 5000
        res["scene_brute_force_iteration"] = {
            "pairs": n * len(T_), "s_all_threads": round(float(np.median(tsb)), 3),
            "threads": th, "s_1_thread_estimated": round(t_one, 2),
            "runs": f"median of 3 on {th} threads; 1 thread timed on 5,000 queries and scaled"}
        for name, pw, leaf in workloads:
            log(f"cpu: oracle KD {name}")
            t0 = time.perf_counter()
            ot = oracle.KDTree(pw.target, leaf)
            tbuild = time.perf_counter() - t0
            ps = ThreadedSearch(ot, pool, th)
            tq = []
            for _ in range(3):
                t0 = time.perf_counter()
                ps.query(pw.source)
                tq.append(time.perf_counter() - t0)
            res[name] = {"queries": len(pw.source), "threads": th,
                         "s_query_all_threads": round(float(np.median(tq)), 3),
                         "queries_per_s_all_threads": round(len(pw.source) / float(np.median(tq))),
                         "oracle_build_s": round(tbuild, 2), "runs": "median of 3 passes"}
            del ot
        if recipe_p is not None:
            log("cpu: oracle KD ICP of the page recipe")
            t0 = time.perf_counter()
            ot = oracle.KDTree(recipe_p.target, recipe_p.leaf_size)
            tb_ = time.perf_counter() - t0
            t0 = time.perf_counter()
            oracle.icp(recipe_p.target, recipe_p.source, recipe_p.iters,
                       tree=ThreadedSearch(ot, pool, th))
            tr_ = time.perf_counter() - t0
            t0 = time.perf_counter()
            oracle.brute_nn(recipe_p.target, recipe_p.source[:2000])
            tbf = (time.perf_counter() - t0) * len(recipe_p.source) / 2000
            res["recipe_200k_icp"] = {
                "s_registration_all_threads": round(tr_, 3), "threads": th,
                "oracle_build_s": round(tb_, 2),
                "brute_force_registration_s_1_thread_estimated": round(tbf * recipe_p.iters, 1),
                "runs": "one registration; brute force timed on 2,000 queries of one "
                        "iteration and scaled to 30 iterations"}
            del ot
        if lidar_pairs:
            log("cpu: oracle KD ICP of the 16 LiDAR pairs")
            t0 = time.perf_counter()
            for q in lidar_pairs:
                ot = oracle.KDTree(q.target, q.leaf_size)
                oracle.icp(q.target, q.source, ITERS, tree=ThreadedSearch(ot, pool, th))
            tl = time.perf_counter() - t0
            res["lidar_16_pairs_icp"] = {"s": round(tl, 2), "threads": th,
                                         "pairs_per_s": round(len(lidar_pairs) / tl, 3),
                                         "runs": "one pass over the 16 pairs (tree builds included)"}
    return res, th, o


# ------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--kernel-reps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=SECTIONS, default=None,
                    help="run one section (for a profiled run of that workload)")
    ap.add_argument("--json-out", default=None, help="also write the JSON line to this file")
    ap.add_argument("--profile-pass", action="store_true",
                    help="only: two Scene ICP registrations (host loop), the 30 iterations' "
                         "transforms through the cold entry point, then three "
                         f"{COPY_MIB} MiB device copies (calibration for HBM counters)")
    ap.add_argument("--summarize", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the profiles/ traffic summary from rocprofv3 CSV output")
    ap.add_argument("--summarize-trace", nargs=3, metavar=("TRACE_DIR", "ONLY", "OUT_NAME"),
                    help="write a profiles/ kernel-trace summary of a `--only` run")
    ap.add_argument("--summarize-counters", metavar="OUT_DIR",
                    help="write the profiles/ counter summary from gpurun_out/pmc_<set> and exit")
    ap.add_argument("--counters-of", nargs=4, metavar=("OUT_DIR", "KERNEL", "OUT_NAME", "ONLY"),
                    help="the same for the kernels named KERNEL of `bench.py --only ONLY "
                         "--steps 2 --warmup 1 --no-cpu-baseline`")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.counters_of:
        d, kern, name, only = args.counters_of
        summarize_counters(d, kern, name, f"{kern} in bench.py --only {only}",
                           f"python3 -u bench.py --only {only} --steps 2 --warmup 1 "
                           "--no-cpu-baseline")
        return
    if args.summarize:
        summarize(*args.summarize)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world})", file=sys.stderr)
        sys.exit(2)

    import numpy as np

    g = Gpu()

    if args.profile_pass:
        import synth
        p = synth.scene()
        tree = g.kdnn.Tree(p.target, p.leaf_size)
        src = g.dev(p.source)
        ws = tree.icp_workspace(len(p.source))
        # two registrations (their fused launches after the first of each are
        # warm-started), then the 30 iterations' transforms through the cold
        # entry point
        for _ in range(PROFILE_REGS):
            r = tree.icp(src, max_iter=ITERS, workspace=ws)
        sums = g.torch.zeros(g.kdnn.KDNN_SUMS_DOUBLES, dtype=g.torch.float64, device="cuda")
        for k in range(ITERS):
            tree.correspond_reduce_async(src, r["Rt_hist"][k, :9], r["Rt_hist"][k, 9:], sums, ws)
        a = g.torch.empty(COPY_MIB << 18, dtype=g.torch.float32, device="cuda")
        b = g.torch.empty_like(a)
        a.fill_(1.0)
        for _ in range(3):
            b.copy_(a)
        g.torch.cuda.synchronize()
        log(f"profile pass done: {PROFILE_REGS} registrations of {ITERS} iterations +", ITERS,
            f"cold fused launches + 3 copies of {COPY_MIB} MiB")
        return

    def want(s):
        return args.only is None or args.only == s

    result = {} if args.only in (None, "scene") else {"only": args.only}
    scene_p = tree = src = ws = r_gpu = None
    if want("scene"):
        scene_p, tree, src, ws, r_gpu = bench_scene(g, args, result)
    elif want("reject") or want("sweep"):
        import synth
        scene_p = synth.scene()
        tree = g.kdnn.Tree(scene_p.target, scene_p.leaf_size)
        src = g.dev(scene_p.source)
        ws = tree.icp_workspace(len(scene_p.source))
    if want("reject"):
        result["icp_with_rejection"] = bench_reject(g, scene_p, tree, src, ws, args)
    if want("sweep"):
        result["leaf_axis_sweep"] = bench_sweep(g, scene_p, src)
    lpairs = lsrc = None
    if want("lidar"):
        result["lidar_pairs"], lpairs, lsrc = bench_lidar(g)
    if want("voxel"):
        if lsrc is None:
            import synth
            lsrc = [g.dev(q.source) for q in synth.lidar_pairs()[:8]]
        result["voxel_downsample"] = bench_voxel(g, lsrc)
    recipe_p = None
    if want("recipe"):
        result["page_recipe"], recipe_p = bench_recipe(g)
    other, cpu_workloads = {}, []
    for name in QUERY_WORKLOADS:
        if want(name):
            other[name], pw = bench_query_workload(g, name)
            cpu_workloads.append((name, pw, other[name]["leaf"]))
    if other:
        result["other_workloads_nn_query"] = other

    if not args.no_cpu_baseline and args.only is None:
        res, th, o = cpu_baseline(scene_p, cpu_workloads, lpairs, recipe_p)
        sc = res["scene_icp"]
        result["cpu_baseline"] = {
            "value": sc["queries_per_s_all_threads"], "unit": "queries/s", "cores": th,
            "kind": "oracle",
            "sample": f"3 full Scene registrations (30 ICP iterations x 100k queries) with the "
                      f"oracle's C KD-tree search split over {th} host threads and its numpy "
                      f"fp64 reduction and Horn solve; median "
                      f"{sc['s_per_registration_all_threads']} s per registration",
            "icp_iters_per_s": sc["icp_iters_per_s_all_threads"],
            "value_1_thread": sc["queries_per_s_1_thread"],
            "host": {"cpu_model": cpu_model(), "nproc": os.cpu_count(),
                     "affinity_cpus": len(os.sched_getaffinity(0)),
                     "omp_num_threads": os.environ.get("OMP_NUM_THREADS")},
            "R_diff_vs_gpu": float(np.linalg.norm(o["R"] - r_gpu["R"])),
        }
        result["cpu_context"] = res
    line = json.dumps(result)
    print(line, flush=True)
    if args.json_out:
        os.makedirs(os.path.dirname(os.path.abspath(args.json_out)), exist_ok=True)
        with open(args.json_out, "w") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
