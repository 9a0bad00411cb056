#!/usr/bin/env python3
"""Benchmark of the balanced expert-parallel hot path on one MI355X.

One step = the whole path over one batch of synthetic router output at the
Kimi-K3-shaped layer (R=32 virtual ranks, E=896, K=16, S=4096, H=7168 bf16,
B=28, weight blocks 3x7168x512 bf16): plan, replicate duplicate weights,
dispatch, combine (identity expert: y = recv), reduce duplicate gradients.
Inputs are resident in HBM before timing starts.

Printed: ONE JSON line. `value` is dispatch+combine throughput in GB/s of
algorithmic bytes (each token row read once, each slot written once, plus the
index and weight arrays), measured with HIP events on the launch stream over the
timed steps. `roofline` describes the dominant kernel; `cpu_baseline` times the
CPU oracle on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "dispatch+combine GB/s (% of HBM peak) + plan latency µs, K3 shape, 1 GPU"
_CSRC = "token_dispatch_amd/csrc/"
KERNEL_SOURCES = tuple(_CSRC + f for f in ("move.hip", "plan.hip", "api.hip", "internal.h",
                                           "backward.hip", "rows.h"))
# The sources that define each call's kernels and their launches: a counter
# summary stays valid for a call while these are unchanged.
_MOVE_SOURCES = tuple(_CSRC + f for f in ("move.hip", "rows.h", "internal.h"))
OP_SOURCES = {"dispatch": _MOVE_SOURCES, "combine": _MOVE_SOURCES, "replicate": _MOVE_SOURCES,
              "reduce": _MOVE_SOURCES, "plan": (_CSRC + "plan.hip", _CSRC + "internal.h")}


def kernel_source_hash(files=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for rel in files:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(wl, n_mat, n_xm):
    row = wl.row_bytes
    d = wl.n_ent * row + wl.n_tok * row + 4 * wl.n_ent
    c = wl.n_ent * row + wl.n_tok * row + 8 * wl.n_ent
    rep = 2 * n_mat * wl.block_bytes
    red = (n_mat + 2 * n_xm) * wl.block_elems * 4
    plan = 12 * wl.n_ent
    # backward: grad_out read once, y read, grad_y written, w / grad_w / dst
    cb = 2 * wl.n_ent * row + wl.n_tok * row + 12 * wl.n_ent
    db = wl.n_ent * row + wl.n_tok * row + 4 * wl.n_ent
    return {"dispatch": d, "combine": c, "replicate": rep, "reduce": red, "plan": plan,
            "combine_backward": cb, "dispatch_backward": db}


TRAFFIC_PATH = os.path.join(ROOT, "profiles", "hbm_traffic_k3.json")

# Library kernels behind each C-ABI call (one call may enqueue several launches).
OP_KERNELS = {"plan": ("k_count", "k_scan", "k_solve", "k_solve_bounded", "k_assign",
                       "k_plan_fused"),
              "replicate": ("k_replicate",),
              "dispatch": ("k_dispatch",), "combine": ("k_combine",), "reduce": ("k_reduce",)}
# (k_combine also serves the backward of dispatch, so traffic is only summed for
# runs without --with-backward)
COPY_CAL_BYTES = 1 << 30


def traffic_for(op: str, workload: str, plan: str):
    """HBM bytes per call of `op` from the committed counter summary, if it was
    taken on this workload and plan and on the current sources of that call's
    kernels; else None."""
    if not os.path.exists(TRAFFIC_PATH):
        return None
    with open(TRAFFIC_PATH) as f:
        rec = json.load(f)
    if rec.get("workload") != workload or rec.get("plan") != plan:
        return None
    k = rec.get("ops", {}).get(op)
    if k is None or k.get("source_hash") != kernel_source_hash(OP_SOURCES[op]):
        return None
    return k.get("hbm_bytes_per_call")


def _pmc_rows(csv_path: str, counter: str):
    """(dispatch id, kernel name, value) of one counter from a rocprofv3 --pmc CSV."""
    import csv
    out = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") != counter:
                continue
            key = int(r["Dispatch_Id"])
            name = r["Kernel_Name"]
            out[key] = (name, out.get(key, (name, 0.0))[1] + float(r["Counter_Value"]))
    return [(k, v[0], v[1]) for k, v in sorted(out.items())]


def traffic_from_pmc(fetch_csv: str, write_csv: str, steps: int, warmup: int, command: str,
                     workload: str, plan: str) -> dict:
    """HBM bytes per C-ABI call from two rocprofv3 --pmc runs of this benchmark
    (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch) on `workload` and `plan`, each
    scaled by what the same counter reads for the plain device copy of
    COPY_CAL_BYTES that --copy-calibration enqueues after the timed steps."""
    rec = {"kernel_source_hash": kernel_source_hash(), "command": command,
           "workload": workload, "plan": plan,
           "copy_calibration_bytes": COPY_CAL_BYTES, "ops": {}}
    calls = steps + warmup
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _pmc_rows(path, counter)
        # the calibration copy is the first runtime copy-kernel dispatch after the
        # last library kernel: --copy-calibration enqueues it right after the steps
        last_lib = max(d for d, n, _ in rows if "moonep" in n)
        copies = [v for d, n, v in rows if d > last_lib and "copyBuffer" in n]
        if not copies:
            raise SystemExit(f"{path}: no copy-kernel dispatch for the calibration")
        cal_kib = copies[0]
        factor = COPY_CAL_BYTES / (cal_kib * 1024.0)
        rec[counter.lower() + "_copy_kib"] = cal_kib
        rec[counter.lower() + "_scale"] = factor
        for op, kernels in OP_KERNELS.items():
            tot = sum(v for _, n, v in rows if any(k + "(" in n or k + "<" in n for k in kernels))
            ent = rec["ops"].setdefault(op, {})
            ent[counter.lower() + "_bytes_per_call"] = tot * 1024.0 * factor / calls
    for op, ent in rec["ops"].items():
        ent["hbm_bytes_per_call"] = ent["fetch_size_bytes_per_call"] + ent["write_size_bytes_per_call"]
        ent["source_hash"] = kernel_source_hash(OP_SOURCES[op])
    return rec


# Kernel classes of a counter summary: the library's kernels and the streaming
# kernels the ceilings are measured with.
PMC_CLASSES = ("k_count", "k_scan", "k_solve", "k_solve_bounded", "k_assign", "k_plan_fused",
               "k_replicate", "k_dispatch", "k_combine", "k_reduce", "k_bwd_dot", "k_bwd_scatter",
               "k_stream_read", "k_stream_write", "k_stream_copy")


def pmc_summary(dirs):
    """Per kernel class, from rocprofv3 runs that each wrote a *counter_collection.csv
    (--pmc) and a *kernel_trace.csv (--kernel-trace) into one of `dirs`: dispatches,
    median duration, the mean of every counter per dispatch and, where the counters
    are there, EA request sizes, latencies (LEVEL / requests, in cycles) and
    requests in flight (LEVEL / GRBM_GUI_ACTIVE x 8: GRBM_GUI_ACTIVE counts the
    cycles of all 8 XCDs)."""
    import csv
    import glob

    def cls(name):
        return next((c for c in PMC_CLASSES if c + "<" in name or c + "(" in name), None)

    out = {}
    for d in dirs:
        rec = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            sums, disp = {}, {}
            for r in csv.DictReader(open(f)):
                c = cls(r["Kernel_Name"])
                if c is None:
                    continue
                sums.setdefault(c, {}).setdefault(r["Counter_Name"], 0.0)
                sums[c][r["Counter_Name"]] += float(r["Counter_Value"])
                disp.setdefault(c, set()).add(r["Dispatch_Id"])
            for c, kv in sums.items():
                rec.setdefault(c, {})["dispatches"] = len(disp[c])
                rec[c].update({k: v / len(disp[c]) for k, v in kv.items()})
        for f in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
            durs = {}
            for r in csv.DictReader(open(f)):
                c = cls(r["Kernel_Name"])
                if c is not None:
                    durs.setdefault(c, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
            for c, v in durs.items():
                v.sort()
                rec.setdefault(c, {})["median_us"] = v[len(v) // 2] / 1e3
        for c, k in rec.items():
            for side in ("RDREQ", "WRREQ"):
                n, lvl = k.get(f"TCC_EA0_{side}_sum"), k.get(f"TCC_EA0_{side}_LEVEL_sum")
                if n and lvl is not None:
                    k[f"{side.lower()}_latency_cycles"] = lvl / n
                    if k.get("GRBM_GUI_ACTIVE"):
                        k[f"{side.lower()}_in_flight"] = lvl / k["GRBM_GUI_ACTIVE"] * 8
        out[os.path.basename(os.path.normpath(d))] = rec
    return out


def plan_latency(plan_fn, dims, ids_d, plan_buf, stream, iters):
    """The plan call alone, timed with events on its stream: warm (the ids were
    just written by a device copy, as a router would leave them) and cold (after
    1 GiB has streamed through the caches). Median and min in microseconds."""
    import numpy as np
    import torch
    src = ids_d.clone()
    flush = torch.empty(1 << 28, dtype=torch.float32, device=ids_d.device)
    out = {}
    for kind in ("warm", "cold"):
        ts = []
        for i in range(iters):
            # the GPU is kept busy ahead of the timed region (a spin, or the flush)
            # so that the host's launches are queued before the first event runs
            if kind == "warm":
                torch.cuda._sleep(200_000)
                ids_d.copy_(src)
            else:
                flush.fill_(float(i))
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            plan_fn(dims, ids_d, plan_buf)
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b) * 1e3)
        out[kind + "_median"] = round(float(np.median(ts)), 2)
        out[kind + "_min"] = round(float(np.min(ts)), 2)
    out["iters"] = iters
    del flush, src
    return out


def graph_replay(step, stream, steps):
    """The whole step captured once in a HIP graph (every chunk launch a kernel
    node) and replayed `steps` times: milliseconds per replay by events on the
    launch stream, or the reason the capture failed."""
    import torch
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        torch.cuda.synchronize()
        g.replay()  # first replay uploads the graph
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            g.replay()
        b.record(stream)
        b.synchronize()
        return {"ms_per_step": round(a.elapsed_time(b) / steps, 4), "replays": steps}
    except Exception as exc:  # report, do not lose the bench line
        return {"error": f"{type(exc).__name__}: {exc}"}


def host_cpu() -> str:
    """The host's CPU model and logical CPU count, as the baseline's context."""
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"{model}, {os.cpu_count()} logical CPUs"


def host_threads() -> int:
    """Threads this process may run on: OMP_NUM_THREADS if set, else the CPUs it
    is allowed on."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_baseline(wl, ids, w, hidden_dev, budget_s):
    """The oracle as it stands, on the host's cores, on a bounded sample of the
    workload: the plan (sequential by nature, one thread); dispatch into a host
    receive buffer; combine of consecutive token batches that read their K rows
    from that buffer inside the timed call (identity expert, y = recv, as on the
    GPU). Dispatch and combine run once with the oracle's OpenMP loops on every
    thread the process may use and once on one thread. The receive buffer is
    allocated and its pages touched by an untimed dispatch first, as a CPU
    implementation would keep it between steps. Times are scaled to the whole
    workload (all slots, all tokens)."""
    import numpy as np
    import torch
    import oracle
    import workloads as W

    threads = host_threads()
    t0 = time.perf_counter()
    p = oracle.plan(wl.R, wl.E, wl.K, wl.S, wl.B, ids)
    t_plan = time.perf_counter() - t0

    hid = hidden_dev.view(wl.n_tok, wl.H).cpu()
    hid = hid.view(torch.int16).numpy().view(np.uint16) if wl.dtype == W.BF16 else hid.numpy()
    recv = np.empty((wl.n_ent, wl.H), dtype=hid.dtype)
    wf = w.reshape(-1)
    dt = W.BF16 if wl.dtype == W.BF16 else W.F32
    nbytes = algorithmic_bytes(wl, 0, 0)
    oracle.set_threads(threads)
    oracle.dispatch(p, wl.K, hid, out=recv)  # untimed: touches every page of recv

    def run(n_threads, budget):
        """(seconds of dispatch scaled to all slots, of combine scaled to all
        tokens, what was sampled) on n_threads threads within about `budget` s."""
        oracle.set_threads(n_threads)
        # dispatch: whole destination-rank windows until half the budget is spent
        t_d, ranks = 0.0, 0
        while ranks < wl.R and (ranks == 0 or t_d < 0.5 * budget):
            step = wl.R if n_threads > 1 and ranks == 0 else 1  # all windows in one call
            lo, hi = ranks * wl.SK, (ranks + step) * wl.SK
            t0 = time.perf_counter()
            oracle.dispatch(p, wl.K, hid, lo, hi, out=recv[lo:hi])
            t_d += time.perf_counter() - t0
            ranks += step
        # combine: batches of at most 8192 tokens until the rest of the budget is spent
        out = np.empty((8192, wl.H), dtype=hid.dtype)
        t_c, n = 0.0, 0
        while n < wl.n_tok and (n == 0 or t_c < budget - t_d):
            m = min(8192, wl.n_tok - n)
            t0 = time.perf_counter()
            res = oracle.combine(p["dst"][n * wl.K:(n + m) * wl.K], wl.K, recv,
                                 wf[n * wl.K:(n + m) * wl.K], dt, dt)
            t_c += time.perf_counter() - t0
            out[:m] = res
            n += m
        sample = (f"dispatch of {ranks} of {wl.R} destination-rank windows ({t_d:.2f} s, "
                  f"scaled x{wl.R / ranks:.2f}); combine of {n} of {wl.n_tok} tokens "
                  f"({t_c:.2f} s, scaled x{wl.n_tok / n:.2f})")
        return t_d / ranks * wl.R, t_c * wl.n_tok / n, t_d + t_c, sample

    d_n, c_n, meas_n, sample_n = run(threads, 0.6 * budget_s)
    d_1, c_1, meas_1, sample_1 = run(1, 0.4 * budget_s)
    oracle.set_threads(threads)
    dc = nbytes["dispatch"] + nbytes["combine"]
    gbs_n = dc / (d_n + c_n) / 1e9
    gbs_1 = dc / (d_1 + c_1) / 1e9
    del recv, hid
    return {
        "value": round(gbs_n, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": (f"full plan of {wl.n_ent} entries, one thread ({t_plan * 1e3:.1f} ms); on "
                   f"{threads} threads: {sample_n}; combine reads its rows from the host "
                   f"receive buffer inside the timed call"),
        "ms": {"dispatch": round(d_n * 1e3, 1), "combine": round(c_n * 1e3, 1)},
        "one_thread": {"value": round(gbs_1, 3), "unit": "GB/s", "sample": sample_1,
                       "ms": {"dispatch": round(d_1 * 1e3, 1), "combine": round(c_1 * 1e3, 1)}},
        "plan_us": round(t_plan * 1e6, 1),
        "measured_s": round(t_plan + meas_n + meas_1, 2),
        "host": host_cpu(),
    }


def ceilings(wl, buf, stream, reps):
    """Practical HBM ceilings on the receive buffer itself (the 30 GB that
    dispatch writes and combine reads at K3): plain sequential reads, writes and
    copies (first half into second half) with this library's streaming kernels in
    both launch shapes (one resident grid; one workgroup per 16 KiB, and for
    writes also per 4 KiB), and torch's
    fill_ (the runtime's memset kernel) and copy_. GB/s of bytes moved (read +
    written), median of `reps` after one warm-up. `read`, `write` and `copy` are
    the best of each kind. The receive buffer is overwritten."""
    import numpy as np
    import torch
    from token_dispatch_amd import stream as ts

    flat = buf.view(-1).view(torch.uint8)
    n = flat.numel() // 32 * 32
    half = n // 2
    a, b = flat[:half], flat[half:2 * half]
    sink = torch.zeros(16, dtype=torch.uint8, device=buf.device)

    def timed(fn, nbytes):
        ms = []
        for i in range(reps + 1):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            if i:
                ms.append(e0.elapsed_time(e1))
        t = float(np.median(ms))
        return round(nbytes / (t * 1e-3) / 1e9, 1)

    chunk = 16384
    runs = {
        "read_grid": timed(lambda: ts.stream_read(flat[:n], sink, 0, stream), n),
        "read_16k": timed(lambda: ts.stream_read(flat[:n], sink, chunk, stream), n),
        "write_grid": timed(lambda: ts.stream_write(flat[:n], 0, 0, stream), n),
        "write_16k": timed(lambda: ts.stream_write(flat[:n], 0, chunk, stream), n),
        "write_4k": timed(lambda: ts.stream_write(flat[:n], 0, 4096, stream), n),
        "torch_fill": timed(lambda: flat[:n].fill_(0), n),
        "copy_grid": timed(lambda: ts.stream_copy(b, a, 0, stream), 2 * half),
        "copy_16k": timed(lambda: ts.stream_copy(b, a, chunk, stream), 2 * half),
        "torch_copy": timed(lambda: b.copy_(a), 2 * half),
    }
    out = {kind: max(v for k, v in runs.items() if kind in k) for kind in ("read", "write", "copy")}
    out["write"] = max(out["write"], runs["torch_fill"])
    # A write stream whose concurrent stores lie far apart (the resident grid
    # walking the buffer) slows down at some physical placements of the buffer,
    # as dispatch does; one whose stores lie in adjacent 4 KiB pieces does not.
    # Their ratio tells which placement this process's receive buffer got.
    out["placement_write_ratio"] = round(runs["write_grid"] / runs["write_4k"], 3)
    out.update({"runs": runs, "bytes": n, "unit": "GB/s", "reps": reps,
                "kernels": "moonep_stream_read / _write / _copy (include/moonep_stream.h): 16-byte "
                           "accesses, non-temporal loads; torch_fill = fill_(0), torch_copy = copy_"})
    return out


def ceiling_time_s(rd, wr, c):
    """Seconds a move of rd bytes read and wr bytes written takes at the measured
    pure-read and pure-write rates (no cost for mixing the two)."""
    return rd / (c["read"] * 1e9) + wr / (c["write"] * 1e9)


def move_directions(wl):
    """(bytes read, bytes written) of dispatch and combine, algorithmic."""
    row = wl.row_bytes
    return {"dispatch": (wl.n_tok * row + 4 * wl.n_ent, wl.n_ent * row),
            "combine": (wl.n_ent * row + 8 * wl.n_ent, wl.n_tok * row)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="k3",
                    choices=["tiny", "uniform", "zipf", "k3", "decode"])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--plan", default="waterfill", choices=["waterfill", "bounded"],
                    help="the plan each step computes: the water-fill (moonep_plan) or the one "
                         "bounded by B duplicates per rank (moonep_plan_bounded)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the CPU baseline sample")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the plain read / write / copy streams over the receive buffer "
                         "(the practical ceilings the moves are compared with)")
    ap.add_argument("--ceiling-reps", type=int, default=5)
    ap.add_argument("--alloc-order", default="model-first",
                    choices=["model-first", "activations-first"],
                    help="allocate the model state (weights, duplicate slots, gradients) before "
                         "the step's activations (hidden, receive buffer), as a training process "
                         "does, or after them; where the 30 GB receive buffer lands in physical "
                         "memory depends on it, and dispatch's speed on that")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay of the step (graph_ms_per_step)")
    ap.add_argument("--with-backward", action="store_true",
                    help="also time combine-backward (grad_out = out, y = recv) and "
                         "dispatch-backward (grad_recv = grad_y) in every step")
    ap.add_argument("--plan-iters", type=int, default=30,
                    help="plan calls timed alone after the steps, warm and cold each "
                         "(0: skip; also skipped with --copy-calibration)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help=f"after the timed steps, one plain device copy of {COPY_CAL_BYTES} bytes "
                         "(the reference dispatch for scaling HBM byte counters)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the HBM traffic summary from two rocprofv3 --pmc counter CSVs "
                         "of a run with --copy-calibration (same --steps/--warmup), then exit")
    ap.add_argument("--pmc-summary", nargs="+", metavar="DIR",
                    help="print a per-kernel summary of rocprofv3 --pmc / --kernel-trace CSVs "
                         "found under each DIR (one JSON object per DIR), then exit")
    ap.add_argument("--traffic-command", default="",
                    help="the profiled command, recorded in the traffic summary")
    args = ap.parse_args()

    if args.pmc_summary:
        print(json.dumps(pmc_summary(args.pmc_summary), indent=1, sort_keys=True))
        return

    if args.traffic_from:
        rec = traffic_from_pmc(args.traffic_from[0], args.traffic_from[1], args.steps,
                               args.warmup, args.traffic_command, args.workload, args.plan)
        with open(TRAFFIC_PATH, "w") as f:
            json.dump(rec, f, indent=1, sort_keys=True)
            f.write("\n")
        print(json.dumps(rec, indent=1, sort_keys=True))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this path has no multi-GPU mode "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import token_dispatch_amd as td
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = W.WORKLOADS[args.workload]
    print(f"# setup {wl.name}: R={wl.R} E={wl.E} K={wl.K} S={wl.S} H={wl.H} B={wl.B}",
          file=sys.stderr, flush=True)
    ids, w = W.make_routing(wl, args.seed)
    dims = td.Dims(wl.R, wl.E, wl.K, wl.S, wl.B, wl.dtype, wl.H)
    # by default the model state first (expert weights, duplicate slots,
    # gradients), then the step's activations, in the order a training process
    # allocates them; --alloc-order activations-first reverses that
    def model_state():
        ew = W.make_expert_weights(wl, args.seed, dev)
        dw = torch.empty((wl.R, wl.B) + tuple(wl.block_shape), dtype=ew.dtype, device=dev)
        return (ew, dw) + tuple(W.make_grads(wl, args.seed, dev))

    if args.alloc_order == "model-first":
        expert_w, dup_w, dup_g, home_g = model_state()
    hidden = W.make_hidden(wl, args.seed, dev)
    recv = torch.empty((wl.R, wl.SK, wl.H), dtype=hidden.dtype, device=dev)
    if args.alloc_order == "activations-first":
        expert_w, dup_w, dup_g, home_g = model_state()
    ids_d = torch.from_numpy(ids).to(dev)
    w_d = torch.from_numpy(w).to(dev)
    out = torch.empty_like(hidden)
    plan_buf = td.new_plan_buffer(dims, dev)
    if args.with_backward:
        grad_y = torch.empty_like(recv)
        grad_w = torch.empty((wl.R, wl.S, wl.K), dtype=torch.float32, device=dev)
        grad_h = torch.empty_like(hidden)
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()
    print("# inputs resident", file=sys.stderr, flush=True)

    ops = ["plan", "replicate", "dispatch", "combine", "reduce"]
    if args.with_backward:
        ops += ["combine_backward", "dispatch_backward"]

    plan_fn = td.moonep_plan_bounded if args.plan == "bounded" else td.moonep_plan

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        plan_fn(dims, ids_d, plan_buf)
        if ev:
            ev[1].record(stream)
        td.moonep_replicate(dims, plan_buf, expert_w, dup_w, wl.block_bytes)
        if ev:
            ev[2].record(stream)
        td.moonep_dispatch(dims, plan_buf, hidden, recv)
        if ev:
            ev[3].record(stream)
        td.moonep_combine(dims, plan_buf, recv, w_d, out)
        if ev:
            ev[4].record(stream)
        td.moonep_reduce_dup_grads(dims, plan_buf, dup_g, home_g, wl.block_elems)
        if ev:
            ev[5].record(stream)
        if args.with_backward:
            td.moonep_combine_backward(dims, plan_buf, out, w_d, recv, grad_y, grad_w)
            if ev:
                ev[6].record(stream)
            td.moonep_dispatch_backward(dims, plan_buf, grad_y, grad_h)
            if ev:
                ev[7].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"# warmup {args.warmup} done", file=sys.stderr, flush=True)

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(ops) + 1)]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    op_ms = {op: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs]))
             for j, op in enumerate(ops)}
    print(f"# timed {args.steps} steps: {ms_per_step:.3f} ms/step", file=sys.stderr, flush=True)
    graph = None
    if not args.no_graph and not args.copy_calibration:
        graph = graph_replay(step, stream, args.steps)
        print(f"# graph replay: {graph}", file=sys.stderr, flush=True)
    plan_lat = None
    if args.plan_iters > 0 and not args.copy_calibration:
        # the form moonep_plan takes for these dims, then the other one forced
        launches = td.moonep_plan_layout(dims).plan_launches
        plan_lat = plan_latency(plan_fn, dims, ids_d, plan_buf, stream, args.plan_iters)
        plan_lat["launches"] = launches
        other = td.PLAN_FOUR_LAUNCH if launches == 2 else td.PLAN_TWO_LAUNCH
        bflag = td.PLAN_BOUNDED if args.plan == "bounded" else 0
        plan_lat["other_form"] = plan_latency(
            lambda d, i, b: td.moonep_plan_ex(d, i, b, other | bflag), dims, ids_d, plan_buf,
            stream, args.plan_iters)
        plan_lat["other_form"]["launches"] = 4 if launches == 2 else 2
        plan_fn(dims, ids_d, plan_buf)  # leave the default form's plan in the buffer
        print(f"# plan latency: {plan_lat}", file=sys.stderr, flush=True)
    ceil = None
    if not args.no_ceiling and not args.copy_calibration:
        ceil = ceilings(wl, recv, stream, args.ceiling_reps)
        print(f"# ceilings: {ceil}", file=sys.stderr, flush=True)
    if args.copy_calibration:
        a = torch.empty(COPY_CAL_BYTES, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
        print(f"# copy calibration: {COPY_CAL_BYTES} bytes", file=sys.stderr, flush=True)

    v = td.plan_views(dims, plan_buf)
    n_dup = v["n_dup"].cpu().numpy()
    n_mat = int(np.minimum(n_dup, wl.B).sum())
    nl = int(v["n_list"][0])
    lb = v["list_b"][:nl].cpu().numpy()
    le = v["list_expert"][:nl].cpu().numpy()
    n_xm = int(np.unique(le[lb < wl.B]).size)
    seg = v["seg_ptr"].cpu().numpy()
    rows = seg[np.arange(wl.R), wl.G + n_dup]
    rank_maxvio_after = float(rows.max()) / wl.SK - 1.0
    status = int(v["status"][0])
    maxvio = float(v["maxvio"][0])
    nbytes = algorithmic_bytes(wl, n_mat, n_xm)
    gbs = {op: nbytes[op] / (op_ms[op] * 1e-3) / 1e9 for op in ops}
    dc_bytes = nbytes["dispatch"] + nbytes["combine"]
    dc_ms = op_ms["dispatch"] + op_ms["combine"]
    value = dc_bytes / (dc_ms * 1e-3) / 1e9

    dom = max(("dispatch", "combine"), key=lambda o: op_ms[o])
    src_hash = kernel_source_hash()
    traffic = traffic_for(dom, args.workload, args.plan)
    # one C-ABI call is n back-to-back launches of the kernel over token chunks;
    # the events bracket the call, so a launch takes the call's time over n on
    # average and moves the call's bytes over n on average
    n_launch = td.moonep_launch_count(dims, td.OP_DISPATCH if dom == "dispatch" else td.OP_COMBINE)
    roofline = {"bound": "hbm", "achieved": round(gbs[dom], 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(gbs[dom] / HBM_PEAK_GBS, 4),
                "traffic": None if traffic is None else round(traffic / n_launch),
                "kernel": f"k_{dom}", "kernel_source_hash": kernel_source_hash(OP_SOURCES[dom]),
                "launches_per_call": n_launch,
                "algorithmic_bytes_per_launch": round(nbytes[dom] / n_launch),
                "avg_launch_ms": round(op_ms[dom] / n_launch, 5),
                "algorithmic_bytes_per_call": nbytes[dom],
                "call_ms": round(op_ms[dom], 4),
                "launch": f"moonep_{dom} enqueues {n_launch} launches of k_{dom} over token "
                          "chunks; per-launch figures are the call's over that count"}

    if ceil is not None:
        # each move against the time its read and written bytes take at the pure
        # read and write rates of the same buffer (direction mixing not charged)
        dirs = move_directions(wl)
        t_dc = 0.0
        fr = {}
        for op in ("dispatch", "combine"):
            t = ceiling_time_s(*dirs[op], ceil)
            t_dc += t
            fr[op] = round(t / (op_ms[op] * 1e-3), 4)
        ceil["dispatch_combine_gbs"] = round(dc_bytes / t_dc / 1e9, 1)
        ceil["frac_of_ceiling"] = dict(fr, dispatch_combine=round(value / (dc_bytes / t_dc / 1e9), 4))
        ceil["frac_of_peak"] = {op: round(gbs[op] / HBM_PEAK_GBS, 4) for op in ops}
        roofline["frac_of_ceiling"] = fr[dom]
    cpu = None
    if not args.no_cpu_baseline:
        print("# cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, ids, w, hidden, args.cpu_budget)

    rec = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16"
        if wl.dtype == W.BF16 else "f32", "data": "synthetic",
        "config": {"workload": f"{wl.name}: R={wl.R} virtual ranks, E={wl.E}, K={wl.K}, "
                               f"S={wl.S}, H={wl.H}, B={wl.B}, weight block "
                               f"{'x'.join(map(str, wl.block_shape))}",
                   "routing": wl.routing, "seed": args.seed, "plan": args.plan,
                   "alloc_order": args.alloc_order,
                   "parallelism": "ep (virtual, 1 GPU)"},
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "plan_us": round(op_ms["plan"] * 1e3, 2), "plan_latency_us": plan_lat,
        "graph": graph,
        "op_ms": {k: round(x, 4) for k, x in op_ms.items()},
        "op_gbs": {k: round(x, 1) for k, x in gbs.items()},
        "maxvio_before": round(maxvio, 4), "rank_maxvio_after": rank_maxvio_after,
        "dups_per_rank_max": int(n_dup.max()), "dups_total": int(n_dup.sum()), "B": wl.B,
        "dups_materialised": n_mat, "experts_with_dups": n_xm,
        "status": status, "kernel_source_hash": src_hash,
        "roofline": roofline, "ceiling": ceil, "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
