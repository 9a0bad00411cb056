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
OP_KERNELS = {"plan": ("k_count", "k_scan", "k_solve", "k_solve_bounded", "k_assign"),
              "replicate": ("k_replicate",),
              "dispatch": ("k_dispatch",), "combine": ("k_combine",), "reduce": ("k_reduce",)}
# (k_combine also serves the backward of dispatch, so traffic is only summed for
# runs without --with-backward)
COPY_CAL_BYTES = 1 << 30


def traffic_for(op: str):
    """HBM bytes per call of `op` from the committed counter summary, if it was
    taken on the current sources of that call's kernels; else None."""
    if not os.path.exists(TRAFFIC_PATH):
        return None
    with open(TRAFFIC_PATH) as f:
        rec = json.load(f)
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


def traffic_from_pmc(fetch_csv: str, write_csv: str, steps: int, warmup: int, command: str) -> dict:
    """HBM bytes per C-ABI call from two rocprofv3 --pmc runs of this benchmark
    (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each scaled by what the same
    counter reads for the plain device copy of COPY_CAL_BYTES that
    --copy-calibration enqueues after the timed steps."""
    rec = {"kernel_source_hash": kernel_source_hash(), "command": command,
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


def cpu_baseline(wl, ids, w, hidden_dev, y_dev, budget_s):
    """The oracle as it stands, single thread, on a bounded sample of the workload:
    the full plan; dispatch of whole destination-rank windows (the oracle streams
    its output by rank) for about half the budget; combine of the first n tokens
    for the rest. Times are scaled to the whole workload (R windows; all tokens)."""
    import numpy as np
    import torch
    import oracle
    import workloads as W

    t0 = time.perf_counter()
    p = oracle.plan(wl.R, wl.E, wl.K, wl.S, wl.B, ids)
    t_plan = time.perf_counter() - t0

    hid = hidden_dev.view(wl.n_tok, wl.H).cpu().view(torch.int16).numpy().view(np.uint16)
    t_disp, ranks = 0.0, 0
    while ranks < wl.R and (ranks == 0 or t_disp < 0.5 * budget_s):
        t0 = time.perf_counter()
        oracle.dispatch(p, wl.K, hid, ranks * wl.SK, (ranks + 1) * wl.SK)
        t_disp += time.perf_counter() - t0
        ranks += 1
    del hid

    def gather(t0, n):
        dsel = p["dst"][t0 * wl.K:(t0 + n) * wl.K].astype(np.int64)
        rows = y_dev.view(-1, wl.H)[torch.from_numpy(dsel).to(y_dev.device)].cpu()
        if wl.dtype == W.BF16:
            return rows.view(torch.int16).numpy().view(np.uint16)
        return rows.numpy()

    def comb(t0, n, y_rows):
        t0w = time.perf_counter()
        oracle.combine(np.arange(n * wl.K, dtype=np.int32), wl.K, y_rows,
                       w.reshape(-1)[t0 * wl.K:(t0 + n) * wl.K], wl.dtype, wl.dtype)
        return time.perf_counter() - t0w

    # consecutive batches of at most 8192 tokens (bounded host memory for the
    # gathered rows) until the rest of the budget is spent or every token is done
    left = max(0.0, budget_s - t_plan - t_disp)
    t_comb, n = 0.0, 0
    while n < wl.n_tok and (n == 0 or t_comb < left):
        m = min(8192, wl.n_tok - n)
        rows = gather(n, m)
        t_comb += comb(n, m, rows)
        n += m
        del rows

    nbytes = algorithmic_bytes(wl, 0, 0)
    t_d_full = t_disp / ranks * wl.R
    t_c_full = t_comb * wl.n_tok / n
    gbs = (nbytes["dispatch"] + nbytes["combine"]) / (t_d_full + t_c_full) / 1e9
    return {
        "value": round(gbs, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
        "sample": (f"full plan of {wl.n_ent} entries ({t_plan * 1e3:.1f} ms); dispatch of "
                   f"{ranks} of {wl.R} destination-rank windows ({t_disp:.2f} s, scaled x"
                   f"{wl.R / ranks:.2f}); combine of {n} of {wl.n_tok} tokens ({t_comb:.2f} s, "
                   f"scaled x{wl.n_tok / n:.1f})"),
        "plan_us": round(t_plan * 1e6, 1),
        "measured_s": round(t_plan + t_disp + t_comb, 2),
        "host": host_cpu(),
    }


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
    ap.add_argument("--traffic-command", default="",
                    help="the profiled command, recorded in the traffic summary")
    args = ap.parse_args()

    if args.traffic_from:
        rec = traffic_from_pmc(args.traffic_from[0], args.traffic_from[1], args.steps,
                               args.warmup, args.traffic_command)
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
    # model state first (expert weights, duplicate slots, gradients), then the
    # step's activations, in the order a training process allocates them
    expert_w = W.make_expert_weights(wl, args.seed, dev)
    dup_w = torch.empty((wl.R, wl.B) + tuple(wl.block_shape), dtype=expert_w.dtype, device=dev)
    dup_g, home_g = W.make_grads(wl, args.seed, dev)
    ids_d = torch.from_numpy(ids).to(dev)
    w_d = torch.from_numpy(w).to(dev)
    hidden = W.make_hidden(wl, args.seed, dev)
    recv = torch.empty((wl.R, wl.SK, wl.H), dtype=hidden.dtype, device=dev)
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
        plan_lat = plan_latency(plan_fn, dims, ids_d, plan_buf, stream, args.plan_iters)
        print(f"# plan latency: {plan_lat}", file=sys.stderr, flush=True)
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
    traffic = traffic_for(dom)
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

    cpu = None
    if not args.no_cpu_baseline:
        print("# cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, ids, w, hidden, recv, args.cpu_budget)

    rec = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16"
        if wl.dtype == W.BF16 else "f32", "data": "synthetic",
        "config": {"workload": f"{wl.name}: R={wl.R} virtual ranks, E={wl.E}, K={wl.K}, "
                               f"S={wl.S}, H={wl.H}, B={wl.B}, weight block "
                               f"{'x'.join(map(str, wl.block_shape))}",
                   "routing": wl.routing, "seed": args.seed, "plan": args.plan,
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
        "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
