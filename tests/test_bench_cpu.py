"""CPU tests of bench.py's own logic: the counter-CSV reduction behind
roofline.traffic, the algorithmic byte counts, and the one-GPU contract."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import workloads as W  # noqa: E402

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
          "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
          "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
          "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _write_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for did, name, kib in rows:
            r = {k: 0 for k in FIELDS}
            r.update({"Dispatch_Id": did, "Kernel_Name": name, "Counter_Name": counter,
                      "Counter_Value": kib})
            w.writerow(r)


def test_traffic_from_pmc_scales_by_the_calibration_copy(tmp_path):
    """Two calls (steps 1 + warm-up 1): dispatch = 2 launches per call, 1000 KiB
    each by the counter; a copy kernel before the library kernels is ignored, the
    first copy after the last library kernel is the calibration."""
    steps, warmup = 1, 1
    disp = "void moonep::(anonymous namespace)::k_dispatch<14, 3>(HIP_vector_type<unsigned int, 4u> const*)"
    comb = "void moonep::(anonymous namespace)::k_combine<14, true, true, false>(int)"
    plan = "moonep::(anonymous namespace)::k_assign(int const*)"
    copy = "__amd_rocclr_copyBuffer"
    cal_bytes = bench.COPY_CAL_BYTES
    rows_f = [(1, copy, 5.0)]  # an input upload: not the calibration
    rows_w = [(1, copy, 7.0)]
    did = 2
    for _ in range(steps + warmup):
        for name, f_kib, w_kib in ((plan, 3.0, 4.0), (disp, 1000.0, 2000.0), (disp, 1000.0, 2000.0),
                                   (comb, 4000.0, 100.0)):
            rows_f.append((did, name, f_kib))
            rows_w.append((did, name, w_kib))
            did += 1
    # the copy reads half of what it moves by this counter, writes all of it
    rows_f.append((did, copy, cal_bytes / 1024.0 / 2.0))
    rows_w.append((did, copy, cal_bytes / 1024.0))
    rows_f.append((did + 1, copy, 1.0))  # later copies are not the calibration
    rows_w.append((did + 1, copy, 1.0))
    fp, wp = tmp_path / "f.csv", tmp_path / "w.csv"
    _write_csv(fp, "FETCH_SIZE", rows_f)
    _write_csv(wp, "WRITE_SIZE", rows_w)
    rec = bench.traffic_from_pmc(str(fp), str(wp), steps, warmup, "cmd", "k3", "waterfill")
    assert rec["workload"] == "k3" and rec["plan"] == "waterfill"
    assert rec["fetch_size_scale"] == pytest.approx(2.0)
    assert rec["write_size_scale"] == pytest.approx(1.0)
    d = rec["ops"]["dispatch"]
    assert d["fetch_size_bytes_per_call"] == pytest.approx(2 * 1000.0 * 1024 * 2.0)
    assert d["write_size_bytes_per_call"] == pytest.approx(2 * 2000.0 * 1024)
    assert d["hbm_bytes_per_call"] == pytest.approx(d["fetch_size_bytes_per_call"] +
                                                    d["write_size_bytes_per_call"])
    assert rec["ops"]["combine"]["fetch_size_bytes_per_call"] == pytest.approx(4000.0 * 1024 * 2.0)
    assert rec["ops"]["plan"]["write_size_bytes_per_call"] == pytest.approx(4.0 * 1024)
    assert d["source_hash"] == bench.kernel_source_hash(bench.OP_SOURCES["dispatch"])


def test_traffic_is_used_only_for_matching_sources_workload_and_plan(tmp_path, monkeypatch):
    path = tmp_path / "t.json"
    good = bench.kernel_source_hash(bench.OP_SOURCES["dispatch"])
    path.write_text(json.dumps({"workload": "k3", "plan": "waterfill",
                                "ops": {"dispatch": {"source_hash": good, "hbm_bytes_per_call": 5.0},
                                        "combine": {"source_hash": "stale", "hbm_bytes_per_call": 6.0}}}))
    monkeypatch.setattr(bench, "TRAFFIC_PATH", str(path))
    assert bench.traffic_for("dispatch", "k3", "waterfill") == 5.0
    assert bench.traffic_for("combine", "k3", "waterfill") is None
    # counters taken on another workload or plan say nothing about this one
    assert bench.traffic_for("dispatch", "decode", "waterfill") is None
    assert bench.traffic_for("dispatch", "k3", "bounded") is None


def test_committed_traffic_summary_names_its_workload():
    with open(bench.TRAFFIC_PATH) as f:
        rec = json.load(f)
    assert rec["workload"] == "k3" and rec["plan"] == "waterfill"
    assert "--workload" not in rec["command"] and "--plan" not in rec["command"]


def test_algorithmic_bytes_by_hand():
    wl = W.WORKLOADS["k3"]
    row = 7168 * 2
    n_tok, n_ent = 32 * 4096, 32 * 4096 * 16
    b = bench.algorithmic_bytes(wl, n_mat=112, n_xm=94)
    assert b["dispatch"] == n_ent * row + n_tok * row + 4 * n_ent == 31_952_207_872
    assert b["combine"] == n_ent * row + n_tok * row + 8 * n_ent == 31_960_596_480
    block = 3 * 7168 * 512
    assert b["replicate"] == 2 * 112 * block * 2 == 4_932_501_504
    assert b["reduce"] == (112 + 2 * 94) * block * 4 == 13_212_057_600


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("name,dt", [("tiny", None), ("tiny", W.BF16)])
def test_cpu_baseline_runs_on_host_tensors(name, dt):
    """The CPU-baseline leg on host tensors, with fp32 rows (the tiny workload as
    given) and bf16 rows: it times the oracle and reports a positive rate."""
    import torch
    wl = W.WORKLOADS[name]
    if dt is not None:
        wl = wl.replace(dtype=dt)
    ids, w = W.make_routing(wl, 0)
    hidden = W.make_hidden(wl, 0)
    rec = bench.cpu_baseline(wl, ids, w, hidden, 0.2)
    assert rec["value"] > 0 and rec["kind"] == "oracle"
    assert rec["cores"] == bench.host_threads() >= 1
    assert rec["one_thread"]["value"] > 0
    assert "destination-rank windows" in rec["sample"] and "tokens" in rec["one_thread"]["sample"]
    assert set(rec["ms"]) == {"dispatch", "combine"}


def test_host_threads_follows_omp_num_threads(monkeypatch):
    monkeypatch.setenv("OMP_NUM_THREADS", "3")
    assert bench.host_threads() == 3
    monkeypatch.delenv("OMP_NUM_THREADS")
    assert bench.host_threads() == len(os.sched_getaffinity(0))


def test_ceiling_fractions_by_hand():
    """A move that takes exactly its read bytes at the read rate plus its written
    bytes at the write rate is at the ceiling."""
    wl = W.WORKLOADS["k3"]
    c = {"read": 7000.0, "write": 6800.0}
    dirs = bench.move_directions(wl)
    rd, wr = dirs["dispatch"]
    assert rd + wr == bench.algorithmic_bytes(wl, 0, 0)["dispatch"]
    assert bench.ceiling_time_s(rd, wr, c) == pytest.approx(rd / 7.0e12 + wr / 6.8e12)
    rd, wr = dirs["combine"]
    assert rd + wr == bench.algorithmic_bytes(wl, 0, 0)["combine"]


def test_pmc_summary_by_hand(tmp_path):
    """Counters are averaged per dispatch and per kernel class; latency is LEVEL
    over requests, requests in flight LEVEL over GRBM_GUI_ACTIVE times 8."""
    import csv as _csv
    d = tmp_path / "run"
    d.mkdir()
    name = "void moonep::(anonymous namespace)::k_combine<14, true, true, false>(int)"
    with open(d / "x_counter_collection.csv", "w", newline="") as f:
        w = _csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for did in (1, 2):
            w.writerow([did, name, "TCC_EA0_RDREQ_sum", 100.0])
            w.writerow([did, name, "TCC_EA0_RDREQ_LEVEL_sum", 5000.0 * did])
            w.writerow([did, name, "GRBM_GUI_ACTIVE", 800.0])
        w.writerow([3, "other_kernel(int)", "TCC_EA0_RDREQ_sum", 1.0])
    with open(d / "x_kernel_trace.csv", "w", newline="") as f:
        w = _csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writerow([name, 0, 1000])
        w.writerow([name, 0, 3000])
        w.writerow([name, 0, 2000])
    rec = bench.pmc_summary([str(d)])["run"]["k_combine"]
    assert rec["dispatches"] == 2 and rec["TCC_EA0_RDREQ_sum"] == 100.0
    assert rec["rdreq_latency_cycles"] == pytest.approx(75.0)
    assert rec["rdreq_in_flight"] == pytest.approx(7500.0 / 800.0 * 8)
    assert rec["median_us"] == pytest.approx(2.0)


def test_every_kernel_is_counted():
    """Every __global__ kernel of the library sources has a class in the counter
    summary, and every forward kernel belongs to one call's traffic (the backward
    kernels are summed only by runs without --with-backward)."""
    import re
    names = set()
    csrc = os.path.join(ROOT, "token_dispatch_amd", "csrc")
    for f in os.listdir(csrc):
        if f.endswith(".hip"):
            text = open(os.path.join(csrc, f)).read()
            names |= set(re.findall(r"__global__[^;{]*?\bvoid\s+(k_\w+)\s*\(", text))
    assert {"k_count", "k_plan_fused", "k_solve_bounded", "k_combine", "k_stream_copy"} <= names
    for n in names:
        assert n in bench.PMC_CLASSES, n
        if not n.startswith(("k_bwd", "k_stream")):
            assert any(n in ks for ks in bench.OP_KERNELS.values()), n
