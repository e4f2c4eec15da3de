"""The benchmark's host logic on the CPU: argument handling, the refusal of
more than one GPU, the counter summary (rocprofv3 CSV -> per-step HBM bytes,
calibrated by the copy), the staleness check of stored counters, and the
workloads' algorithmic byte counts."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from transformer_residual_add_amd import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_defaults():
    a = bench.parse_args([])
    assert a.gpus == 1 and a.steps > 0 and a.warmup >= 0 and a.workload == bench.HEADLINE
    assert bench.HEADLINE in W.WORKLOADS
    for name in bench.SWEEP:
        W.get(name)  # every sweep workload exists


def test_algorithmic_bytes():
    """Every streamed tensor once, a broadcast skip once, vectors once."""
    c2 = W.WORKLOADS["bert_base_8x128x768_f32"]
    assert c2.algorithmic_bytes() == 4 * 1024 * 768 * 4 + 3 * 768 * 4       # x, skip, res, out; g, b, bias
    c4 = W.WORKLOADS["bcast_64x512x4096_f32"]
    assert c4.algorithmic_bytes() == 2 * 32768 * 4096 * 4 + 512 * 4096 * 4 + 2 * 4096 * 4
    sm = W.EXTRA["softmax_attn_16x16x512x512_f16_padmask"]
    assert sm.algorithmic_bytes() == 2 * 131072 * 512 * 2 + 16 * 512 * 2    # data, out; mask rows once
    ba = W.EXTRA["biasadd_64x512x4096_f16"]
    assert ba.algorithmic_bytes() == 3 * 32768 * 4096 * 2 + 4096 * 2


def _write_run(root, name, counter, rows):
    d = os.path.join(root, f"{name}_{counter}")
    os.makedirs(d)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
        for kernel, value in rows:
            w.writerow([kernel, counter, value])


def test_counter_summary(tmp_path, monkeypatch):
    """Copy calibration (FETCH_SIZE reads half), medians for one kernel per
    step, sums over dispatches / steps for a step of several dispatches (the
    split-row pair, per batch of rows), other kernels (runtime copies)
    ignored; the kernel named is the automatic choice."""
    root = str(tmp_path)
    gib_kib = (1 << 30) / 1024
    _write_run(root, "copy1g", "FETCH_SIZE", [("skipln::copy_kernel", gib_kib / 2)] * 12)
    _write_run(root, "copy1g", "WRITE_SIZE", [("skipln::copy_kernel", gib_kib)] * 12)
    w = W.WORKLOADS["bert_base_8x128x768_f32"]
    half = w.algorithmic_bytes() / 2 / 1024
    _write_run(root, w.name, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 1e6)] +
               [("rowtile_kernel<skipln...>", half / 2)] * 11 + [("rowtile_kernel<skipln...>", 10 * half)])
    _write_run(root, w.name, "WRITE_SIZE", [("rowtile_kernel<skipln...>", half)] * 12)
    v = W.EXTRA["softmax_vocab_4096x128256_f16"]
    per_step = v.algorithmic_bytes() / 1024
    # 12 steps of 8 batches x 2 kernels: half the bytes read (FETCH_SIZE counts
    # half of them), half written by the second kernel of each batch
    _write_run(root, v.name, "FETCH_SIZE", [("_ZN6skipln_stats", per_step / 64)] * 96 +
               [("_ZN6skipln_apply", per_step / 64)] * 96)
    _write_run(root, v.name, "WRITE_SIZE", [("_ZN6skipln_apply", per_step / 16)] * 96)
    out = str(tmp_path / "counters.json")
    assert bench.summarize_counters(root, out, 12) == 0
    data = json.load(open(out))
    assert data["copy_calibration"]["fetch_scale"] == pytest.approx(2.0)
    e = {x["workload"]: x for x in data["entries"]}
    assert e[w.name]["traffic_over_algorithmic"] == pytest.approx(1.0, abs=2e-4)  # median, not the outlier
    assert e[v.name]["traffic_over_algorithmic"] == pytest.approx(1.0, abs=2e-4)
    assert e[v.name]["kernel"] == "softmax_regrow_f16"
    # a stored entry is used only while the kernel's sources are unchanged
    monkeypatch.setattr(bench, "COUNTERS", out)
    assert bench.counter_traffic(e[w.name]["kernel"], w.name) == e[w.name]["fetch_bytes"] + e[w.name]["write_bytes"]
    data["entries"][0]["source_sha256"] = "0" * 64
    json.dump(data, open(out, "w"))
    assert bench.counter_traffic(data["entries"][0]["kernel"], data["entries"][0]["workload"]) is None
    assert bench.counter_traffic("no_such_kernel", w.name) is None


def test_launch_config_arguments():
    a = bench.parse_args(["--launch-configs", "bcast_64x512x4096_f32", "--config=-1:0:2:1", "--config=7:1:1:0"])
    assert [bench.parse_config(c) for c in a.config] == [(-1, 0, 2, 1), (7, 1, 1, 0)]
    with pytest.raises(SystemExit):
        bench.parse_config("1:2:3")
    # a cyclic broadcast skip adds the skip-stationary tiling; both store policies each
    c4 = bench.default_configs(W.WORKLOADS["bcast_64x512x4096_f32"])
    assert (-1, 3, 2, 0) in c4 and (-1, 64, 2, 1) in c4 and len(c4) == 8
    c5 = bench.default_configs(W.WORKLOADS["rows65536_h8192_f16_mean100"])
    assert all(t != 2 for _, _, t, _ in c5) and len(c5) == 4


def test_config_counter_summary(tmp_path, monkeypatch, capsys):
    """Library dispatches are split by the plan in dispatch order (other
    kernels ignored, rows out of order sorted by Dispatch_Id), per-config
    medians scaled by the stored copy calibration; a plan that does not match
    the dispatch count is refused."""
    root = tmp_path / "pmc"
    cal = tmp_path / "counters.json"
    json.dump({"copy_calibration": {"fetch_scale": 2.0, "write_scale": 1.0}}, open(cal, "w"))
    monkeypatch.setattr(bench, "COUNTERS", str(cal))
    plan = {"workload": "w", "algorithmic_bytes": 3 * 1024 * 100,
            "plan": [{"label": "first", "config": None, "kernel": "k0", "dispatches": 3},
                     {"label": "second", "config": [-1, 0, 1, 0], "kernel": "k0", "dispatches": 3}]}
    plan_path = tmp_path / "plan.json"
    plan_path.write_text("[bench] log line\n" + json.dumps({"launch_configs": plan}) + "\n")
    for counter, values in (("FETCH_SIZE", [100, 100, 900, 200, 200, 200]), ("WRITE_SIZE", [100] * 6)):
        d = root / counter
        d.mkdir(parents=True)
        with open(d / "run_counter_collection.csv", "w", newline="") as fh:
            w = csv.writer(fh)
            w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
            w.writerow([1, "__amd_rocclr_copyBuffer", counter, 5])
            rows = [(i + 2, "void skipln::rowtile::rowtile_kernel<...>", counter, v) for i, v in enumerate(values)]
            for r in reversed(rows):
                w.writerow(r)
    assert bench.summarize_config_counters(str(root), str(plan_path)) == 0
    out = capsys.readouterr().out.splitlines()
    first = [ln for ln in out if ln.startswith("| first")][0]
    second = [ln for ln in out if ln.startswith("| second")][0]
    assert "204,800" in first and "102,400" in first and "| 1.000 |" in first   # median 100 KiB x 2, 100 KiB x 1
    assert "409,600" in second and "| 1.667 |" in second
    plan["plan"][1]["dispatches"] = 4
    plan_path.write_text(json.dumps(plan) + "\n")
    with pytest.raises(SystemExit):
        bench.summarize_config_counters(str(root), str(plan_path))
