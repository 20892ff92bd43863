"""Host logic of bench.py without a GPU: the one-GPU guard, kernel-name
parsing, the algorithmic work it prices the dominant kernel at, and the
ingestion of rocprofv3 counter files into traffic figures."""

import csv
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from synth import WORKLOADS  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_kernel_short_names():
    assert bench.kernel_short_name(
        "void moe::k_expert_gemm<0, 3, 8, 1, 5>(unsigned short const*, int)") == \
        "k_expert_gemm<0, 3, 8, 1, 5>"
    assert bench.kernel_short_name(
        "void moe::(anonymous namespace)::k_x<moe::(anonymous namespace)::Geo<8, 1> >(int)") == \
        "k_x<Geo<8, 1> >"
    assert bench._matches("k_expert_gemm<0, 3, 8, 1, 5>", "k_expert_gemm<0>")
    assert not bench._matches("k_expert_gemm<1, 2, 16, 1, 5>", "k_expert_gemm<0>")
    assert bench._matches("k_gateup_stream<4, false, 1, 8>", "k_gateup_stream")


def test_dominant_kernel_work():
    d, F = 2048, 3072
    counts = np.array([2] * 11 + [0] * 5)  # 11 experts touched
    dec = bench.dominant_kernel(WORKLOADS[1], counts)
    assert dec["bound"] == "hbm" and dec["units"] == 11
    assert dec["per_unit"] == 2 * F * d * 2 == 25165824
    assert dec["work"] == 11 * 25165824 + 32 * d * 2 + 32 * F * 2
    f8 = bench.dominant_kernel(WORKLOADS[1], counts, fp8=True)
    assert f8["per_unit"] == 2 * F * d + 2 * F * 4
    pre = bench.dominant_kernel(WORKLOADS[3], np.full(16, 512))
    assert pre["bound"] == "mfma" and pre["units"] == 4096 * 2
    assert pre["work"] == 4096 * 2 * 4 * F * d
    lbytes, lflops, touched = bench.layer_work(WORKLOADS[2], np.full(16, 256))
    assert touched == 16 and lflops == 4096 * 6 * F * d + 2 * 4096 * d * 16
    assert lbytes == 16 * 3 * F * d * 2 + 2 * 4096 * d * 2 + 16 * d * 2 + 16 * 4 + d * 2


def test_dominant_kernel_of_the_fp32_layer():
    d, F = 256, 512
    c0 = bench.dominant_kernel(WORKLOADS[0], np.array([20, 0, 30, 14]))
    assert c0["kernel"] == "k_gateup_f32" and c0["bound"] == "hbm"
    assert c0["units"] == 3 and c0["work"] == 3 * 2 * F * d * 4
    lbytes, lflops, touched = bench.layer_work(WORKLOADS[0], np.array([20, 0, 30, 14]))
    assert touched == 3 and lbytes == 3 * 3 * F * d * 4 + 2 * 64 * d * 4 + 4 * d * 4 + 4 * 4 + d * 4
    assert bench.kernel_source_hash("k_gateup_f32")


def test_routing_check_counts_near_ties_and_mismatches():
    from oracle import moe_oracle as O
    from synth import make_inputs, gen
    inp = make_inputs(0)
    vals = gen.values_f32(inp)
    x = O.rmsnorm(vals["hidden"], vals["gain"], 1e-6)
    _, sc = O.router_scores(x, vals["w_router"], vals["bias"])
    sel, margin = O.select_topk(sc, 1)
    r = bench.routing_check(inp, sel)
    assert r["firm_mismatches"] == 0 and r["near_tie_flips"] == 0
    assert r["near_ties"] == int(np.sum(margin < O.MARGIN_TOL)) and r["tokens"] == 64
    bad = sel.copy()
    t = int(np.argmax(margin))          # the firmest token, routed elsewhere
    bad[t, 0] = (bad[t, 0] + 1) % 4
    assert bench.routing_check(inp, bad)["firm_mismatches"] == 1


def _write_run(dirname, rows):
    os.makedirs(dirname)
    with open(os.path.join(dirname, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for i, (kern, name, val) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": kern, "Counter_Name": name,
                        "Counter_Value": val})


def test_counter_ingestion_scales_by_the_copy(tmp_path, monkeypatch):
    # copy kernel: FETCH_SIZE reads half of the 1 GiB it moves, WRITE_SIZE all of it
    gib_kib = (1 << 30) / 1024
    _write_run(tmp_path / "copy_fetch", [("void at::neg_kernel(...)", "FETCH_SIZE", gib_kib / 2)])
    _write_run(tmp_path / "copy_write", [("void at::neg_kernel(...)", "WRITE_SIZE", gib_kib)])
    gu = "void moe::k_gateup_stream<4, false, 1, 8>(int)"
    _write_run(tmp_path / "c1_fetch", [(gu, "FETCH_SIZE", 1000.0), (gu, "FETCH_SIZE", 1200.0)])
    _write_run(tmp_path / "c1_write", [(gu, "WRITE_SIZE", 10.0), (gu, "WRITE_SIZE", 10.0)])
    out = tmp_path / "traffic.json"
    # an entry of a workload this directory does not profile is kept
    out.write_text(json.dumps({WORKLOADS[4].name: {"kernel": "k_expert_gemm<0>",
                                                   "bytes_per_launch": 7}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    bench.ingest_counters(str(tmp_path))
    t = json.loads(out.read_text())
    assert t["_calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert t["_calibration"]["write_factor"] == pytest.approx(1.0)
    rec = t[WORKLOADS[1].name]
    assert rec["kernel"] == "k_gateup_stream"
    assert rec["source_hash"] == bench.kernel_source_hash("k_gateup_stream")
    # mean 1100 KiB read x 2 + 10 KiB written x 1
    assert rec["bytes_per_launch"] == round(1100 * 1024 * 2) + round(10 * 1024)
    assert t[WORKLOADS[4].name]["bytes_per_launch"] == 7
