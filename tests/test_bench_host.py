"""Host logic of bench.py: algorithmic work figures and the rocprofv3 summary's attribution of
dispatches to stages (no GPU: synthetic rocprofv3-style csv rows)."""
import csv
import json
import os

import pytest

import bench
from hymba_synth import ABLATION_300M, SWA_8K, TINY_F32, workload


def test_visible_keys_matches_brute_force():
    for M, W, T in [(3, 4, 10), (0, 1, 5), (2, 0, 7), (5, 16, 9)]:
        s = workload(TINY_F32).shape.with_(n_meta=M, window=W)
        brute = sum(M + (i + 1 if W == 0 else min(i + 1, W)) for i in range(T))
        assert bench.visible_keys(s, T) == brute


def test_prefill_work_stages():
    s = workload(SWA_8K).shape
    w = bench.prefill_work(s, 16, 8192)
    assert set(w) == {"in_proj", "attention", "w_o", "out_proj", "ssm", "epilogue", "convert"}
    R = 16 * 8192
    assert w["in_proj"] == ("mfma", 2.0 * R * s.d_model * s.n_in)
    assert w["epilogue"] == ("hbm", float(R * s.d_inner * 2 * 4))
    assert "kv_write" in bench.prefill_work(workload(ABLATION_300M).shape, 8, 2048)


def _trace_rows():
    seq = ["convert_kernel<a>", "Cijk_gemm_ssm", "convert_kernel<b>", "selective_scan_kernel<h,16,8>",
           "Cijk_gemm_attn", "swa_meta_attn_kernel<h>", "Cijk_gemm", "epilogue_kernel<h>", "Cijk_gemm"]
    rows, d, t = [], 0, 0
    # one small meta pass, then three timed calls, then the copy probe
    for grid, calls in (("64", 1), ("4096", 3)):
        for _ in range(calls):
            for k in seq:
                dur = {"Cijk_gemm": 100, "Cijk_gemm_ssm": 60, "Cijk_gemm_attn": 40,
                       "swa_meta_attn_kernel<h>": 50}.get(k, 10) * (1 if grid == "64" else 10)
                rows.append({"Dispatch_Id": str(d), "Kernel_Name": k, "Grid_Size": grid,
                             "Start_Timestamp": str(t), "End_Timestamp": str(t + dur * 1000)})
                d += 1
                t += dur * 1000 + 5
    rows.append({"Dispatch_Id": str(d), "Kernel_Name": "vectorized_elementwise_kernel<neg_kernel>",
                 "Grid_Size": "9", "Start_Timestamp": "0", "End_Timestamp": "1000"})
    return rows


def test_dispatch_labels():
    lab = [st for st, _ in bench._label(_trace_rows())]
    assert lab[:9] == ["convert", "in_proj", "convert", "ssm", "in_proj", "attention", "w_o", "epilogue",
                       "out_proj"]
    assert lab[-1] == "copy_probe"
    g = bench._main_groups(bench._label(_trace_rows()),
                           lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    assert g["in_proj"][1:] == ("several", 3, 1000.0)   # two projection GEMMs per call summed
    assert g["w_o"][1:] == ("4096", 3, 1000.0)
    assert g["attention"][2:] == (3, 500.0)
    assert g["convert"][2:] == (3, 200.0)      # two conversion kernels summed


def _write(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def test_summary_traffic_scaling(tmp_path):
    rows = _trace_rows()
    _write(str(tmp_path / "trace" / "host" / "1_kernel_trace.csv"), rows)
    fetch, write = [], []
    for r in rows:
        k = bench._kernel_stage(r["Kernel_Name"])
        big = r["Grid_Size"] != "64"
        f = 2 * 1024 ** 2 if k == "copy_probe" else (100.0 if big else 1.0)   # KiB: the probe reads 2x too much
        base = {"Dispatch_Id": r["Dispatch_Id"], "Kernel_Name": r["Kernel_Name"], "Grid_Size": r["Grid_Size"]}
        fetch.append(dict(base, Counter_Name="FETCH_SIZE", Counter_Value=str(f)))
        write.append(dict(base, Counter_Name="WRITE_SIZE", Counter_Value=str(f / 2)))
    _write(str(tmp_path / "fetch" / "h" / "1_counter_collection.csv"), fetch)
    _write(str(tmp_path / "write" / "h" / "1_counter_collection.csv"), write)
    out_txt, out_json = str(tmp_path / "s.txt"), str(tmp_path / "t.json")
    cmd = {"title": "t", "trace": "x", "summary": "y"}
    bench.summarize_rocprof(str(tmp_path / "trace"), None, str(tmp_path / "fetch"), str(tmp_path / "write"), cmd,
                            out_txt, out_json)
    t = json.load(open(out_json))
    assert t["copy_probe"]["fetch_scale"] == pytest.approx(0.5)
    assert t["copy_probe"]["write_scale"] == pytest.approx(1.0)
    # 100 KiB fetched (x0.5) + 50 KiB written (x1.0)
    assert t["attention"]["bytes_per_launch"] == pytest.approx(100 * 1024 * 0.5 + 50 * 1024)
    assert t["attention"]["source_sha256"] == bench.source_sha("attention")
    assert "in_proj" in open(out_txt).read()


def test_griffin_summary_attribution(tmp_path):
    """Each 8K conv dispatch anchors one prefill call; its neighbours in dispatch order are the
    x conversion and input GEMM, then the gate GEMM, RG-LRU, output GEMM and y conversion."""
    seq = [("convert_kernel<bf16,f16>", 100), ("Cijk_in", 1300), ("griffin_conv_kernel<h>", 180),
           ("Cijk_gate", 1500), ("rglru_kernel<h,8>", 660), ("Cijk_out", 700), ("convert_kernel<f16,bf16>", 110)]
    rows, t, d = [], 0, 0
    for call in range(3):
        for name, us in seq:
            grid = "2097152" if "conv" in name and "griffin" in name else "4096"
            rows.append({"Dispatch_Id": str(d), "Kernel_Name": name, "Grid_Size_X": grid, "Grid_Size_Y": "1",
                         "Grid_Size_Z": "1", "Start_Timestamp": str(t), "End_Timestamp": str(t + us * 1000)})
            t += us * 1000 + 10
            d += 1
    # a decode call afterwards: a small conv grid that must not be picked
    for name, us in seq:
        grid = "256" if "griffin_conv" in name else "64"
        rows.append({"Dispatch_Id": str(d), "Kernel_Name": name, "Grid_Size_X": grid, "Grid_Size_Y": "1",
                     "Grid_Size_Z": "1", "Start_Timestamp": str(t), "End_Timestamp": str(t + 5000)})
        t += 5010
        d += 1
    _write(str(tmp_path / "tr" / "h" / "1_kernel_trace.csv"), rows)
    out = str(tmp_path / "g.txt")
    bench.summarize_griffin(str(tmp_path / "tr"), None, {"title": "t", "trace": "x", "summary": "y"}, out)
    txt = open(out).read()
    got = {l.split()[0]: float(l.split()[2]) for l in txt.splitlines()
           if l.split() and l.split()[0] in ("in_proj", "conv", "gate_proj", "rglru", "out_proj")}
    assert got == {"in_proj": 1300.0, "conv": 180.0, "gate_proj": 1500.0, "rglru": 660.0, "out_proj": 700.0}


def test_decode_summary_groups_by_kernel_and_grid(tmp_path):
    """Kernels with the same name but different grids (the two projections' GEMMs) stay apart;
    the median of each group is reported and groups are ordered by total time."""
    rows, t, d = [], 0, 0
    for call in range(5):
        for name, grid, us in [("decode_attn_mfma_kernel<5>", "320", 33 + call), ("rows_gemm_kernel", "1024", 11),
                               ("rows_gemm_kernel", "2048", 12), ("ssm_step_kernel", "4096", 13)]:
            rows.append({"Dispatch_Id": str(d), "Kernel_Name": name, "Grid_Size_X": grid, "Grid_Size_Y": "1",
                         "Grid_Size_Z": "1", "Start_Timestamp": str(t), "End_Timestamp": str(t + us * 1000)})
            t += us * 1000 + 10
            d += 1
    _write(str(tmp_path / "tr" / "h" / "1_kernel_trace.csv"), rows)
    out = str(tmp_path / "d.txt")
    bench.summarize_decode(str(tmp_path / "tr"), None, {"title": "t", "trace": "x", "summary": "y"}, out)
    body = [l.split() for l in open(out).read().splitlines() if l and l[0] == " " or (l and l[0].isdigit())]
    got = [(r[-1], r[3], int(r[0]), float(r[1])) for r in body if len(r) >= 5]
    assert got == [("decode_attn_mfma_kernel<5>", "320x1x1", 5, 35.0), ("ssm_step_kernel", "4096x1x1", 5, 13.0),
                   ("rows_gemm_kernel", "2048x1x1", 5, 12.0), ("rows_gemm_kernel", "1024x1x1", 5, 11.0)]
