"""bench.py --summarize-profile on small synthetic rocprofv3 outputs (CPU):
medians and means of the kernel trace per step part, the copy calibration
of FETCH_SIZE / WRITE_SIZE, the traffic ratio against the algorithmic bytes
of the bench line, and the figures file bench.py reads back."""
import csv
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(header)
        wr.writerows(rows)


def test_profile_summary(tmp_path):
    kt = tmp_path / "kt"
    names = {"route": "void moe::(anonymous namespace)::route_topk_kernel<4, false>(float const*)",
             "dispatch": "void moe::(anonymous namespace)::dispatch_fused_kernel<0, 2, 4, 2>(moe::P)",
             "combine": "void moe::(anonymous namespace)::combine_bf16_kernel<8, false>(int)"}
    durs = {"route": [3000, 3100, 3200], "dispatch": [4000, 4200, 4400, 9000],
            "combine": [4100, 4300, 4500]}
    rows, t = [], 1000
    for part, ds in durs.items():
        for d in ds:
            rows.append(["KERNEL_DISPATCH", names[part], t, t + d])
            t += d + 500
    _write(str(kt / "host" / "run_kernel_trace.csv"),
           ["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    cc_header = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    gib_kib = float(1 << 20)
    _write(str(tmp_path / "calf" / "run_counter_collection.csv"), cc_header,
           [["__amd_rocclr_copyBuffer", "FETCH_SIZE", gib_kib / 2]] * 5)
    _write(str(tmp_path / "calw" / "run_counter_collection.csv"), cc_header,
           [["__amd_rocclr_copyBuffer", "WRITE_SIZE", gib_kib]] * 5)
    _write(str(tmp_path / "fetch" / "run_counter_collection.csv"), cc_header,
           [[names["dispatch"], "FETCH_SIZE", 900.0], [names["combine"], "FETCH_SIZE", 7000.0],
            [names["route"], "FETCH_SIZE", 70.0]])
    _write(str(tmp_path / "write" / "run_counter_collection.csv"), cc_header,
           [[names["dispatch"], "WRITE_SIZE", 14000.0], [names["combine"], "WRITE_SIZE", 1750.0],
            [names["route"], "WRITE_SIZE", 8.0]])
    nb = {"route": 100000, "dispatch": 16000000, "combine": 17000000}
    (tmp_path / "bench.json").write_text(json.dumps(
        {"algorithmic_bytes": nb, "route_us": 3.0, "dispatch_us": 4.0, "combine_us": 4.3}) + "\n")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--summarize-profile",
                        "--workload", "dsv3_decode", "--trace-dir", str(kt),
                        "--fetch-dir", str(tmp_path / "fetch"), "--write-dir",
                        str(tmp_path / "write"), "--cal-fetch-dir", str(tmp_path / "calf"),
                        "--cal-write-dir", str(tmp_path / "calw"),
                        "--bench-json", str(tmp_path / "bench.json")],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    out = r.stdout
    # dispatch median of 4000, 4200, 4400, 9000 ns is 4.3 us; mean 5.4 us
    assert "| dispatch | dispatch_fused_kernel | 4.300 | 5.400 | 16000000 |" in out
    assert "FETCH_SIZE x 2.0000, WRITE_SIZE x 1.0000" in out
    # dispatch traffic: (900 * 2 + 14000) KiB
    assert f"| dispatch | {1024 * (900 * 2 + 14000):.0f} | 16000000 |" in out
    # event comparison: combine median 4.3 us against 4.3 us per launch
    assert "| combine | 4.300 | 4.300 | 1.000 |" in out

    # with --write-figures: the whole profile file and the figures file
    _write(str(kt / "host" / "run_kernel_stats.csv"),
           ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"],
           [[names["dispatch"], 4, 21600, 5400.0, 40.0, 4000, 9000],
            [names["combine"], 3, 12900, 4300.0, 30.0, 4100, 4500],
            ["at::native::other_kernel", 2, 100, 50.0, 1.0, 40, 60]])
    pdir = tmp_path / "profiles"
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--summarize-profile",
                        "--workload", "dsv3_decode", "--groups", "8", "--topk-groups", "4",
                        "--trace-dir", str(kt), "--bench-json", str(tmp_path / "bench.json"),
                        "--write-figures", "--profiles-dir", str(pdir)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    md = (pdir / "dsv3_decode_grouped_kernels_and_traffic.md").read_text()
    assert md.startswith("# dsv3_decode_grouped: kernel durations and HBM traffic")
    assert ("python3 bench.py --workload dsv3_decode --groups 8 --topk-groups 4 --steps 200 "
            "--warmup 20 > bench_line.json") in md
    # --stats rows of the path's kernels only, longest average first
    assert "| dispatch_fused_kernel<0, 2, 4, 2> | 4 | 5400 | 4000 | 9000 |" in md
    assert md.index("dispatch_fused_kernel<0, 2, 4, 2> | 4 |") < \
        md.index("combine_bf16_kernel<8, false> | 3 |")
    assert "other_kernel" not in md.split("## Kernel trace")[0]
    assert "| dispatch | dispatch_fused_kernel | 4.300 | 5.400 | 16000000 |" in md
    assert md.rstrip().endswith(json.dumps(json.loads((tmp_path / "bench.json").read_text())))
    fig = (pdir / "figures_dsv3_decode_grouped.txt").read_text()
    assert f"dispatch_source_sha = {bench.source_sha('dispatch')}" in fig
    assert "dispatch_rocprof_median_us = 4.300" in fig


def test_timeline_summary_on_synthetic_records():
    """bench.py --timeline's summary: phases in us from each launch's earliest
    entry (100 MHz ticks), pooled over launches, unwritten records ignored,
    the metadata block's waves reported apart."""
    import numpy as np
    phases = bench.TRACE_PHASES["dispatch"]
    recs = []
    for launch, base in enumerate((10_000, 55_000)):
        r = np.zeros((4 + 3, 8), np.int64)
        # metadata block (4 waves): enters first, done at +250 ticks
        for wv in range(4):
            r[wv, :6] = [base, base, base, base, base + 200, base + 250]
            r[wv, 7] = 1
        # two scatter waves, one record left unwritten
        r[4, :6] = base + np.array([10, 40, 70, 90, 200, 210])
        r[5, :6] = base + np.array([30, 60, 90, 110, 260, 270])
        r[4:6, 7] = 1
        r[6, :6] = base + 9999   # not written (word 7 == 0): ignored
        recs.append(r)
    out = bench.timeline_summary(recs, phases, first_slots=4)
    ph = out["phases_us"]
    assert ph["entry"]["max"] == 0.3 and ph["entry"]["p50"] == 0.2
    assert ph["rows_known"]["p50"] == 1.0 and ph["stores_done"]["max"] == 2.7
    assert out["metadata_block_us"] == {"entry_p50": 0.0, "done_p50": 2.5, "done_max": 2.5}
    assert out["last_done_us_p50"] == 2.7 and out["records_per_launch"] == 6
