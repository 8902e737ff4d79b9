"""The benchmark's command-line contract and byte accounting.

CPU: --gpus above 1 is refused with a message; the algorithmic bytes are the
payload the method must move (k rows per token each way, bf16 or fp8 with
its scales) plus the per-pair metadata.  GPU: one short run on the tiny
workload prints one JSON line with every field the contract names.
"""
import json
import os
import subprocess
import sys

import pytest

import bench
from combine_moe_dispatch_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("name", inputs.WORKLOAD_ORDER)
def test_algorithmic_bytes_are_payload_plus_metadata(name):
    w = inputs.WORKLOADS[name]
    nb = bench.algorithmic_bytes(w)
    payload = w.tokens * w.k * bench.nbytes_row(w)  # k rows each way
    x_or_out = w.tokens * 2 * w.H                       # the token rows in or out
    meta = w.tokens * 8 * w.k                           # ids + rows, or rows + weights
    assert nb["dispatch"] == payload + x_or_out + meta
    assert nb["combine"] == payload + x_or_out + meta
    assert bench.payload_bytes(w) == payload


def test_decode_payload_matches_the_worked_size():
    # DeepSeek-V3 decode: 128 tokens x 8 rows x 7168 bf16 values = 14,680,064 bytes
    # each way; with the token rows (1,835,008 bytes) 16,515,072
    w = inputs.WORKLOADS["dsv3_decode"]
    assert bench.payload_bytes(w) == 14_680_064
    assert bench.algorithmic_bytes(w)["dispatch"] - w.tokens * 8 * w.k == 16_515_072


@pytest.mark.gpu
def test_bench_prints_one_contract_line():
    print("[case] bench.py tiny workload", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny",
                        "--steps", "5", "--warmup", "1", "--cpu-seconds", "0.2", "--no-warm"],
                       capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 1
    assert d["config"]["workload"] == "tiny"
    assert d["value"] > 0 and d["ms_per_step"] > 0
    rl = d["roofline"]
    assert rl["bound"] == "hbm" and rl["unit"] == "GB/s" and rl["peak"] == 8000.0
    assert abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-3
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0
    assert d["device_status"] == 0
    # the adjacent paths timed in the default run
    nx = d["next"]
    assert set(nx) == {"combine_partial", "split", "route_grouped"}
    assert nx["combine_partial"]["send_us"] > 0 and nx["combine_partial"]["recv_us"] > 0
    assert nx["split"]["dispatch_recv_us"] > 0 and nx["split"]["combine_send_us"] > 0
    assert nx["route_grouped"]["route_us"] > 0


@pytest.mark.gpu
def test_bench_flag_paths_run():
    """The two-stage combine, the split timing and the group-limited router
    as the main path of a bench run (tiny workload)."""
    print("[case] bench.py tiny workload with --combine two-stage --split --groups 4", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny",
                        "--steps", "5", "--warmup", "1", "--no-cpu-baseline", "--no-warm",
                        "--no-floor", "--combine", "two-stage", "--split", "--groups", "4",
                        "--topk-groups", "2"],
                       capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads([l for l in r.stdout.splitlines() if l.strip()][-1])
    assert d["config"]["combine"].startswith("sender-side")
    assert d["config"]["router"].startswith("group-limited")
    assert d["two_stage_combine"]["send_us"] > 0 and d["split"]["dispatch_recv_us"] > 0
    assert d["device_status"] == 0
