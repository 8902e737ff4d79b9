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


def test_cold_sets_exceed_twice_the_cache_per_graph():
    """Each timed graph rotates through enough sets that the bytes it touches
    between two uses of a set exceed twice the 256 MB Infinity Cache."""
    w = inputs.WORKLOADS["dsv3_decode"]
    nb = bench.algorithmic_bytes(w)
    for part in ("dispatch", "combine"):
        S = bench.sets_for(nb[part], 64)
        assert S * nb[part] >= 2 * bench.MALL_BYTES
        assert (S - 1) * nb[part] < 2 * bench.MALL_BYTES  # no more than needed
    assert bench.sets_for(nb["dispatch"], 64) == 33
    # a launch that alone exceeds the cache still alternates two sets
    assert bench.sets_for(1 << 30, 64) == 2


def test_per_launch_statistics():
    st = bench.summarize([4.0, 5.0, 4.5, 4.4, 4.6], 33, 33)
    assert st["us"] == 4.5 and st["launches"] == [33, 66] and st["sets"] == 33
    assert 4.0 <= st["p10"] <= st["us"] <= st["p90"] <= 5.0


def test_decode_payload_matches_the_worked_size():
    # DeepSeek-V3 decode: 128 tokens x 8 rows x 7168 bf16 values = 14,680,064 bytes
    # each way; with the token rows (1,835,008 bytes) 16,515,072
    w = inputs.WORKLOADS["dsv3_decode"]
    assert bench.payload_bytes(w) == 14_680_064
    assert bench.algorithmic_bytes(w)["dispatch"] - w.tokens * 8 * w.k == 16_515_072


def test_tokens_option_resizes_the_workload():
    """--tokens T: the named workload at T tokens per source, a fixed capacity
    resized by the same one-sender bound, packed regions kept packed, and a
    profile tag of its own (committed figures are for the workload's size)."""
    args = bench.parse(["--workload", "dsv3_decode", "--tokens", "512"])
    w = bench.workload_of(args)
    assert (w.T, w.C, w.H, w.E, w.k, w.N) == (512, 512 * 8, 7168, 256, 8, 32)
    assert bench.profile_tag(args) == "dsv3_decode_T512"
    p = bench.workload_of(bench.parse(["--workload", "skewed_prefill", "--tokens", "100"]))
    assert (p.T, p.C, p.zipf) == (100, 0, 1.2)
    kimi = bench.workload_of(bench.parse(["--workload", "kimi_k2_decode", "--tokens", "64"]))
    assert kimi.C == 64 * 8  # min(k, E/N) = min(8, 24)
    assert bench.workload_of(bench.parse([])) == inputs.WORKLOADS["dsv3_decode"]
    with pytest.raises(ValueError):
        inputs.with_tokens(inputs.WORKLOADS["tiny"], 0)


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
    tm = d["timing"]
    for part in ("route", "dispatch", "combine", "step"):
        assert tm[part]["p10"] <= tm[part]["us"] <= tm[part]["p90"], part
        n1, n2 = tm[part]["launches"]
        assert n2 == 2 * n1 and n1 % tm[part]["sets"] == 0 and n1 >= 5
    assert d["dispatch_us"] == tm["dispatch"]["us"]
    # the adjacent paths timed in the default run
    nx = d["next"]
    assert set(nx) == {"combine_partial", "split", "route_grouped"}
    assert nx["combine_partial"]["send_us"] > 0 and nx["combine_partial"]["recv_us"] > 0
    assert nx["split"]["dispatch_recv_us"] > 0 and nx["split"]["combine_send_us"] > 0
    assert nx["route_grouped"]["route_us"] > 0
    # the floors, with the dispatch's own grid handed its rows
    fl = d["stream_floor"]
    assert fl["read_us"] > 0 and fl["write_us"] > 0 and fl["empty_launch_us"] > 0
    ds = fl["dispatch_shape"]
    for key in ("fill_dense_us", "copy_dense_us", "fill_rows_us", "copy_rows_us"):
        assert ds[key] > 0, key
    assert abs(ds["dispatch_over_copy_rows"] - d["dispatch_us"] / ds["copy_rows_us"]) < 2e-3
    assert fl["dispatch_io_us"] > 0 and fl["combine_io_us"] > 0
    assert abs(fl["io_floor_sum_us"] - fl["dispatch_io_us"] - fl["combine_io_us"]) < 2e-3
    assert abs(fl["dispatch_over_io_floor"] - d["dispatch_us"] / fl["dispatch_io_us"]) < 2e-3
    cs = fl["combine_shape"]
    assert cs["gather_rows_us"] > 0 and cs["gather_dense_us"] > 0
    assert abs(cs["combine_over_gather_rows"] - d["combine_us"] / cs["gather_rows_us"]) < 2e-3
    rl = d["roofline"]
    assert rl["timing"].startswith("HIP events")


@pytest.mark.gpu
def test_bench_timeline_line():
    """bench.py --timeline (tiny workload): one JSON line with the dispatch's
    and the combine's phases from the tracing library, percentiles ordered,
    one record per wave of each launch."""
    print("[case] bench.py --timeline tiny workload", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny",
                        "--timeline", "--launches", "8"],
                       capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    assert d["workload"] == "tiny" and d["launches"] == 8
    for part, phases in bench.TRACE_PHASES.items():
        t = d["timeline"][part]
        got = t["phases_us"]
        assert list(got) == [p for p in phases if not p.endswith("_")]
        for v in got.values():
            assert 0 <= v["p10"] <= v["p50"] <= v["p90"] <= v["max"]
        assert t["records_per_launch"] > 0
    assert d["timeline"]["dispatch"]["metadata_block_us"]["done_p50"] > 0


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
