"""bench.py host logic without a GPU: the one-GPU refusal, and the HBM-traffic
summary that turns rocprofv3 counter folders into bytes per launch."""
from __future__ import annotations

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
          "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
          "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
          "Counter_Value", "Start_Timestamp", "End_Timestamp"]
MAIN = "void smla::smla_rows_kernel<false, 512, 16, false>(smla::FwdParams)"
COMBINE = "void smla::smla_combine_kernel<false, 1>(smla::FwdParams)"
COPY = "void at::native::vectorized_elementwise_kernel<4, MulFunctor<float> >(int)"


def write_counters(folder, rows):
    """rows: (dispatch, kernel, counter, value) -- several rows of one dispatch
    and counter are instances that the summary adds up."""
    os.makedirs(folder, exist_ok=True)
    with open(os.path.join(folder, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for d, k, c, v in rows:
            w.writerow({f: 0 for f in FIELDS} | {"Dispatch_Id": d, "Kernel_Name": k,
                                                  "Counter_Name": c, "Counter_Value": v})


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_traffic_summary_scales_counters_by_the_copy(tmp_path, monkeypatch):
    # profiles go to a scratch root; the kernel sources (hashed) stay the real ones
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    os.symlink(os.path.join(ROOT, "sparse_mla_attention_03_amd"), tmp_path / "sparse_mla_attention_03_amd")
    # the main kernel: two dispatches, counters split over two instances each;
    # the merge kernel and other kernels must be ignored
    kf = tmp_path / "kf"
    write_counters(kf, [(1, MAIN, "FETCH_SIZE", 300.0), (1, MAIN, "FETCH_SIZE", 700.0),
                        (2, MAIN, "FETCH_SIZE", 500.0), (2, MAIN, "FETCH_SIZE", 500.0),
                        (3, COMBINE, "FETCH_SIZE", 9e9), (4, COPY, "FETCH_SIZE", 9e9)])
    kw = tmp_path / "kw"
    write_counters(kw, [(1, MAIN, "WRITE_SIZE", 40.0), (2, MAIN, "WRITE_SIZE", 60.0),
                        (3, COMBINE, "WRITE_SIZE", 9e9)])
    # a copy of 1 MiB read and written: 512 fetch units (2 KiB each), 1024 write units (1 KiB)
    cf = tmp_path / "cf"
    write_counters(cf, [(7, COPY, "FETCH_SIZE", 512.0), (8, COPY, "FETCH_SIZE", 512.0),
                        (9, MAIN, "FETCH_SIZE", 1.0)])
    cw = tmp_path / "cw"
    write_counters(cw, [(7, COPY, "WRITE_SIZE", 1024.0)])
    bench.traffic_summary("unit_workload", [str(kf), str(kw), str(cf), str(cw)], 1 << 20)
    rec = json.load(open(tmp_path / "profiles" / "traffic_unit_workload.json"))
    assert rec["dispatches"] == [2, 2]
    assert rec["fetch_size_per_dispatch"] == 1000.0 and rec["write_size_per_dispatch"] == 50.0
    assert rec["read_bytes_per_unit"] == 2048.0 and rec["write_bytes_per_unit"] == 1024.0
    assert rec["hbm_read_bytes_per_launch"] == 1000 * 2048
    assert rec["hbm_write_bytes_per_launch"] == 50 * 1024
    assert rec["hbm_bytes_per_launch"] == 1000 * 2048 + 50 * 1024
    assert rec["kernels"] == [MAIN]
    # reported while the kernel sources are the ones the counters were taken on
    assert bench.traffic_from_profiles("unit_workload", 0) == 1000 * 2048 + 50 * 1024
    rec["kernel_source_hash"] = "0" * 16
    json.dump(rec, open(tmp_path / "profiles" / "traffic_unit_workload.json", "w"))
    assert bench.traffic_from_profiles("unit_workload", 0) is None
    assert bench.traffic_from_profiles("no_such_workload", 0) is None


def test_missing_counter_rows_are_an_error(tmp_path):
    f = tmp_path / "empty"
    write_counters(f, [(1, COPY, "FETCH_SIZE", 1.0)])
    with pytest.raises(RuntimeError):
        bench._counter_per_dispatch(str(f), "FETCH_SIZE", lambda k: "smla_" in k)


def test_kernel_source_hash_is_stable():
    assert bench.kernel_source_hash() == bench.kernel_source_hash()
    assert len(bench.kernel_source_hash()) == 16


def test_kernel_source_hash_covers_the_forward_sources():
    csrc = os.path.join(ROOT, "sparse_mla_attention_03_amd", "csrc")
    listed = {f for f in os.listdir(csrc) if f.endswith((".hip", ".h"))}
    # every source except the fused RoPE / cache write's own file and the
    # device-ceiling probes (a library of their own)
    assert set(bench.FWD_SOURCES) == listed - {"smla_rope_cache.hip", "smla_ceiling.hip"}
