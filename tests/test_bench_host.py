"""Host logic of bench.py that its reported figures rest on: the kernel names
the counter summaries key on, the copy-calibrated HBM bytes, the source-hash
check that voids stale traffic figures, and the algorithmic work per call.
No GPU needed: the counter files are synthetic CSVs of rocprofv3's layout."""
import csv
import json
import os
import shutil

import pytest

import bench
from workloads import get_workload

BUILD = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "_build", "tests", "bench_host")


def test_kernel_keys():
    k = bench._kernel_key
    assert k("void rtv::(anonymous namespace)::attend16_kernel<false, false, false>(rtv::AttendArgs)") == \
        "attend16_kernel<false, false, false>"
    assert k("void rtv::(anonymous namespace)::attend_kernel<64, true, true, true>(rtv::AttendArgs)") == \
        "attend_kernel<64, true, true, true>"
    assert k("void rtv::(anonymous namespace)::append_rope_quant_kernel<128, 3>(rtv::AppendArgs)") == \
        "append_rope_quant_kernel<128, 3>"
    assert k("rtv::(anonymous namespace)::factors_kernel(rtv::AttendArgs)") == "factors_kernel"
    assert k("__amd_rocclr_copyBuffer") == "copy"
    assert k("void at::native::vectorized_elementwise_kernel<4, ...>") is None


def _write_pmc(dirname, counter, rows):
    os.makedirs(dirname, exist_ok=True)
    with open(os.path.join(dirname, "pmc_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for disp, name, value in rows:
            w.writerow({"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_pmc_summary_calibrates_by_the_copy_kernel():
    """FETCH_SIZE of a 1 GiB copy reading half its bytes gives a factor of 2
    (taken from the largest copy dispatch); per-dispatch sums over counter
    instances are averaged over dispatches."""
    shutil.rmtree(BUILD, ignore_errors=True)
    att = "void rtv::(anonymous namespace)::attend16_kernel<false, false, false>(rtv::AttendArgs)"
    copy = "__amd_rocclr_copyBuffer"
    gib = 1 << 30
    fetch, write = os.path.join(BUILD, "fetch"), os.path.join(BUILD, "write")
    # two dispatches of the attention, each reported as two counter instances
    # the runtime's own small copies use the copy kernel too: the calibration
    # is the largest copy dispatch, not their mean
    _write_pmc(fetch, "FETCH_SIZE", [(1, att, 100.0), (1, att, 300.0), (2, att, 500.0), (2, att, 100.0),
                                     (3, copy, gib / 1024 / 2), (4, copy, 2.0)])
    _write_pmc(write, "WRITE_SIZE", [(1, att, 10.0), (2, att, 30.0), (3, copy, gib / 1024), (4, copy, 0.0)])
    out = os.path.join(BUILD, "traffic.json")
    bench.pmc_summary(fetch, write, gib, out)
    with open(out) as f:
        t = json.load(f)
    assert t["calibration"] == {"copy_bytes": gib, "fetch_factor": 2.0, "write_factor": 1.0}
    k = t["kernels"]["attend16_kernel<false, false, false>"]
    assert k["dispatches"] == 2
    assert k["fetch_bytes"] == round(500.0 * 1024 * 2.0)      # mean of 400 and 600 KiB, x 2
    assert k["write_bytes"] == round(20.0 * 1024 * 1.0)
    assert k["bytes"] == k["fetch_bytes"] + k["write_bytes"]
    assert k["source"] == "kv_cache_attention_rtv_amd/csrc/attend.hip"
    # the figures hold only for the source they were measured on
    assert bench.traffic_of(out, "attend16_kernel<false, false, false>") is not None
    t["kernels"]["attend16_kernel<false, false, false>"]["source_sha256_16"] = "0" * 16
    with open(out, "w") as f:
        json.dump(t, f)
    assert bench.traffic_of(out, "attend16_kernel<false, false, false>") is None
    assert bench.traffic_of(os.path.join(BUILD, "missing.json"), "attend16_kernel") is None


def test_pmc_summary_needs_the_copy_kernel():
    shutil.rmtree(BUILD, ignore_errors=True)
    att = "void rtv::(anonymous namespace)::attend16_kernel<false, false, false>(rtv::AttendArgs)"
    fetch, write = os.path.join(BUILD, "fetch"), os.path.join(BUILD, "write")
    _write_pmc(fetch, "FETCH_SIZE", [(1, att, 100.0)])
    _write_pmc(write, "WRITE_SIZE", [(1, att, 10.0)])
    with pytest.raises(SystemExit):
        bench.pmc_summary(fetch, write, 1 << 30, os.path.join(BUILD, "traffic.json"))


def test_algorithmic_work_of_the_step_workload():
    """Per call at the step shape: 111.45 MB for the append (K, V bf16 read,
    codes and f32 scales written) and 3.520 TFLOP for the full-window attention."""
    wl = get_workload("step")
    append_bytes, attend_flops = bench.algorithmic(wl, wl.capacity_frames)
    n, H, D = 11968, 12, 128
    assert append_bytes == 2 * n * H * D * 2 + 2 * n * H * D + 2 * n * H * 4 == 111_446_016
    assert attend_flops == 4.0 * n * (16 * 2992) * D * 12
    assert round(attend_flops / 1e12, 3) == 3.520
