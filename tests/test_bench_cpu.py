"""Host logic of bench.py, no GPU: the one-GPU refusal, and the HBM-traffic
summary built from rocprofv3 counter files (every counter scaled by what the
same counter reads for a device copy of known size)."""
import csv
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _counter_dir(base, name, counter, rows):
    d = base / name / "vm"
    d.mkdir(parents=True)
    with open(d / "1_counter_collection.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for kernel, value in rows:
            w.writerow({"Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": value})
    return str(base / name)


def test_traffic_summary_scales_by_the_copy(tmp_path):
    b = _bench()
    copy_bytes = (b.COPY_PROBE_MB * 1e6) // 4 * 4
    # the copy reads half its bytes in FETCH_SIZE (KiB) and all of them in WRITE_SIZE
    cf = _counter_dir(tmp_path, "cf", "FETCH_SIZE", [("__amd_rocclr_copyBuffer", copy_bytes / 2 / 1024)] * 3)
    cw = _counter_dir(tmp_path, "cw", "WRITE_SIZE", [("__amd_rocclr_copyBuffer", copy_bytes / 1024)] * 3)
    kernels = {"router_gemv_t1_kernel": (3000.0, 20.0), "gateup_t1_kernel<4, 3, 1, false, false>": (55000.0, 70.0),
               "down_combine_t1_kernel<4, 1, 1, false, 1>": (28000.0, 240.0)}
    # two dispatches each, whose mean the summary takes; a kernel with fewer
    # dispatches of the same name family is not the one picked
    pf = _counter_dir(tmp_path, "pf", "FETCH_SIZE",
                      [(k, v[0] - 10) for k, v in kernels.items()] + [(k, v[0] + 10) for k, v in kernels.items()]
                      + [("gateup_t1_kernel<4, 3, 1, true, true>", 1.0)])
    pw = _counter_dir(tmp_path, "pw", "WRITE_SIZE",
                      [(k, v[1]) for k, v in kernels.items()] + [(k, v[1]) for k, v in kernels.items()])
    out = tmp_path / "traffic.md"
    b.pmc_summary(pf, pw, cf, cw, str(out))
    line = [ln for ln in open(out) if ln.startswith("traffic_json: ")][0]
    info = json.loads(line[len("traffic_json: "):])
    assert info["source_hash"] == b.kernel_source_hash()
    assert info["fetch_scale"] == pytest.approx(2.0) and info["write_scale"] == pytest.approx(1.0)
    for short, key in (("router", "router_gemv_t1_kernel"), ("gateup", "gateup_t1_kernel<4, 3, 1, false, false>"),
                       ("down", "down_combine_t1_kernel<4, 1, 1, false, 1>")):
        t = info["kernels"][short]
        assert t["dispatches"] == 2
        assert t["fetch_bytes"] == pytest.approx(kernels[key][0] * 1024 * 2.0, rel=1e-9)
        assert t["write_bytes"] == pytest.approx(kernels[key][1] * 1024, rel=1e-9)
