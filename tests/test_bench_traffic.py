"""bench.py's HBM-traffic bookkeeping on the host: per-dispatch counter means from
rocprofv3's csv output, the copy-calibrated scale factors, the bytes per launch of
each call, and the rule that a figure taken from other kernel sources reads as
null (no GPU: the csv files are written by the test)."""

import csv
import json
import os
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FIELDS = ["Kernel_Name", "Counter_Name", "Counter_Value"]


def _write(folder, counter, rows):
    os.makedirs(os.path.join(folder, "pass_1"), exist_ok=True)
    with open(os.path.join(folder, "pass_1", "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_counter_means_per_kernel(tmp_path):
    d = str(tmp_path / "FETCH_SIZE_fwd")
    _write(d, "FETCH_SIZE", [("fa_fwd_kernel<128, true, false>", 10.0), ("fa_fwd_kernel<128, true, false>", 20.0),
                             ("other", 5.0)])
    means = bench.counter_means(d, "FETCH_SIZE")
    assert means == {"fa_fwd_kernel<128, true, false>": 15.0, "other": 5.0}
    assert bench.counter_means(d, "WRITE_SIZE") == {}


def test_make_traffic_scales_by_the_copy_and_sums_kernels(tmp_path):
    gib_kib = float(1 << 20)
    base = str(tmp_path)
    # the 1 GiB copy reads half and writes all of what it moves, as the counters report it
    _write(os.path.join(base, "FETCH_SIZE_copy"), "FETCH_SIZE", [("__amd_rocclr_copyBuffer", gib_kib / 2)])
    _write(os.path.join(base, "WRITE_SIZE_copy"), "WRITE_SIZE", [("__amd_rocclr_copyBuffer", gib_kib)])
    _write(os.path.join(base, "FETCH_SIZE_fwd"), "FETCH_SIZE", [("void fa::fa_fwd_kernel<128, true, false>", 1000.0)])
    _write(os.path.join(base, "WRITE_SIZE_fwd"), "WRITE_SIZE", [("void fa::fa_fwd_kernel<128, true, false>", 300.0)])
    _write(os.path.join(base, "FETCH_SIZE_decode"), "FETCH_SIZE",
           [("fa_decode_split_kernel<128, 1, false>", 4000.0), ("fa_decode_combine_kernel<128>", 100.0)])
    _write(os.path.join(base, "WRITE_SIZE_decode"), "WRITE_SIZE",
           [("fa_decode_split_kernel<128, 1, false>", 50.0), ("fa_decode_combine_kernel<128>", 10.0)])
    out_path = str(tmp_path / "traffic.json")
    args = types.SimpleNamespace(make_traffic=base, traffic=out_path)
    assert bench.make_traffic(args) == 0
    t = json.load(open(out_path))
    assert t["fetch_scale"] == 2.0 and t["write_scale"] == 1.0
    assert t["fwd"]["bytes_per_launch"] == round((1000.0 * 2 + 300.0) * 1024)
    # a call of two kernels counts both
    assert t["decode"]["bytes_per_launch"] == round(((4000.0 + 100.0) * 2 + 60.0) * 1024)
    assert "gqa" not in t  # no counter runs for it
    # the figures hold for the sources they were taken from ...
    assert bench.traffic_bytes(t, "fwd") == t["fwd"]["bytes_per_launch"]
    # ... and read as null once those sources differ
    t["fwd"]["sources_sha256"] = "0" * 16
    assert bench.traffic_bytes(t, "fwd") is None
    assert bench.traffic_bytes(t, "gqa") is None


def test_make_traffic_needs_every_kernel_of_a_call(tmp_path):
    base = str(tmp_path)
    _write(os.path.join(base, "FETCH_SIZE_copy"), "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 1.0)])
    _write(os.path.join(base, "WRITE_SIZE_copy"), "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 1.0)])
    _write(os.path.join(base, "FETCH_SIZE_decode"), "FETCH_SIZE", [("fa_decode_split_kernel<128, 1, false>", 1.0)])
    _write(os.path.join(base, "WRITE_SIZE_decode"), "WRITE_SIZE", [("fa_decode_split_kernel<128, 1, false>", 1.0)])
    args = types.SimpleNamespace(make_traffic=base, traffic=str(tmp_path / "t.json"))
    with pytest.raises(SystemExit, match="fa_decode_combine_kernel"):
        bench.make_traffic(args)

