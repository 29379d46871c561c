"""Host logic of bench.py (no GPU): the vector-unit roofline arithmetic, the
per-dispatch counter sums and the HBM-traffic writer's choice of dispatches,
on synthetic counter tables in a temporary root."""
import csv
import json
import os

import pytest

import bench


def test_valu_roofline_workload5():
    units = 8 * 16 * 65536
    r = bench.valu_roofline(units, 4, 128, 1, 0.5, "k")
    flop = units * 4 * 128 * 7                       # rotation 3 + score 2 + P.V 2
    assert r["algorithmic_flop_per_launch"] == flop
    assert r["achieved"] == pytest.approx(flop / 0.5e-3 / 1e12)
    assert r["frac"] == pytest.approx(r["achieved"] / 157.3)
    assert r["bound"] == "alu" and r["unit"] == "TFLOP/s"
    # GQA 4: the rotation is shared by the group, scores and P.V are per q-head
    assert bench.valu_roofline(1, 4, 128, 4, 1.0, "k")["algorithmic_flop_per_launch"] == 4 * 128 * (3 + 16)


def test_per_dispatch_sums_counter_instances():
    rows = [{"Dispatch_Id": "7", "Kernel_Name": "k(int)", "Grid_Size": "256", "Counter_Name": "FETCH_SIZE",
             "Counter_Value": "10"},
            {"Dispatch_Id": "7", "Kernel_Name": "k(int)", "Grid_Size": "256", "Counter_Name": "FETCH_SIZE",
             "Counter_Value": "5.5"},
            {"Dispatch_Id": "7", "Kernel_Name": "k(int)", "Grid_Size": "256", "Counter_Name": "WRITE_SIZE",
             "Counter_Value": "99"},
            {"Dispatch_Id": "8", "Kernel_Name": "m(int)", "Grid_Size": "64", "Counter_Name": "FETCH_SIZE",
             "Counter_Value": "1"}]
    d = bench._per_dispatch(rows, "FETCH_SIZE")
    assert d == {"7": ("k", "256", 15.5), "8": ("m", "64", 1.0)}


def _write_csv(d, table, counter):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, grid, val) in enumerate(table):
            w.writerow({"Dispatch_Id": str(100 + i), "Kernel_Name": name + "(args)", "Grid_Size": str(grid),
                        "Counter_Name": counter, "Counter_Value": str(val)})


def test_write_traffic_takes_the_step_loop_calls(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda kern: "h-" + kern)
    os.makedirs(tmp_path / "profiles")
    enc = "void loopvq::encode_kernel<16, 4, false>"
    dec, mrg = "loopvq::decode_half_kernel", "loopvq::merge_kernel"
    # fetch: calibration read of 1 GiB counted as 0.5 GiB; two steps of
    # (encode K, encode V, decode, merge); then recent-window calls that read more
    fetch = [("loopvq_calib::calib_read_kernel", 1, 524288), ("loopvq_calib::calib_copy_kernel", 1, 524288)]
    write = [("loopvq_calib::calib_read_kernel", 1, 0), ("loopvq_calib::calib_copy_kernel", 1, 1048576)]
    for _ in range(2):
        fetch += [(enc, 8, 2000), (enc, 8, 2002), (dec, 4, 150), (mrg, 2, 1)]
        write += [(enc, 8, 130), (enc, 8, 130), (dec, 4, 2), (mrg, 2, 3)]
    for _ in range(3):
        fetch += [(dec, 4, 215), (mrg, 2, 1)]
        write += [(dec, 4, 2), (mrg, 2, 3)]
    _write_csv(str(tmp_path / "f"), fetch, "FETCH_SIZE")
    _write_csv(str(tmp_path / "w"), write, "WRITE_SIZE")
    bench.write_traffic(2, str(tmp_path / "f"), str(tmp_path / "w"), "cmd")
    d = json.load(open(tmp_path / "profiles" / "traffic.json"))
    e = d["kernels"]["decode_half@2"]
    assert e["dispatches_averaged"] == [[2, 2], [2, 2]]
    assert e["fetch_KiB"] == pytest.approx(151.0)          # 150 + 1, not the recent-window 215
    assert e["write_KiB"] == pytest.approx(5.0)
    assert e["bytes_per_launch"] == pytest.approx((151.0 * 2.0 + 5.0 * 1.0) * 1024)
    assert e["source_hash"] == "h-decode_half"
    assert d["kernels"]["encode@2"]["fetch_KiB"] == pytest.approx(2001.0)
    assert d["commands"]["workload 2"] == "cmd"
