"""Host logic of the profile summaries (bit_weight_quantized_qw_amd.profsum)
on synthetic rocprofv3 CSV files: kernel-trace statistics, counter
compaction, per-call traffic from split launches and the copy calibration."""

import csv
import json
import os

import pytest

from bit_weight_quantized_qw_amd import profsum


def _write_csv(path, fields, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def _pmc(dirname, rows):
    """rows: (kernel name, grid, counter, value), one per dispatch."""
    _write_csv(os.path.join(dirname, "host", "run_counter_collection.csv"),
               ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"],
               [{"Kernel_Name": k + "(Args)", "Grid_Size": g, "Counter_Name": c, "Counter_Value": v}
                for k, g, c, v in rows])


def test_kernel_trace_table(tmp_path):
    rows = []
    for i, (k, g, us) in enumerate([("qw::a", 512, 10.0), ("qw::a", 512, 14.0), ("qw::b", 256, 3.0),
                                    ("other", 256, 1.0)]):
        rows.append({"Kernel_Name": k + "(int)", "Grid_Size_X": g, "Workgroup_Size_X": 256,
                     "LDS_Block_Size": 0, "VGPR_Count": 64, "Accum_VGPR_Count": 0, "Scratch_Size": 0,
                     "Start_Timestamp": 1000 * i, "End_Timestamp": 1000 * i + int(us * 1000)})
    _write_csv(str(tmp_path / "kt" / "run_kernel_trace.csv"), list(rows[0]), rows)
    st = profsum.kernel_stats(str(tmp_path / "kt"), ["qw::"])
    assert [(s[0], s[1], s[7], s[8]) for s in st] == [("qw::a", 512, 2, 12.0), ("qw::b", 256, 1, 3.0)]


def test_compact_and_counters(tmp_path):
    _pmc(str(tmp_path / "p"), [("k1", 512, "FETCH_SIZE", 10.0), ("k1", 512, "FETCH_SIZE", 14.0),
                               ("k1", 256, "FETCH_SIZE", 1.0), ("k2", 512, "FETCH_SIZE", 5.0)])
    c = profsum.compact(str(tmp_path / "p"))
    assert {(r["kernel"], r["grid"], r["n"], r["sum"]) for r in c["rows"]} == {
        ("k1", 512, 2, 24.0), ("k1", 256, 1, 1.0), ("k2", 512, 1, 5.0)}
    path = str(tmp_path / "c.json")
    json.dump(c, open(path, "w"))
    assert profsum.counters([path], "k1", 512) == {"FETCH_SIZE": (12.0, 2)}
    assert profsum.counters([str(tmp_path / "p")], "k1") == {"FETCH_SIZE": (25.0 / 3, 3)}


def test_traffic_per_call_and_calibration(tmp_path, monkeypatch):
    d = tmp_path / "t"
    d.mkdir()
    kib = (1 << 30) / 1024
    for ctr, raw in (("FETCH_SIZE", kib / 2), ("WRITE_SIZE", kib)):  # fetch counts half the bytes
        _pmc(str(tmp_path / f"cal_{ctr}"), [("AUnaryFunctor<float>", 1 << 20, ctr, raw)] * 3)
        json.dump(profsum.compact(str(tmp_path / f"cal_{ctr}")), open(d / f"copy_calib_{ctr}.json", "w"))
    # two calls, each two part launches (100 and 60 KiB fetched) and a
    # reduction (4 KiB); writes 8 KiB per call in the reduction
    rows_f = [("qw::gemv2m::kernel<8>", 4096, "FETCH_SIZE", 100.0), ("qw::gemv2m::kernel<8>", 4096, "FETCH_SIZE", 60.0),
              ("qw::gemv2m::split_reduce_kernel", 256, "FETCH_SIZE", 4.0)] * 2
    rows_w = [(k, g, "WRITE_SIZE", 8.0 if "reduce" in k else 0.0) for k, g, _, _ in rows_f]
    _pmc(str(tmp_path / "wf"), rows_f)
    _pmc(str(tmp_path / "ww"), rows_w)
    json.dump(profsum.compact(str(tmp_path / "wf")), open(d / "down70b_b8_FETCH_SIZE.json", "w"))
    json.dump(profsum.compact(str(tmp_path / "ww")), open(d / "down70b_b8_WRITE_SIZE.json", "w"))
    json.dump({"kernels": {"qgemv_2bit": {"amount": 330000}}}, open(d / "down70b_b8.json", "w"))
    monkeypatch.setattr(profsum, "TRAFFIC", {"down70b_b8": profsum.TRAFFIC["down70b_b8"]})
    out = str(tmp_path / "traffic.json")
    t = profsum.traffic(str(d), out)
    assert t["fetch_scale"] == pytest.approx(2.0) and t["write_scale"] == pytest.approx(1.0)
    e = t["down70b_b8"]["qgemv_2bit"]
    assert e["calls"] == 2
    assert e["fetch_bytes"] == 164 * 1024 * 2 and e["write_bytes"] == 8 * 1024
    assert e["bytes"] == 164 * 2048 + 8192
    assert e["ratio"] == pytest.approx((164 * 2048 + 8192) / 330000, abs=1e-4)
    assert len(e["sha256"]) == 64 and json.load(open(out))["down70b_b8"]["qgemv_2bit"] == e
    # a dispatch count that is not a whole number of calls is refused
    _pmc(str(tmp_path / "bad"), rows_f[:-1])
    json.dump(profsum.compact(str(tmp_path / "bad")), open(d / "down70b_b8_FETCH_SIZE.json", "w"))
    with pytest.raises(ValueError):
        profsum.traffic(str(d), out)
