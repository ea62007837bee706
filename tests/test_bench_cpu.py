"""bench.py's host-side helpers (no GPU): the counter-pass report and the
lookup of stored traffic by kernel-source hash."""
import csv
import json
import os

import bench

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for d, name, v in rows:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": v})


def test_traffic_report_scales_by_the_copy(tmp_path):
    copy = "void at::native::vectorized_elementwise_kernel<4, neg ...>"
    large = bench.TRAFFIC_KERNELS["large_exact"][0] + "(mxg::GemmArgs)"
    skinny = bench.TRAFFIC_KERNELS["skinny_exact"][0] + "(mxg::GemmArgs)"
    quant = bench.QUANT_KERNEL + "(mxg::quant::QuantArgs)"
    gib_kib = bench.COPY_BYTES / 1024
    # FETCH_SIZE reads half the bytes, WRITE_SIZE all of them
    _csv(tmp_path / "f.csv", "FETCH_SIZE",
         [(1, copy, gib_kib / 2), (2, large, 1000.0), (3, large, 1002.0), (4, skinny, 50.0),
          (5, quant, 400.0), (6, "other", 7.0)])
    _csv(tmp_path / "w.csv", "WRITE_SIZE",
         [(1, copy, gib_kib), (2, large, 10.0), (3, large, 10.0), (4, skinny, 5.0),
          (5, quant, 100.0)])
    out = tmp_path / "t.json"
    bench.traffic_report(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(out))
    d = json.load(open(out))
    assert abs(d["scale_FETCH_SIZE"] - 2.0) < 1e-12 and abs(d["scale_WRITE_SIZE"] - 1.0) < 1e-12
    k = d["kernels"]
    assert k["large_exact"]["fetch_bytes"] == round(1001.0 * 1024 * 2)
    assert k["large_exact"]["write_bytes"] == 10 * 1024
    assert k["skinny_exact"]["bytes_per_launch"] == round(50 * 1024 * 2 + 5 * 1024)
    assert k["mx_quantize"]["bytes_per_launch"] == round(400 * 1024 * 2 + 100 * 1024)
    assert d["kernel_hash"] == bench.kernel_hash()


def test_traffic_lookup_needs_the_current_hash(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    for f in bench.KERNEL_SOURCES:  # the hash reads the sources under ROOT
        dst = tmp_path / f
        dst.parent.mkdir(parents=True, exist_ok=True)
        dst.write_text(open(os.path.join(os.path.dirname(bench.__file__), f)).read())
    h = bench.kernel_hash()
    json.dump({"kernel_hash": h, "kernels": {"large_exact": {"bytes_per_launch": 123}}},
              open(prof / "hbm_traffic.json", "w"))
    assert bench.traffic_from_profiles("large_exact") == 123
    assert bench.traffic_from_profiles("mx_quantize") is None
    json.dump({"kernel_hash": "stale", "kernels": {"large_exact": {"bytes_per_launch": 123}}},
              open(prof / "hbm_traffic.json", "w"))
    assert bench.traffic_from_profiles("large_exact") is None


def test_kernel_hash_ignores_comments(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    for f in bench.KERNEL_SOURCES:
        dst = tmp_path / f
        dst.parent.mkdir(parents=True, exist_ok=True)
        dst.write_text(open(os.path.join(os.path.dirname(bench.__file__), f)).read())
    h0 = bench.kernel_hash()
    f0 = tmp_path / bench.KERNEL_SOURCES[0]
    f0.write_text(f0.read_text() + "\n// a comment\n/* another */\n")
    assert bench.kernel_hash() == h0
    f0.write_text(f0.read_text() + "\nint extra_symbol;\n")
    assert bench.kernel_hash() != h0


def test_launch_stats():
    t = [1e-3, 2e-3, 3e-3, 4e-3, 5e-3]  # seconds
    st = bench.launch_stats(t, 3e9, 1e9, 10.0)  # 3e9 units, reported in 1e9
    assert st["median_us"] == 3000.0 and st["min_us"] == 1000.0
    assert st["p25_us"] == 2000.0 and st["p75_us"] == 4000.0 and st["iqr_us"] == 2000.0
    assert abs(st["rate_at_median"] - 1000.0) < 1e-9 and abs(st["rate_at_min"] - 3000.0) < 1e-9
    assert abs(st["frac_at_median"] - 100.0) < 1e-9
