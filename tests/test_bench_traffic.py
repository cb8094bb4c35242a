"""Host logic of bench.py's traffic records: rocprofv3 FETCH_SIZE and
WRITE_SIZE values (KiB per dispatch, one row per counter instance) are
summed per dispatch, scaled by what the same counter reads for a device copy
of known size, and averaged over the launches of the measured op. Synthetic
counter files; nothing runs on a GPU."""
import csv
import importlib.util
import json
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def write_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for d, k, v in rows:
            # two instances per dispatch, as the per-XCD rows of a real file
            w.writerow({"Dispatch_Id": d, "Kernel_Name": k, "Counter_Name": counter, "Counter_Value": v / 2})
            w.writerow({"Dispatch_Id": d, "Kernel_Name": k, "Counter_Name": counter, "Counter_Value": v / 2})


def test_cache_write_and_decode_records(tmp_path, monkeypatch):
    bench = load_bench()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    copy = "__amd_rocclr_copyBuffer"
    # 64 MiB copy: FETCH reads half its bytes in KiB, WRITE all of them
    fetch = [(1, copy, 32768.0), (2, "cache_write_fp8x16_kernel<0, 0>", 1000.0),
             (3, "cache_write_fp8x16_kernel<0, 0>", 3000.0), (4, "other_kernel", 9e9)]
    write = [(1, copy, 65536.0), (2, "cache_write_fp8x16_kernel<0, 0>", 500.0),
             (3, "cache_write_fp8x16_kernel<0, 0>", 700.0), (4, "other_kernel", 9e9)]
    write_csv(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    write_csv(tmp_path / "w.csv", "WRITE_SIZE", write)
    out = bench.traffic_from_counters("cache_write_fp8", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), 64)
    assert out["FETCH_SIZE"]["launches"] == 2 and out["FETCH_SIZE"]["merge_dispatches"] == 0
    assert out["FETCH_SIZE"]["scale"] == 0.5 and out["WRITE_SIZE"]["scale"] == 1.0
    assert out["FETCH_SIZE"]["bytes_per_launch"] == 2000 * 1024 * 2
    assert out["WRITE_SIZE"]["bytes_per_launch"] == 600 * 1024
    assert out["bytes_per_launch"] == (4000 + 600) * 1024
    assert out["kernel_sha"] == bench.kernel_sha(bench.CACHE_WRITE_SRCS) != bench.kernel_sha()
    rec = json.load(open(tmp_path / "profiles" / "traffic_cache_write_fp8.json"))
    assert rec == out
    assert bench.measured_traffic("cache_write_fp8") == out["bytes_per_launch"]
    # a record taken on other kernel code is not reported
    rec["kernel_sha"] = "0" * 16
    json.dump(rec, open(tmp_path / "profiles" / "traffic_cache_write_fp8.json", "w"))
    assert bench.measured_traffic("cache_write_fp8") is None

    # decode: the decode kernel and its merge dispatches, per decode launch
    fetch = [(1, copy, 32768.0), (2, "decode_kernel<...>", 100.0), (3, "merge_kernel<4>", 10.0),
             (4, "decode_kernel<...>", 300.0), (5, "merge_wide_kernel", 30.0)]
    write = [(1, copy, 65536.0), (2, "decode_kernel<...>", 8.0), (3, "merge_kernel<4>", 2.0),
             (4, "decode_kernel<...>", 8.0), (5, "merge_wide_kernel", 2.0)]
    write_csv(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    write_csv(tmp_path / "w.csv", "WRITE_SIZE", write)
    out = bench.traffic_from_counters("verify_causal", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), 64)
    assert out["FETCH_SIZE"]["launches"] == 2 and out["FETCH_SIZE"]["merge_dispatches"] == 2
    assert out["bytes_per_launch"] == (440 / 2 * 2 + 20 / 2) * 1024
    assert bench.measured_traffic("verify_causal") == out["bytes_per_launch"]
