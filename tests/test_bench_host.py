"""Host-side logic of bench.py (CPU): the traffic record written from counter files, the
algorithmic work of a step, and the guard that keeps a stale counter record out of the
bench line."""

import csv
import importlib.util
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


FIELDS = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write_counters(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Correlation_Id": i, "Dispatch_Id": i, "Kernel_Name": name,
                        "Counter_Name": counter, "Counter_Value": value})


def test_traffic_record_scales_by_the_calibration_copy(bench, tmp_path, monkeypatch):
    main = "mla::(anonymous namespace)::mla_main_bf16_kernel<false, false>(...)"
    copy = "__amd_rocclr_copyBuffer"
    # the first main-kernel dispatch (cold) is left out of the mean
    _write_counters(tmp_path / "fetch.csv", "FETCH_SIZE",
                    [(copy, 3.0), (main, 999.0), (main, 100.0), (main, 102.0),
                     ("mla_combine_kernel", 7.0), (copy, 262144.0)])
    _write_counters(tmp_path / "write.csv", "WRITE_SIZE",
                    [(copy, 0.5), (main, 50.0), (main, 10.0), (main, 10.0), (copy, 524288.0)])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    bench.record_traffic(str(tmp_path / "fetch.csv"), str(tmp_path / "write.csv"), "gate_b64_l8192")
    rec = json.loads(out.read_text())
    # the copy moves 512 MiB each way: FETCH_SIZE read half of it here (scale 2), WRITE_SIZE all
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["fetch_kib_per_dispatch"] == 101.0 and rec["dispatches"] == 2
    assert rec["read_bytes_per_launch"] == 101 * 2 * 1024
    assert rec["write_bytes_per_launch"] == 10 * 1024
    assert rec["bytes_per_launch"] == rec["read_bytes_per_launch"] + rec["write_bytes_per_launch"]
    assert rec["kernel_hash"] == bench.kernel_hash()
    # a record of this kernel and workload is reported; another workload's is not
    assert bench.measured_traffic("gate_b64_l8192") == rec["bytes_per_launch"]
    assert bench.measured_traffic("paged_b16_l4096") is None


def test_stale_traffic_record_is_not_reported(bench, tmp_path, monkeypatch):
    out = tmp_path / "traffic.json"
    out.write_text(json.dumps({"kernel_hash": "0" * 16, "workload": "gate_b64_l8192",
                               "bytes_per_launch": 1}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    assert bench.measured_traffic("gate_b64_l8192") is None


def test_committed_traffic_record_matches_the_kernel_source(bench):
    """The committed record was taken on the kernel as it is now (else bench.py reports
    traffic null and the record must be retaken)."""
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    assert rec["kernel_hash"] == bench.kernel_hash()


def test_algorithmic_work_of_the_gate(bench):
    """bytes and flops of the 64 x 8K workload from the definition: each KV row once,
    Q, O and LSE, the block numbers and lengths; 2 H (576 + 512) flops per visible key."""
    from mla_decode_attention_flashmla_amd import inputs as I

    w = I.WORKLOADS["gate_b64_l8192"]
    d = {"workload": w, "seqlens": __import__("numpy").full(64, 8192, dtype="int32"),
         "causal": False}
    byt, kv, flops = bench.algorithmic_work(d)
    assert kv == 64 * 8192 * 576 * 2
    assert byt == kv + 64 * 128 * (576 * 2 + 512 * 4 + 4) + 64 * 128 * 4 + 64 * 4
    assert flops == 2 * 128 * (576 + 512) * 64 * 8192
    assert abs(byt - 630.26e6) < 0.01e6 and abs(flops - 146.03e9) < 0.01e9
