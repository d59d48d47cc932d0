"""bench.py's host-side records (CPU only): roofline.traffic is reported only
while the kernel sources match the counter run it was measured on, and the
oracle baseline names the host it ran on."""
import json

import bench


def test_traffic_follows_kernel_source_hash(tmp_path, monkeypatch):
    rec = {"kernel_source_sha256": bench.kernel_source_hash(), "bytes_per_launch": 123456}
    path = tmp_path / "t.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench._recorded_traffic() == 123456
    rec["kernel_source_sha256"] = "0" * 64
    path.write_text(json.dumps(rec))
    assert bench._recorded_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench._recorded_traffic() is None


def test_committed_traffic_record_is_well_formed():
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    derived = (rec["fetch_size_kib_per_dispatch"] * rec["fetch_scale"]
               + rec["write_size_kib_per_dispatch"] * rec["write_scale"]) * 1024
    assert abs(rec["bytes_per_launch"] - derived) <= 1e-6 * derived   # counters stored to 0.1 KiB
    assert rec["bytes_per_launch"] >= rec["algorithmic_bytes_per_launch"]


def test_cpu_baseline_record_names_its_host():
    # the oracle leg of bench.py on the small fp32 workload: one head is
    # enough; the record names what it ran on
    from exact_attention_forward_06_amd.inputs import WORKLOADS, workload_inputs
    w = WORKLOADS["small_fp32"]
    rec = bench._cpu_baseline(w, workload_inputs(w), budget_s=0.0)
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOP/s" and rec["value"] > 0
    assert rec["cores"] >= 1 and "1 of 2 heads" in rec["sample"]
    assert isinstance(rec["cpu_model"], str) and isinstance(rec["blas"], str)
