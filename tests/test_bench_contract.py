"""bench.py's contract pieces that need no GPU: roofline objects and the one-GPU refusal."""
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_hbm_roofline_fields(bench):
    r = bench.roofline_hbm(1_358_954_496, 0.17, "decode", "no_such_workload", False)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["achieved"] == pytest.approx(1_358_954_496 / 0.17e-3 / 1e9, rel=1e-4)
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], rel=1e-3)
    assert r["traffic"] is None  # no counter record for this workload
    assert "dram_gbs" not in r["per_launch"]
    assert r["kernel"] == "decode_bf16_kernel"
    split = bench.roofline_hbm(1e9, 1.0, "decode", "no_such_workload", True)
    assert split["kernel"] == "decode_bf16_kernel + decode_combine_kernel"


def test_mfma_roofline_fields(bench):
    r = bench.roofline_mfma(704_408_190_976, 0.88, "prefill", "no_such_workload")
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert r["achieved"] == pytest.approx(704_408_190_976 / 0.88e-3 / 1e12, rel=1e-4)
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], rel=1e-3)


def test_traffic_follows_the_kernel_source(bench, tmp_path, monkeypatch):
    # a record is used only while the kernel source hash matches the one it was taken on
    rec = {"decode:w": {"source_sha256_16": bench.src_hash("decode"),
                        "hbm_bytes_per_launch": 959_507_142}}
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    assert bench.traffic_for("decode", "w") == 959_507_142
    r = bench.roofline_hbm(1_358_954_496, 0.17, "decode", "w", False)
    assert r["traffic"] == 959_507_142
    assert r["per_launch"]["dram_gbs"] == pytest.approx(959_507_142 / 0.17e-3 / 1e9, rel=1e-3)
    rec["decode:w"]["source_sha256_16"] = "0" * 16
    p.write_text(json.dumps(rec))
    assert bench.traffic_for("decode", "w") is None


def test_committed_traffic_records_name_their_profiles():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        recs = json.load(f)
    assert recs
    for key, rec in recs.items():
        assert os.path.exists(os.path.join(ROOT, rec["profile"])), key
        assert rec["hbm_bytes_per_launch"] > 0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr or "1 GPU" in r.stderr or "--gpus 1" in r.stderr
    assert r.stdout.strip() == ""
