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
    sys.modules["bench_under_test"] = mod  # its worker functions pickle by module name
    spec.loader.exec_module(mod)
    return mod


def _res(nbytes, ms):
    return {"event_ms_mean": ms, "logical_kv_bytes": nbytes, "unique_kv_bytes": nbytes // 4}


def test_hbm_roofline_without_counter_record_reports_no_fraction(bench):
    r = bench.roofline_hbm(_res(1_358_954_496, 0.17), "decode", "no_such_workload", False)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    # logical bytes may exceed what HBM delivers (shared documents): no fraction from them
    assert r["frac"] is None and r["achieved"] is None and r["traffic"] is None
    assert r["per_launch"]["logical_gbs"] == pytest.approx(1_358_954_496 / 0.17e-3 / 1e9,
                                                           rel=1e-4)
    assert r["kernel"] == "decode_bf16_kernel"
    split = bench.roofline_hbm(_res(10 ** 9, 1.0), "decode", "no_such_workload", True)
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
    r = bench.roofline_hbm(_res(1_358_954_496, 0.17), "decode", "w", False)
    assert r["traffic"] == 959_507_142
    # the fraction is taken on HBM bytes, never on the logical ones
    assert r["achieved"] == pytest.approx(959_507_142 / 0.17e-3 / 1e9, rel=1e-4)
    assert r["frac"] == pytest.approx(r["achieved"] / 8000.0, rel=1e-3)
    assert r["frac"] <= 1.0
    rec["decode:w"]["source_sha256_16"] = "0" * 16
    p.write_text(json.dumps(rec))
    assert bench.traffic_for("decode", "w") is None


def test_shared_decode_traffic_follows_the_plan(bench, tmp_path, monkeypatch):
    # a shared-decode record also names the plan blob it was taken with
    rec = {"decode_shared:w": {"source_sha256_16": bench.src_hash("decode_shared"),
                               "plan_sha256_16": "ab" * 8, "hbm_bytes_per_launch": 400_000_000}}
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    res = dict(_res(1_358_954_496, 0.08), decode_kernel="shared", plan={"sha256_16": "ab" * 8})
    r = bench.roofline_hbm(res, "decode", "w", False)
    assert r["traffic"] == 400_000_000 and r["kernel"].startswith("decode_shared_kernel")
    res["plan"] = {"sha256_16": "cd" * 8}  # another chunking: the counters no longer apply
    assert bench.roofline_hbm(res, "decode", "w", False)["traffic"] is None


def test_parity_summary(bench):
    import numpy as np
    ref = [np.ones((4, 8)), np.full((4, 8), 2.0)]
    ok = bench._parity([x + 1e-3 for x in ref], ref, "x")
    assert ok["pass"] and ok["max_abs"] == pytest.approx(1e-3)
    bad = bench._parity([x + 5e-2 for x in ref], ref, "x")
    assert not bad["pass"]
    nan = bench._parity([ref[0] * np.nan, ref[1]], ref, "x")
    assert not nan["pass"]


def test_oracle_pool_runs_the_oracle_over_processes(bench):
    """The CPU baseline's worker pool gives the oracle's own numbers."""
    from oracle import run_decode
    from workloads import build_workload
    w = build_workload(name="t", kind="decode", dtype="bf16", num_q_heads=4, num_kv_heads=2,
                       head_dim=16, block_size=4, rope_base=1e4, doc_lens=[7, 9],
                       requests=[[("doc", 0), ("doc", 1)], [("doc", 1)]], seed=3)
    bench._ORACLE_W["t"] = w
    pool = bench.OraclePool()
    try:
        got, dt = pool.decode("t", range(w.batch))
    finally:
        pool.close()
    want = run_decode(w)
    for r in range(w.batch):
        assert (got[r][0] == want[r][0]).all() and (got[r][1] == want[r][1]).all()
    assert dt > 0 and pool.cores == len(os.sched_getaffinity(0))


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
