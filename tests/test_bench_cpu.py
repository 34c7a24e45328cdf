"""bench.py's host-side logic on the CPU: how the timed launches are split
into batches and summarised, the source-hash gate of the traffic record, and
the CPU baseline (the oracle on token slices in a thread pool gives the
whole-input result)."""
import json
import os
from dataclasses import replace

import bench
import rope_inputs


def test_batches_cover_every_launch():
    assert bench._batches(200) == [20] * 10
    for k in (1, 5, 7, 23, 99, 1000):
        b = bench._batches(k)
        assert sum(b) == k and len(b) == min(10, k) and max(b) - min(b) <= 1


def test_summary_median_spread_and_mean():
    s = bench._summary([2.0, 1.0, 3.0], [10, 10, 5])
    assert s["median"] == 2.0 and s["min"] == 1.0 and s["max"] == 3.0 and s["batches"] == 3
    assert abs(s["mean"] - (20.0 + 10.0 + 15.0) / 25.0) < 1e-12


def test_traffic_record_used_only_for_the_current_sources(tmp_path, monkeypatch):
    rec = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    assert bench.traffic_for_headline() is None                     # no record
    rec.write_text(json.dumps({"source_sha256": bench.kernel_source_sha(), "traffic_bytes_per_launch": 123}))
    assert bench.traffic_for_headline() == 123
    rec.write_text(json.dumps({"source_sha256": "0" * 64, "traffic_bytes_per_launch": 123}))
    assert bench.traffic_for_headline() is None                     # taken on other sources


def test_committed_traffic_record_names_its_sources():
    with open(os.path.join(bench.ROOT, "profiles", "traffic_c2_rope_f16_prefill.json")) as f:
        rec = json.load(f)
    assert len(rec["source_sha256"]) == 64
    assert rec["algorithmic_bytes_per_launch"] == rope_inputs.get(bench.HEADLINE).algorithmic_bytes()


def test_cpu_baseline_pooled_equals_whole():
    w = replace(rope_inputs.get("c2_rope_f16_prefill"), x_shape=(2, 300, 4 * 128), num_heads=4,
                name="c2_small")
    r = bench.cpu_baseline(w, min_reps=1, single_s=0.0, pool_s=0.0)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s" and r["cores"] >= 1
    assert r["value"] > 0 and r["single_thread"]["value"] > 0 and r["single_thread"]["cores"] == 1
    assert r["host"]["nproc"] >= 1
