"""Host-side checks of bench.py (no GPU): the one-GPU guard, the stage ->
source map behind the counter hashes, and the counter lookup."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_stage_sources_exist_and_hash_differently_per_file_set():
    for stage, files in bench.STAGE_SOURCES.items():
        for f in files:
            assert os.path.exists(os.path.join(bench.CSRC, f)), (stage, f)
    assert bench.kernel_source_sha("moba_past_attn") == bench.kernel_source_sha("moba_current_attn")
    assert bench.kernel_source_sha("moba_past_attn") != bench.kernel_source_sha("esa_prefill_attn")
    assert len(bench.kernel_source_sha("cca_attn")) == 16


def test_counter_lookup_requires_matching_sources(tmp_path, monkeypatch):
    sha = bench.kernel_source_sha("cca_attn")
    path = tmp_path / "counters.json"
    path.write_text(json.dumps({"w/cca_attn": {"hbm_bytes_per_launch": 123, "source_sha": sha},
                                "w/cca_pool": {"hbm_bytes_per_launch": 5, "source_sha": "0" * 16}}))
    monkeypatch.setattr(bench, "COUNTERS", str(path))
    assert bench.traffic_for("cca_attn", "w") == 123
    assert bench.traffic_for("cca_pool", "w") is None   # taken on other sources
    assert bench.traffic_for("cca_attn", "other") is None


def test_committed_counters_name_known_stages():
    with open(bench.COUNTERS) as fh:
        c = json.load(fh)
    for key, e in c.items():
        workload, stage = key.split("/", 1)
        assert e["hbm_bytes_per_launch"] > 0 or stage in ("moba_bwd_runs",), key
        assert len(e["source_sha"]) == 16
