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


def test_oracle_tasks_run_over_the_worker_pool():
    """The oracle baseline's worker pool and tasks on tiny staged inputs:
    every row is processed once, and the ESA task's view of the staged key
    rows returns the rows of the requested positions."""
    import numpy as np
    from oracle import esa as oesa
    r = np.random.default_rng(3)
    try:
        n, hq, hkv, d, block = 64, 4, 2, 8, 16
        qp = bench._stage("t_q", r.standard_normal((n, hq, d)).astype(np.float32))
        kp = bench._stage("t_k", r.standard_normal((n, hkv, d)).astype(np.float32))
        vp = bench._stage("t_v", r.standard_normal((n, hkv, d)).astype(np.float32))
        from oracle import moba as omoba
        kbar = omoba.block_means(np.load(kp).astype(np.float64), block)
        items = [(qp, kp, vp, kbar, list(range(i, i + 8)), block, 3, 0.3) for i in range(0, n, 8)]
        res, el = bench._run_parallel(bench._moba_rows_task, items, 60.0)
        assert sum(res) == n and el > 0
        # ESA: attention over a staged subset of rows equals attention over the full cache
        T, m, H = 40, 4, 2
        K, V = r.standard_normal((T, H, d)), r.standard_normal((T, H, d))
        q = r.standard_normal((m, H, d))
        c0, n_init, W, sel = T - m, 2, 6, np.array([5, 9, 20])
        pos = oesa.key_list(sel, c0, n_init, W, T - 1)
        a = (bench._stage("e_q", q), bench._stage("e_k", K[pos]), bench._stage("e_v", V[pos]), pos, sel, c0,
             n_init, W, 0.5, [0, 3])
        assert bench._esa_attend_task(a) == 2
        # the view the task builds maps positions to the staged rows: same result as the full cache
        o_full, _ = oesa.attend(q, K, V, sel, c0, n_init, W, 0.5, rows=[0, 3])
        o_list, _ = oesa.attend(q, bench._ListedRows(K[pos], pos), bench._ListedRows(V[pos], pos), sel, c0,
                                n_init, W, 0.5, rows=[0, 3])
        assert np.array_equal(o_full, o_list)
    finally:
        bench.close_cpu_pool()


def _pmc_csv(path, rows):
    """rows: (dispatch id, kernel name, counter, value)."""
    with open(path, "w") as fh:
        fh.write("Correlation_Id,Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for d, k, c, v in rows:
            fh.write(f'{d},{d},"{k}",{c},{v}\n')


def test_traffic_ingestion_scales_by_the_copy_and_charges_stage_kernels(tmp_path):
    """Two counter runs (FETCH_SIZE, WRITE_SIZE): the calibration copy fixes the
    scales, a stage's several kernels are charged per launch of its first one,
    torch's kernels are ignored, and the entry carries the source hash."""
    gib = 1 << 30
    copy = "__amd_rocclr_copyBuffer"
    past = "void qat::moba_past_persist_kernel<128>(...)"
    cnt, scan = "qat::moba_count_kernel(...)", "qat::moba_scan_kernel(...)"
    f = tmp_path / "f.csv"
    w = tmp_path / "w.csv"
    _pmc_csv(f, [(1, copy, "FETCH_SIZE", gib / 2048), (2, "at::native::fill", "FETCH_SIZE", 999.0),
                 (3, past, "FETCH_SIZE", 100.0), (4, cnt, "FETCH_SIZE", 10.0), (5, scan, "FETCH_SIZE", 2.0),
                 (6, past, "FETCH_SIZE", 300.0), (7, cnt, "FETCH_SIZE", 30.0), (8, scan, "FETCH_SIZE", 6.0)])
    _pmc_csv(w, [(1, copy, "WRITE_SIZE", gib / 1024), (3, past, "WRITE_SIZE", 50.0),
                 (4, cnt, "WRITE_SIZE", 1.0), (6, past, "WRITE_SIZE", 50.0), (7, cnt, "WRITE_SIZE", 1.0)])
    out = tmp_path / "counters.json"
    new = bench.ingest_traffic("wl", str(f), str(w), gib, out=str(out))
    assert set(new) == {"wl/moba_past_attn", "wl/moba_dispatch"}
    p = new["wl/moba_past_attn"]
    assert p["fetch_scale"] == 2048.0 and p["write_scale"] == 1024.0
    assert p["read_bytes_per_launch"] == 200 * 2048 and p["write_bytes_per_launch"] == 50 * 1024   # medians
    assert p["source_sha"] == bench.kernel_source_sha("moba_past_attn")
    dsp = new["wl/moba_dispatch"]
    assert dsp["read_bytes_per_launch"] == 24 * 2048   # median of the launches' sums 12 and 36
    assert json.loads(out.read_text())["wl/moba_past_attn"]["hbm_bytes_per_launch"] == 200 * 2048 + 50 * 1024


def test_stage_medians_skip_a_one_off_setup_launch():
    """A launch is a run of consecutive dispatches of one stage's kernels."""
    k = "void qat::moba_decode_piece_kernel<bf16, 128>(...)"
    c = "void qat::moba_decode_combine_kernel<bf16, 128>(...)"
    d = [(k, {"FETCH_SIZE": 1e9}), (k, {"FETCH_SIZE": 1.0})]   # one setup launch of two dispatches
    for _ in range(4):
        d += [(c, {"FETCH_SIZE": 2.0}), (k, {"FETCH_SIZE": 5.0})]
    m = bench.stage_counter_means(d, "FETCH_SIZE")
    assert m == {"moba_decode_attn": 5.0, "moba_decode_combine": 2.0}


def test_mfma_table_normalises_busy_cycles_per_xcd_and_simd(tmp_path):
    k = "void qat::cca_attn_kernel<128>(...)"
    c = tmp_path / "m.csv"
    _pmc_csv(c, [(1, k, "SQ_INSTS_MFMA", 1000.0), (1, k, "SQ_INSTS_VALU", 2500.0),
                 (1, k, "SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * 100 * 1024), (1, k, "SQ_BUSY_CYCLES", 7.0),
                 (1, k, "GRBM_GUI_ACTIVE", 100 * 8)])
    t = bench.mfma_table(str(c))
    row = [r for r in t.splitlines() if r.startswith("| cca_attn")][0]
    assert "| 2.50 |" in row and row.endswith("| 0.500 |")


def test_every_library_kernel_maps_to_a_stage():
    import re
    names = set()
    for f in os.listdir(bench.CSRC):
        if f.endswith(".hip"):
            names |= set(re.findall(r"void ([a-z_0-9]+_kernel)\(", open(os.path.join(bench.CSRC, f)).read()))
    unmapped = {n for n in names if bench.stage_of_kernel(n) is None}
    assert not unmapped, unmapped
