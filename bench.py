"""Benchmark of the query-aware sparse attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
block gating (mean pool, block scores, top-k with the forced block) and
block-sparse attention for MoBA; key compression of the new tokens, query
compression, scoring, correction, neighbour pooling, top-k and fused
attention for ESA. Inputs are generated on the GPU (seeded) and resident in
HBM before timing starts; outputs and workspaces are preallocated.

Prints one JSON line. Default workload: MoBA prefill at the 8B-style GQA
shape (32 query / 8 KV heads x 128, N = 32768, block 512, top-k 3 with the
forced block, 8 planted key blocks), reported as query tokens per second.
Other workloads (--workload): moba_fp32_4k, esa_prefill_64k,
esa_decode_128k, moba_long_512k, moba_decode_128k, moba_bwd_32k and esa_bwd_64k (gradients), cca_64k
(CCA-style core-token attention), and
esa_prefill_64k_votes /
esa_decode_128k_votes (the softmax-vote reading of ESA's score correction),
esa_prefill_64k_heads / esa_decode_128k_heads (one selection per head).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-attn prefill query-tokens/s + decode us/step; % MFMA peak / % HBM BW"
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")
CSRC = os.path.join(ROOT, "query_aware_top_amd", "csrc")


# Sources each timed stage is built from (the C ABI and launcher declarations
# included): a stored counter reading stays valid while these are unchanged.
_COMMON = ["abi.hip", "launch.h", "common.h"]
STAGE_SOURCES = {
    "moba_meanpool": ["moba_select.hip"],
    "moba_select": ["moba_select.hip"],
    "moba_dispatch": ["moba_attn.hip"],
    "moba_past_attn": ["moba_attn.hip", "attn_core.h"],
    "moba_current_attn": ["moba_attn.hip", "attn_core.h"],
    "moba_generic_attn": ["attn_generic.hip"],
    "moba_decode_select": ["moba_select.hip"],
    "moba_decode_attn": ["attn_generic.hip"],
    "moba_decode_combine": ["attn_generic.hip"],
    "moba_bwd_dq": ["moba_bwd.hip", "attn_core.h", "attn_bwd.h"],
    "moba_bwd_dq_past": ["moba_bwd.hip", "attn_core.h", "attn_bwd.h"],
    "moba_bwd_own": ["moba_bwd.hip", "attn_core.h", "attn_bwd.h"],
    "moba_bwd_gated": ["moba_bwd.hip", "attn_core.h", "attn_bwd.h"],
    "esa_bwd_dq": ["esa_bwd.hip", "attn_core.h", "attn_bwd.h"],
    "esa_bwd_kv": ["esa_bwd.hip", "attn_core.h", "attn_bwd.h"],
    "cca_pool": ["cca.hip"],
    "cca_attn": ["cca.hip", "attn_core.h"],
    "esa_compress*": ["compress.hip"],
    "esa_scores": ["esa_select.hip"],
    "esa_colsum": ["esa_select.hip"],
    "esa_topk": ["esa_select.hip"],
    "esa_decode_scan": ["esa_select.hip"],
    "esa_prefill_attn": ["esa_attn.hip", "attn_core.h"],
    "esa_decode_attn": ["esa_attn.hip"],
    # helper kernels that have counter rows of their own
    "fill_i32": ["moba_attn.hip"],
    "esa_rowmax": ["esa_select.hip"],
    "esa_keylist": ["esa_attn.hip"],
    "esa_decode_combine": ["esa_attn.hip"],
    "moba_bwd_runs": ["moba_bwd.hip"],
    "moba_bwd_kv_reduce": ["moba_bwd.hip"],
}


# The kernel a stage's roofline times (its main kernel, or all kernels of a
# stage timed as a whole), by a substring of the (demangled) kernel name, for
# attributing rocprofv3 per-dispatch counters. Helper kernels of a timed
# stage get labels of their own so they are not charged to it; the two
# compression stages share their kernels and count together as "esa_compress*".
KERNEL_STAGE = (
    ("moba_past_persist_kernel", "moba_past_attn"), ("moba_past_kernel", "moba_past_attn"),
    ("moba_current_kernel", "moba_current_attn"),
    ("meanpool_", "moba_meanpool"),
    ("moba_select_resident", "moba_select"), ("moba_select_mfma_kernel", "moba_select"),
    ("moba_score_select_kernel", "moba_select"),
    ("moba_count_kernel", "moba_dispatch"), ("moba_scan_kernel", "moba_dispatch"),
    ("moba_tiles_kernel", "moba_dispatch"), ("moba_scatter_kernel", "moba_dispatch"),
    ("moba_stable_", "moba_dispatch"), ("moba_wg_scan_kernel", "moba_dispatch"),
    ("fill_i32_kernel", "fill_i32"),
    ("moba_generic_kernel", "moba_generic_attn"),
    ("moba_select_group_kernel", "moba_decode_select"),
    ("moba_decode_piece_kernel", "moba_decode_attn"), ("moba_decode_combine_kernel", "moba_decode_combine"),
    ("moba_bwd_dq_past_kernel", "moba_bwd_dq_past"), ("moba_bwd_dq_cur_kernel", "moba_bwd_dq"),
    ("moba_bwd_dq_kernel", "moba_bwd_dq"), ("moba_bwd_kv_own_kernel", "moba_bwd_own"),
    ("moba_bwd_own_kernel", "moba_bwd_own"), ("moba_bwd_kv_gated_kernel", "moba_bwd_gated"),
    ("moba_bwd_gated_kernel", "moba_bwd_gated"), ("moba_bwd_runs_kernel", "moba_bwd_runs"),
    ("moba_bwd_kv_reduce_kernel", "moba_bwd_kv_reduce"),
    ("esa_bwd_dq_kernel", "esa_bwd_dq"), ("esa_bwd_kv_kernel", "esa_bwd_kv"),
    ("cca_pool_kernel", "cca_pool"), ("cca_attn_kernel", "cca_attn"),
    ("compress_", "esa_compress*"),
    ("esa_rowmax", "esa_rowmax"), ("esa_colsum_kernel", "esa_colsum"),
    ("esa_topk_", "esa_topk"), ("esa_decode_scan_kernel", "esa_decode_scan"),
    ("esa_keylist_kernel", "esa_keylist"), ("esa_prefill_kernel", "esa_prefill_attn"),
    ("esa_decode_attn_kernel", "esa_decode_attn"), ("esa_decode_combine_kernel", "esa_decode_combine"),
    ("esa_generic_kernel", "esa_generic_attn"),
)


def stage_of_kernel(name: str):
    """The timed stage a dispatched kernel belongs to, or None (torch's own
    kernels, the calibration copy, small helpers)."""
    for key, stage in KERNEL_STAGE:
        if key in name:
            return stage
    return None


def read_pmc_csv(path):
    """Per-dispatch counters of a rocprofv3 --pmc run (its *counter_collection.csv):
    a list of (kernel name, {counter: value}) in dispatch order."""
    import csv
    rows = {}
    with open(path, newline="") as fh:
        for r in csv.DictReader(fh):
            d = int(r["Dispatch_Id"])
            name, cnt = rows.setdefault(d, (r["Kernel_Name"], {}))
            cnt[r["Counter_Name"]] = cnt.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [rows[d] for d in sorted(rows)]


def stage_counter_means(dispatches, counter):
    """Per stage: the median over its launches of `counter` summed over the
    launch's dispatches, a launch being a run of consecutive dispatches of
    the stage's kernels (a stage that runs several kernels back to back is
    charged all of them; the median skips one-off launches such as a
    workload's setup)."""
    launches, prev = {}, None
    for name, cnt in dispatches:
        st = stage_of_kernel(name)
        if st is not None and counter in cnt:
            if st != prev:
                launches.setdefault(st, []).append(0.0)
            launches[st][-1] += cnt[counter]
        prev = st
    out = {}
    for st, v in launches.items():
        v = sorted(v)
        n = len(v)
        out[st] = v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])
    return out


def copy_scale(dispatches, counter, copy_bytes):
    """Bytes per counter unit from the calibration copy (the dispatch of a
    kernel with "copy" in its name and the largest reading): the copy reads
    and writes copy_bytes."""
    best = None
    for name, cnt in dispatches:
        if "copy" in name.lower() and counter in cnt and (best is None or cnt[counter] > best):
            best = cnt[counter]
    if not best:
        raise SystemExit(f"no calibration copy with {counter} in the counter file")
    return copy_bytes / best


def ingest_traffic(workload, fetch_csv, write_csv, copy_bytes, out=None):
    """HBM bytes per launch of every stage seen in two counter runs of one
    workload (FETCH_SIZE, then WRITE_SIZE), each scaled by what the same
    counter reads for the calibration copy; stored in profiles/counters.json
    with the hash of the stage's sources. Returns the new entries."""
    out = out or COUNTERS
    f = read_pmc_csv(fetch_csv)
    w = read_pmc_csv(write_csv)
    fs, ws = copy_scale(f, "FETCH_SIZE", copy_bytes), copy_scale(w, "WRITE_SIZE", copy_bytes)
    fm, wm = stage_counter_means(f, "FETCH_SIZE"), stage_counter_means(w, "WRITE_SIZE")
    try:
        with open(out) as fh:
            c = json.load(fh)
    except OSError:
        c = {}
    new = {}
    for st in sorted(set(fm) & set(wm)):
        new[f"{workload}/{st}"] = {"fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
                                   "read_bytes_per_launch": int(fm[st] * fs),
                                   "write_bytes_per_launch": int(wm[st] * ws),
                                   "hbm_bytes_per_launch": int(fm[st] * fs + wm[st] * ws),
                                   "source_sha": kernel_source_sha(st)}
    c.update(new)
    with open(out, "w") as fh:
        json.dump(c, fh, indent=1, sort_keys=True)
        fh.write("\n")
    return new


def mfma_table(csv_path, n_simd=1024, n_xcd=8):
    """Markdown rows from one counter run with SQ_INSTS_MFMA, SQ_INSTS_VALU,
    SQ_VALU_MFMA_BUSY_CYCLES, SQ_BUSY_CYCLES and GRBM_GUI_ACTIVE: per stage the
    per-launch instruction counts, the VALU : MFMA instruction ratio, and the
    matrix-core busy fraction = MFMA busy cycles / (GUI-active cycles of one
    XCD x the chip's SIMDs); GRBM_GUI_ACTIVE is summed over the XCDs."""
    d = read_pmc_csv(csv_path)
    names = ("SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE")
    m = {n: stage_counter_means(d, n) for n in names}
    rows = ["| stage | MFMA instr / launch | VALU instr / launch | VALU : MFMA | GUI-active cycles (one XCD) | "
            "MFMA busy |", "|---|---|---|---|---|---|"]
    for st in sorted(m["SQ_INSTS_MFMA"]):
        mf, va = m["SQ_INSTS_MFMA"][st], m["SQ_INSTS_VALU"].get(st, 0.0)
        gui = m["GRBM_GUI_ACTIVE"].get(st, 0.0) / n_xcd
        busy = m["SQ_VALU_MFMA_BUSY_CYCLES"].get(st, 0.0) / (gui * n_simd) if gui else 0.0
        ratio = f"{va / mf:.2f}" if mf else "-"
        rows.append(f"| {st} | {mf:.4g} | {va:.4g} | {ratio} | {gui:.4g} | {busy:.3f} |")
    return "\n".join(rows)


def kernel_source_sha(stage: str = "") -> str:
    """Hash of the sources a stage is built from (every source if the stage
    is unknown or empty)."""
    files = sorted(os.listdir(CSRC))
    if stage in STAGE_SOURCES:
        files = sorted(set(STAGE_SOURCES[stage] + _COMMON))
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or
    None when absent or taken on different kernel sources."""
    try:
        with open(COUNTERS) as fh:
            c = json.load(fh)
    except OSError:
        return None
    e = c.get(f"{workload}/{kernel}")
    if not e or e.get("source_sha") != kernel_source_sha(kernel):
        return None
    return e["hbm_bytes_per_launch"]


# ----------------------------------------------------------------- workloads
class Workload:
    name = ""
    unit = ""
    higher_is_better = True
    dtype = "bf16"
    dominant = ""
    bound = "mfma"

    def step(self):
        raise NotImplementedError

    def value(self, sec_per_step):
        raise NotImplementedError

    def dominant_work(self):
        """Algorithmic FLOPs (mfma) or bytes (hbm) per launch of the dominant kernel."""
        raise NotImplementedError


class MobaWorkload(Workload):
    def __init__(self, name, seed, n, hq, hkv, d, block, topk, dtype, planted=0, attn_rows=None):
        import query_aware_top_amd as qat
        import synth
        self.qat = qat
        self.name = name
        self.unit = "query-tokens/s"
        self.dtype = "bf16" if dtype == torch.bfloat16 else "f32"
        self.n, self.hq, self.hkv, self.d, self.block, self.topk = n, hq, hkv, d, block, topk
        self.q, self.k, self.v, _ = synth.moba_inputs(seed, 1, n, hq, hkv, d, dtype, "cuda", planted=planted,
                                                      block=block)
        self.q_start = 0 if attn_rows is None else n - attn_rows
        self.p_sel = qat.moba_params(batch=1, seq_len=n, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, block=block,
                                     topk=topk, dtype=dtype)
        self.p_att = qat.moba_params(batch=1, seq_len=n, n_q_heads=hq, n_kv_heads=hkv, head_dim=d,
                                     q_start=self.q_start, q_len=n - self.q_start, block=block, topk=topk,
                                     dtype=dtype)
        ws = max(qat.moba_workspace_size(self.p_sel), qat.moba_workspace_size(self.p_att))
        self.ws = torch.empty(ws, dtype=torch.uint8, device="cuda")
        self.blk = torch.empty(1, n, hq, topk, dtype=torch.int32, device="cuda")
        self.out = torch.empty(1, n - self.q_start, hq, d, dtype=dtype, device="cuda")
        self.lse = torch.empty(1, n - self.q_start, hq, dtype=torch.float32, device="cuda")
        self.dominant = "moba_past_attn"
        self.bound = "mfma" if dtype == torch.bfloat16 else "alu"
        if dtype != torch.bfloat16:
            self.dominant = "moba_generic_attn"

    def step(self):
        qat = self.qat
        qat.moba_block_select(self.p_sel, self.q, self.k, blk=self.blk, ws=self.ws)
        qat.moba_sparse_attn(self.p_att, self.q, self.k, self.v, self.blk[:, self.q_start:], out=self.out,
                             lse=self.lse, ws=self.ws)

    def value(self, sec):
        return (self.n - self.q_start) / sec

    def pair_counts(self):
        blk = self.blk[0, self.q_start:].to(torch.int64)
        t = torch.arange(self.q_start, self.n, device="cuda")
        cur = (t // self.block)[:, None, None]
        past = ((blk >= 0) & (blk < cur)).sum().item()
        cur_pairs = ((t % self.block) + 1).sum().item() * self.hq
        return past * self.block, cur_pairs

    def dominant_work(self):
        past_pairs, cur_pairs = self.pair_counts()
        if self.dominant == "moba_past_attn":
            return past_pairs * 4 * self.d
        return (past_pairs + cur_pairs) * 4 * self.d

    def config(self):
        return {"workload": self.name, "batch": 1, "seq_len": self.n, "n_q_heads": self.hq,
                "n_kv_heads": self.hkv, "head_dim": self.d, "block": self.block, "topk_incl_current": self.topk,
                "query_rows": self.n - self.q_start}

    def cpu_baseline(self, budget_s=12.0):
        """The float64 oracle on all host cores (one worker process each) over
        the workload's query rows in random order, as many 128-row chunks as
        the budget allows (block gating + attention, every head of each
        row); the block means over the whole sequence are computed first,
        inside the timed region."""
        import numpy as np
        from oracle import moba as omoba
        qp = _stage_gpu("moba_q", self.q[0])
        kp = _stage_gpu("moba_k", self.k[0])
        vp = _stage_gpu("moba_v", self.v[0])
        rows_all = np.random.default_rng(0).permutation(np.arange(self.q_start, self.n))
        chunks = [rows_all[i:i + 128].tolist() for i in range(0, len(rows_all), 128)]
        _, ncores = cpu_pool()
        t0 = time.perf_counter()
        kbar = omoba.block_means(np.load(kp).astype(np.float64), self.block)
        t_means = time.perf_counter() - t0
        items = [(qp, kp, vp, kbar, c, self.block, self.topk, self.p_att.scale) for c in chunks]
        res, el = _run_parallel(_moba_rows_task, items, budget_s - t_means)
        done = sum(res)
        el += t_means
        whole = done == len(rows_all)
        what = (f"all {done} query rows" if whole else
                f"{done} of the {len(rows_all)} query rows (random 128-row chunks)")
        return {"value": done / el, "unit": "query-tokens/s", "cores": ncores, "kind": "oracle",
                "sample": f"{what} of the {self.n}-token sequence, all {self.hq} heads each, block means over "
                          f"the whole sequence included; float64 numpy, {ncores} worker processes of one "
                          f"thread; {el:.1f} s"}

    def selection_bytes(self):
        """Gating of every row reads K once (mean pool) and Q once (block
        scores) and writes the gated lists."""
        el = 2 if self.dtype == "bf16" else 4
        return (self.n * self.hkv * self.d + self.n * self.hq * self.d) * el + self.n * self.hq * self.topk * 4


class MobaDecodeWorkload(Workload):
    """One MoBA decode step for a batch of sequences: the newest complete
    block's mean enters the kept cache (charged to every step, although a
    block completes only once per `block` steps), the new token's query rows
    are gated against the cache, and attend their gated blocks plus their own
    block up to the token."""

    def __init__(self, name, seed, batch, n, hq, hkv, d, block, topk, planted=0):
        import query_aware_top_amd as qat
        import synth
        self.qat = qat
        self.name = name
        self.unit, self.higher_is_better = "us/step", False
        self.dtype = "bf16"
        self.B, self.n, self.hq, self.hkv, self.d, self.block, self.topk = batch, n, hq, hkv, d, block, topk
        self.q, self.k, self.v, _ = synth.moba_decode_inputs(seed, batch, n, 1, hq, hkv, d, torch.bfloat16,
                                                             "cuda", planted=planted, block=block)
        self.p = qat.moba_params(batch=batch, seq_len=n, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, q_start=n - 1,
                                 q_len=1, block=block, topk=topk, dtype=torch.bfloat16)
        self.ws = torch.empty(qat.moba_workspace_size(self.p), dtype=torch.uint8, device="cuda")
        # the cache as earlier steps left it: every complete block before the
        # newest one (untimed prologue)
        self.newest = (n - 1) // block - 1
        self.kbar = qat.moba_block_means(self.p, self.k, 0, self.newest, ws=self.ws)
        self.blk = torch.empty(batch, 1, hq, topk, dtype=torch.int32, device="cuda")
        self.out = torch.empty(batch, 1, hq, d, dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty(batch, 1, hq, dtype=torch.float32, device="cuda")
        self.dominant, self.bound = "moba_decode_attn", "hbm"
        # the three calls of a step, marshalled once (fixed buffers): a step's
        # kernels take ~65 us, about what the Python-side checks of three
        # calls cost on the host, so each step re-issues the marshalled C ABI
        # calls (the library still validates every call)
        self.calls = [
            qat.plan(qat.moba_block_means, self.p, self.k, self.newest, 1, self.kbar, ws=self.ws),
            qat.plan(qat.moba_decode_select, self.p, self.q, self.kbar, blk=self.blk),
            qat.plan(qat.moba_decode_attn, self.p, self.q, self.k, self.v, self.blk, out=self.out, lse=self.lse,
                     ws=self.ws),
        ]

    def step(self):
        for c in self.calls:
            c()

    def value(self, sec):
        return sec * 1e6

    def dominant_work(self):
        """Distinct K and V rows the step must read (per sequence and KV
        head: the union of its query heads' gated blocks, plus the own block
        up to the token) and the query rows, in bytes."""
        blk = self.blk[:, 0].to("cpu")
        t = self.n - 1
        cur = t // self.block
        own = t - cur * self.block + 1
        rows = 0
        grp = self.hq // self.hkv
        for bi in range(self.B):
            for g in range(self.hkv):
                b = blk[bi, g * grp:(g + 1) * grp].flatten().tolist()
                past = {x for x in b if 0 <= x < cur}
                rows += len(past) * self.block + own
        return rows * self.d * 2 * 2 + self.B * self.hq * self.d * 2

    def config(self):
        return {"workload": self.name, "batch": self.B, "seq_len": self.n, "n_q_heads": self.hq,
                "n_kv_heads": self.hkv, "head_dim": self.d, "block": self.block, "topk_incl_current": self.topk,
                "query_rows_per_sequence": 1}

    def cpu_baseline(self, budget_s=12.0):
        """The float64 oracle on host cores for sequence 0, with the block
        means of its complete blocks computed beforehand (the kept cache):
        the newest block's mean, gating and attention of all heads; scaled by
        the batch."""
        import numpy as np
        from oracle import attention as oatt
        from oracle import moba as omoba
        kn = self.k[0].to("cpu").to(torch.float64).numpy()
        vn = self.v[0].to("cpu").to(torch.float64).numpy()
        kbar = omoba.block_means(kn, self.block)
        qt = self.q[0, 0].to("cpu").to(torch.float64).numpy()
        t = self.n - 1
        reps = 0
        t0 = time.perf_counter()
        while reps < 1 or time.perf_counter() - t0 < budget_s:
            nb = self.newest
            omoba.block_means(kn[nb * self.block:(nb + 1) * self.block], self.block)
            for h in range(self.hq):
                g = omoba.kv_head(h, self.hq, self.hkv)
                blk, _ = omoba.select_row(qt[h], kbar[:, g], t, self.block, self.topk)
                idx = omoba.key_set(blk, t, self.block)
                oatt.attend(qt[h], kn[idx, g], vn[idx, g], self.p.scale)
            reps += 1
        el = time.perf_counter() - t0
        return {"value": el / reps * 1e6 * self.B, "unit": "us/step", "cores": _blas_threads(), "kind": "oracle",
                "sample": f"sequence 0 of {self.B}, {reps} repetitions of its step (newest block mean, gating "
                          f"and attention of all {self.hq} heads; the other block means computed beforehand as "
                          f"the kept cache), scaled by {self.B} sequences; float64 numpy, one process; "
                          f"{el:.1f} s"}


class MobaBwdWorkload(Workload):
    """Gradients of MoBA prefill (gating held fixed) at the 32k GQA shape:
    the forward (gating, attention, lse) runs once before timing; a step is
    the backward call (dispatch, dq + D, own-block and gated-row key
    gradients)."""

    def __init__(self, name, seed, n, hq, hkv, d, block, topk, planted=0):
        import query_aware_top_amd as qat
        import synth
        self.qat = qat
        self.name = name
        self.unit = "query-tokens/s"
        self.dtype = "bf16"
        self.n, self.hq, self.hkv, self.d, self.block, self.topk = n, hq, hkv, d, block, topk
        self.q, self.k, self.v, _ = synth.moba_inputs(seed, 1, n, hq, hkv, d, torch.bfloat16, "cuda",
                                                      planted=planted, block=block)
        self.p = qat.moba_params(batch=1, seq_len=n, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, block=block,
                                 topk=topk, dtype=torch.bfloat16)
        self.ws = torch.empty(qat.moba_bwd_workspace_size(self.p), dtype=torch.uint8, device="cuda")
        self.blk = qat.moba_block_select(self.p, self.q, self.k, ws=self.ws)
        self.out, self.lse = qat.moba_sparse_attn(self.p, self.q, self.k, self.v, self.blk, ws=self.ws)
        self.do = synth.normal(seed, 7, (1, n, hq, d), torch.bfloat16, "cuda")
        self.dq = torch.empty(1, n, hq, d, dtype=torch.float32, device="cuda")
        self.dk = torch.empty(1, n, hkv, d, dtype=torch.float32, device="cuda")
        self.dv = torch.empty(1, n, hkv, d, dtype=torch.float32, device="cuda")
        self.dominant, self.bound = "moba_bwd_gated", "mfma"

    def step(self):
        self.qat.moba_sparse_attn_bwd(self.p, self.q, self.k, self.v, self.blk, self.do, self.lse, dq=self.dq,
                                      dk=self.dk, dv=self.dv, ws=self.ws)

    def value(self, sec):
        return self.n / sec

    def dominant_work(self):
        """The gated-row key kernel: 4 products of d per (row, key) pair of
        the gated blocks (s = q.k, dp = dO.v, dv += p dO, dk += ds q), 2 flops
        each: 8 d flops per pair (the hi + lo split of p and ds executes two
        of them twice; that is not counted)."""
        blk = self.blk[0].to(torch.int64)
        cur = (torch.arange(self.n, device="cuda") // self.block)[:, None, None]
        past = ((blk[..., :self.topk - 1] >= 0) & (blk[..., :self.topk - 1] < cur)).sum().item()
        return past * self.block * 8 * self.d

    def config(self):
        return {"workload": self.name, "batch": 1, "seq_len": self.n, "n_q_heads": self.hq,
                "n_kv_heads": self.hkv, "head_dim": self.d, "block": self.block, "topk_incl_current": self.topk,
                "query_rows": self.n, "pass": "backward"}

    def cpu_baseline(self, budget_s=12.0):
        """The float64 oracle's gradients on host cores for a bounded sample
        of query positions (all heads; their dq and their contributions to
        dk, dv), extrapolated to the sequence."""
        import numpy as np
        from oracle import moba as omoba
        kn = self.k[0].to("cpu").to(torch.float64).numpy()
        vn = self.v[0].to("cpu").to(torch.float64).numpy()
        qn = self.q[0].to("cpu").to(torch.float64).numpy()
        dn = self.do[0].to("cpu").to(torch.float64).numpy()
        blk = self.blk[0].cpu().numpy()
        order = np.random.default_rng(0).permutation(self.n)
        t0 = time.perf_counter()
        done = 0
        while done < self.n and (time.perf_counter() - t0 < budget_s or done < 4):
            t = int(order[done])
            omoba.backward_rows(qn, kn, vn, self.block, blk[[t]], [t], self.p.scale, dn[[t]])
            done += 1
        el = time.perf_counter() - t0
        return {"value": done / el, "unit": "query-tokens/s", "cores": 1, "kind": "oracle",
                "sample": f"{done} random query positions (all {self.hq} heads) of the {self.n}-token sequence: "
                          f"their dq and their dk, dv contributions; float64 numpy, one process and thread; "
                          f"{el:.1f} s"}


class CcaWorkload(Workload):
    """CCA-style core-token attention over a whole prefill: the core tokens of
    every group are pooled (each group's last query weighting its keys and
    values), then every position attends its core tokens plus its
    group-aligned window in one softmax."""

    def __init__(self, name, seed, n, h, d, group, window):
        import query_aware_top_amd as qat
        import synth
        self.qat = qat
        self.name = name
        self.unit = "query-tokens/s"
        self.dtype = "bf16"
        self.n, self.h, self.d, self.g, self.w = n, h, d, group, window
        self.q, self.k, self.v, _ = synth.moba_inputs(seed, 1, n, h, h, d, torch.bfloat16, "cuda")
        self.p = qat.cca_params(batch=1, seq_len=n, n_q_heads=h, n_kv_heads=h, head_dim=d, group=group,
                                window=window)
        self.kc = torch.empty(1, n // group, h, d, dtype=torch.bfloat16, device="cuda")
        self.vc = torch.empty_like(self.kc)
        self.out = torch.empty(1, n, h, d, dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty(1, n, h, dtype=torch.float32, device="cuda")
        self.dominant, self.bound = "cca_attn", "mfma"

    def step(self):
        self.qat.cca_pool(self.p, self.q, self.k, self.v, self.kc, self.vc)
        self.qat.cca_attn(self.p, self.q, self.k, self.v, self.kc, self.vc, out=self.out, lse=self.lse)

    def value(self, sec):
        return self.n / sec

    def _keys(self):
        t = torch.arange(self.n, dtype=torch.int64)
        wg = -(-self.w // self.g) * self.g
        ls = torch.clamp((t // self.g) * self.g - wg, min=0)
        return (ls // self.g) + (t - ls + 1)

    def dominant_work(self):
        """One (query, key, head) pair of the attention: 4 d flops (q.k and
        p v); keys per query = its core tokens + its window."""
        return int(self._keys().sum()) * self.h * 4 * self.d

    def config(self):
        return {"workload": self.name, "batch": 1, "seq_len": self.n, "n_heads": self.h, "head_dim": self.d,
                "group": self.g, "window": self.w}

    def cpu_baseline(self, budget_s=12.0):
        """The float64 oracle on host cores: pooling of the groups the
        sampled rows read plus attention of random rows (all heads),
        extrapolated to the sequence."""
        import numpy as np
        from oracle import cca as occa
        qn = self.q[0].to("cpu").to(torch.float64).numpy()
        kn = self.k[0].to("cpu").to(torch.float64).numpy()
        vn = self.v[0].to("cpu").to(torch.float64).numpy()
        t0 = time.perf_counter()
        need = occa.window_start(self.n - 1, self.g, self.w) // self.g
        kc, vc = occa.pool(qn, kn, vn, self.g, self.p.scale, need)
        t_pool = time.perf_counter() - t0
        order = np.random.default_rng(0).permutation(self.n)
        done = 0
        while done < self.n and (time.perf_counter() - t0 < budget_s or done < 2):
            occa.attend_rows(qn, kn, vn, kc, vc, self.g, self.w, self.p.scale, [int(order[done])])
            done += 1
        el = time.perf_counter() - t0
        est = t_pool + (el - t_pool) / done * self.n
        return {"value": self.n / est, "unit": "query-tokens/s", "cores": _blas_threads(), "kind": "oracle",
                "sample": f"pooling of all {need} groups ({t_pool:.1f} s) plus attention of {done} random rows "
                          f"(all {self.h} heads), extrapolated to the {self.n} rows; float64 numpy, one process; "
                          f"{el:.1f} s"}


class EsaBwdWorkload(Workload):
    """Gradients of the ESA chunk attention (selection held fixed) at the 64k
    prefill shape: compression, selection and attention run once before
    timing; a step is the backward call (dq + D, then dK/dV of the key
    list) into zeroed gradient buffers."""

    def __init__(self, name, seed, T, m, H, d, d_c, n_init, W, topk, radius, clip):
        import query_aware_top_amd as qat
        import synth
        self.qat = qat
        self.name = name
        self.unit = "query-tokens/s"
        self.dtype = "bf16"
        self.T, self.m, self.H, self.d, self.d_c = T, m, H, d, d_c
        self.c0, self.n_init, self.W, self.topk = T - m, n_init, W, topk
        _, self.k, self.v, _ = synth.esa_inputs(seed, 1, T, 1, H, d, torch.bfloat16, "cuda")
        self.q = synth.normal(seed, synth.gen.TID_Q, (1, m, H, d), torch.bfloat16, "cuda", start=1 << 40)
        Wq = synth.compression_weights(seed, d_c, H * d, synth.gen.TID_W, torch.bfloat16, "cuda")
        self.p = qat.esa_params(batch=1, n_heads=H, head_dim=d, d_c=d_c, ctx_len=T, chunk_start=self.c0,
                                chunk_len=m, n_init=n_init, window=W, topk=topk, radius=radius, clip=clip)
        kc = qat.esa_compress(self.k.view(T, H * d), Wq).view(1, T, d_c)
        self.sel, self.n_sel, _ = qat.esa_select(self.p, self.q, Wq, None, kc)
        _, self.lse = qat.esa_sparse_attn(self.p, self.q, self.k, self.v, self.sel, self.n_sel)
        self.do = synth.normal(seed, 7, (1, m, H, d), torch.bfloat16, "cuda")
        self.ws = torch.empty(qat.esa_bwd_workspace_size(self.p), dtype=torch.uint8, device="cuda")
        self.dq = torch.empty(1, m, H, d, dtype=torch.float32, device="cuda")
        self.dk = torch.zeros(1, T, H, d, dtype=torch.float32, device="cuda")
        self.dv = torch.zeros(1, T, H, d, dtype=torch.float32, device="cuda")
        self.dominant, self.bound = "esa_bwd_kv", "mfma"

    def step(self):
        self.qat.esa_sparse_attn_bwd(self.p, self.q, self.k, self.v, self.sel, self.n_sel, self.do, self.lse,
                                     dq=self.dq, dk=self.dk, dv=self.dv, ws=self.ws)

    def value(self, sec):
        return self.m / sec

    def dominant_work(self):
        """dK/dV kernel: 4 products of d per (query, key, head) pair (s, dp,
        dv, dk), 8 d flops; pairs per head m (gathered keys) + m (m + 1) / 2."""
        ng = min(self.n_init, self.c0) + int(self.n_sel[0]) + (self.c0 - max(self.n_init, self.c0 - self.W))
        pairs = self.m * ng + self.m * (self.m + 1) // 2
        return pairs * self.H * 8 * self.d

    def config(self):
        return {"workload": self.name, "batch": 1, "ctx_len": self.T, "chunk_len": self.m, "n_heads": self.H,
                "head_dim": self.d, "d_c": self.d_c, "n_init": self.n_init, "topk": self.topk, "window": self.W,
                "pass": "backward"}

    def cpu_baseline(self, budget_s=12.0):
        """The float64 oracle's gradients on host cores for a bounded sample of
        the chunk's queries (all heads: dq and their dK, dV contributions),
        extrapolated to the chunk."""
        import numpy as np
        from oracle import esa as oesa
        sg = self.sel[0, :int(self.n_sel[0])].cpu().numpy().astype(np.int64)
        idx = oesa.key_list(sg, self.c0, self.n_init, self.W, self.T - 1)
        kk = np.zeros((self.T, self.H, self.d))
        vv = np.zeros((self.T, self.H, self.d))
        ix = torch.as_tensor(idx, device="cuda")
        kk[idx] = self.k[0, ix].to("cpu").to(torch.float64).numpy()
        vv[idx] = self.v[0, ix].to("cpu").to(torch.float64).numpy()
        qn = self.q[0].to("cpu").to(torch.float64).numpy()
        dn = self.do[0].to("cpu").to(torch.float64).numpy()
        order = np.random.default_rng(0).permutation(self.m)
        t0 = time.perf_counter()
        done = 0
        while done < self.m and (time.perf_counter() - t0 < budget_s or done < 2):
            i = int(order[done])
            oesa.backward(qn, kk, vv, sg, self.c0, self.n_init, self.W, self.p.scale, dn[[i]], rows=[i])
            done += 1
        el = time.perf_counter() - t0
        return {"value": done / el, "unit": "query-tokens/s", "cores": _blas_threads(), "kind": "oracle",
                "sample": f"{done} random queries (all {self.H} heads) of the {self.m}-query chunk: their dq and "
                          f"dK, dV contributions; float64 numpy, one process; {el:.1f} s"}


class EsaWorkload(Workload):
    def __init__(self, name, seed, batch, T, m, H, d, d_c, n_init, W, topk, radius, clip, needles=0,
                 correction="clamp", per_head=False):
        import query_aware_top_amd as qat
        import synth
        self.qat = qat
        self.name = name
        self.B, self.T, self.m, self.H, self.d, self.d_c = batch, T, m, H, d, d_c
        self.c0 = T - m
        self.n_init, self.W, self.topk = n_init, W, topk
        dtype = torch.bfloat16
        _, self.k, self.v, _ = synth.esa_inputs(seed, batch, T, 1, H, d, dtype, "cuda")
        self.q = synth.normal(seed, synth.gen.TID_Q, (batch, m, H, d), dtype, "cuda", start=1 << 40)
        if needles:
            for bi in range(batch):
                pos = synth.needle_positions(seed, bi, needles, n_init, self.c0 - W, 2 * radius + 1)
                val = (self.q[bi, 0].to(torch.float64) * 0.375).to(dtype)
                for t in pos:
                    self.k[bi, t] = val
        self.correction = correction
        self.per_head = per_head
        self.p = qat.esa_params(batch=batch, n_heads=H, head_dim=d, d_c=d_c, ctx_len=T, chunk_start=self.c0,
                                chunk_len=m, n_init=n_init, window=W, topk=topk, radius=radius, clip=clip,
                                correction=correction, per_head=per_head)
        self.ws = torch.empty(qat.esa_workspace_size(self.p), dtype=torch.uint8, device="cuda")
        if not per_head:
            self.Wq = synth.compression_weights(seed, d_c, H * d, synth.gen.TID_W, dtype, "cuda")
            self.Wk = self.Wq
            # compressed-key cache of the tokens before the chunk: state written
            # by earlier steps (untimed prologue)
            self.kc = torch.zeros(batch, T, d_c, dtype=dtype, device="cuda")
            qat.esa_compress(self.k.view(batch * T, H * d), self.Wk, out=self.kc.view(batch * T, d_c))
            import ctypes
            nb = ctypes.c_size_t(0)
            qat.lib().esa_compress_workspace_size(batch * m, H * d, d_c, ctypes.byref(nb))
            self.ws_c = torch.empty(max(nb.value, 256), dtype=torch.uint8, device="cuda")
        nsel = (batch, H) if per_head else (batch,)
        self.sel = torch.empty(*nsel, topk, dtype=torch.int32, device="cuda")
        self.n_sel = torch.empty(*nsel, dtype=torch.int32, device="cuda")
        self.out = torch.empty(batch, m, H, d, dtype=dtype, device="cuda")
        self.lse = torch.empty(batch, m, H, dtype=torch.float32, device="cuda")
        self.n_mid = max(n_init, self.c0 - W) - n_init if self.c0 > n_init else 0
        if m == 1:
            self.unit, self.higher_is_better = "us/step", False
            self.dominant, self.bound = ("esa_decode_scan" if per_head else "esa_decode_attn"), "hbm"
        else:
            self.unit = "query-tokens/s"
            self.dominant, self.bound = ("esa_colsum" if per_head else "esa_prefill_attn"), "mfma"

    def step(self):
        qat = self.qat
        B, T, H, d, m = self.B, self.T, self.H, self.d, self.m
        if self.per_head:   # one selection per (sequence, head) from the raw q, k; then attention
            qat.esa_select_heads(self.p, self.q, self.k, sel=self.sel, n_sel=self.n_sel, ws=self.ws)
            qat.esa_sparse_attn(self.p, self.q, self.k, self.v, self.sel, self.n_sel, out=self.out, lse=self.lse,
                                ws=self.ws)
            return
        # compress the chunk's new keys into the cache
        qat.esa_compress(self.k.view(B * T, H * d)[self.c0:], self.Wk, out=self.kc.view(B * T, -1)[self.c0:],
                         n=B if m == 1 else m, x_stride=T * H * d if m == 1 else H * d,
                         out_stride=T * self.d_c if m == 1 else self.d_c, ws=self.ws_c)
        qat.esa_select(self.p, self.q, self.Wq, None, self.kc, sel=self.sel, n_sel=self.n_sel, ws=self.ws)
        qat.esa_sparse_attn(self.p, self.q, self.k, self.v, self.sel, self.n_sel, out=self.out, lse=self.lse,
                            ws=self.ws)

    def value(self, sec):
        return sec * 1e6 if self.m == 1 else self.B * self.m / sec

    def n_keys(self):
        n_i = min(self.n_init, self.c0)
        n_l = self.c0 - max(self.n_init, self.c0 - self.W) if self.c0 > self.n_init else 0
        return n_i + int(self.n_sel.flatten()[0]) + n_l

    def dominant_work(self):
        if self.per_head:
            if self.m == 1:   # decode scan: every head's K row of every middle token, + the query rows
                return self.B * self.H * self.n_mid * self.d * 2 + self.B * self.H * self.d * 2
            # second scoring pass: q.k of every (query, middle token, head), 2 d flop
            return 2 * self.m * self.n_mid * self.H * self.d * self.B
        if self.m == 1:   # gathered K and V rows of every head + q and out
            return self.B * (self.n_keys() + 1) * self.H * self.d * 2 * 2 + 2 * self.B * self.H * self.d * 2
        g = self.n_keys()
        pairs = self.m * g + self.m * (self.m + 1) // 2
        return pairs * self.H * 4 * self.d

    def config(self):
        return {"workload": self.name, "batch": self.B, "ctx_len": self.T, "chunk_len": self.m,
                "n_heads": self.H, "head_dim": self.d, "d_c": self.d_c, "n_init": self.n_init,
                "topk": self.topk, "window": self.W, "correction": self.correction,
                "selection": "per_head" if self.per_head else "merged_heads"}

    def cpu_baseline(self, budget_s=12.0):
        """The float64 oracle doing the GPU step's work on all host cores:
        compression of the chunk's new keys into the cache of earlier keys
        (that cache is state, staged from the library's bit-identical
        cache), the selection, and attention of the chunk's rows. Prefill:
        compression and selection in this process (its BLAS on every core),
        attention rows over the worker pool. Decode: the sequences' selections
        over the pool, then their attention over the pool. Staging the
        inputs, and the selected K/V rows between the two phases, is not
        timed."""
        if self.per_head:
            return self._cpu_baseline_heads(budget_s)
        import numpy as np
        from oracle import esa as oesa
        _, ncores = cpu_pool()
        W = self.Wq.to("cpu").to(torch.float64).numpy()
        if self.m > 1:
            bi = 0
            kc = self.kc[bi].to("cpu").to(torch.float64).numpy()
            knew = self.k[bi, self.c0:].to("cpu").to(torch.float64).numpy()
            qn = self.q[bi].to("cpu").to(torch.float64).numpy()
            qp = _stage("esa_q", qn.astype(np.float32))
            t0 = time.perf_counter()
            kc[self.c0:] = oesa.key_cache(knew, W)
            sel, _, _, _ = oesa.select(qn, W, None, kc, self.c0, self.n_init, self.W, self.topk, self.p.radius,
                                       self.p.clip, correction=self.correction)
            t_sel = time.perf_counter() - t0
            pos = oesa.key_list(sel, self.c0, self.n_init, self.W, self.T - 1)
            ix = torch.as_tensor(pos, device="cuda")
            kp = _stage_gpu("esa_k", self.k[bi].index_select(0, ix))
            vp = _stage_gpu("esa_v", self.v[bi].index_select(0, ix))
            order = np.random.default_rng(0).permutation(self.m)
            items = [(qp, kp, vp, pos, sel, self.c0, self.n_init, self.W, self.p.scale, order[i:i + 16].tolist())
                     for i in range(0, self.m, 16)]
            res, t_att = _run_parallel(_esa_attend_task, items, budget_s - t_sel)
            rows = sum(res)
            est = t_sel + t_att * self.m / rows
            what = (f"compression of the chunk's {self.m} new keys and the selection ({t_sel:.1f} s, this "
                    f"process, BLAS threads {_blas_threads()}), then attention of "
                    + (f"all {rows} rows" if rows == self.m else f"{rows} of the {self.m} rows, extrapolated")
                    + f" over {ncores} worker processes")
            return {"value": self.m / est, "unit": "query-tokens/s", "cores": ncores, "kind": "oracle",
                    "sample": f"{what}; float64 numpy; {t_sel + t_att:.1f} s"}
        # decode: every sequence of the batch
        qp = _stage_gpu("esa_q", self.q[:, 0])
        kcp = _stage_gpu("esa_kc", self.kc)
        knp = _stage_gpu("esa_knew", self.k[:, self.c0:self.c0 + 1])
        Wp = _stage("esa_W", W)
        items = [(qp, kcp, knp, Wp, bi, self.c0, self.n_init, self.W, self.topk, self.p.radius, self.p.clip,
                  self.correction) for bi in range(self.B)]
        res, t_sel = _run_parallel(_esa_select_task, items, 1e9)
        sels = dict(res)
        items = []
        for bi in range(self.B):
            pos = oesa.key_list(sels[bi], self.c0, self.n_init, self.W, self.T - 1)
            ix = torch.as_tensor(pos, device="cuda")
            q1 = _stage_gpu(f"esa_q{bi}", self.q[bi])
            kp = _stage_gpu(f"esa_k{bi}", self.k[bi].index_select(0, ix))
            vp = _stage_gpu(f"esa_v{bi}", self.v[bi].index_select(0, ix))
            items.append((q1, kp, vp, pos, sels[bi], self.c0, self.n_init, self.W, self.p.scale, [0]))
        res, t_att = _run_parallel(_esa_attend_task, items, 1e9)
        el = t_sel + t_att
        return {"value": el * 1e6, "unit": "us/step", "cores": ncores, "kind": "oracle",
                "sample": f"all {self.B} sequences: compression of the new key into each cache and the "
                          f"selection ({t_sel:.2f} s), then attention of all {self.H} heads ({t_att:.2f} s), "
                          f"one sequence per task over {ncores} worker processes; float64 numpy"}

    def step_bytes(self):
        """Algorithmic bytes of one decode step: the compressed keys of the
        middle part (scan), the gathered K and V rows of every head, the new
        token's key row compressed into the cache, q, out and the two
        compression maps."""
        B, H, d, dc = self.B, self.H, self.d, self.d_c
        scan = B * self.n_mid * dc * 2
        kv = B * (self.n_keys() + 1) * H * d * 2 * 2
        newkey = B * (H * d * 2 + dc * 2)
        qo = 2 * B * H * d * 2
        maps = 2 * dc * H * d * 2
        return scan + kv + newkey + qo + maps


    def _cpu_baseline_heads(self, budget_s):
        """Per-head selection of sequence 0 for as many heads as fit in about
        two thirds of the budget (at least one), scaled to all heads; then
        attention rows over per-head lists (the computed heads' lists reused
        for the others, which costs the same), scaled to the chunk."""
        import numpy as np
        from oracle import esa as oesa
        bi = 0
        _, M, _ = oesa.partition(self.c0, self.n_init, self.W)
        qn = self.q[bi].to("cpu").to(torch.float64).numpy()
        t0 = time.perf_counter()
        sels = []
        while len(sels) < self.H and (time.perf_counter() - t0 < budget_s * 2 / 3 or not sels):
            h = len(sels)
            kh = self.k[bi, int(M[0]):int(M[-1]) + 1, h:h + 1].to("cpu").to(torch.float64).numpy() if M.size else None

            class _View:   # K[M, 0] of the one head loaded above
                def __getitem__(self, idx, kh=kh):
                    return kh[np.asarray(idx[0]) - int(M[0]), 0]

            s, _ = oesa.select_heads(qn[:, h:h + 1], _View(), self.c0, self.n_init, self.W, self.topk,
                                     self.p.radius, self.p.clip, correction=self.correction)
            sels.append(s[0])
        t_sel = (time.perf_counter() - t0) * self.H / len(sels)
        nh = len(sels)
        all_sels = [sels[h % nh] for h in range(self.H)]
        kk, vv = _GpuRows(self.k[bi]), _GpuRows(self.v[bi])
        order = np.random.default_rng(0).permutation(self.m)
        t1 = time.perf_counter()
        rows = 0
        while rows < self.m and (time.perf_counter() - t0 < budget_s or rows < 1):
            oesa.attend(qn, kk, vv, all_sels, self.c0, self.n_init, self.W, self.p.scale, rows=[int(order[rows])])
            rows += 1
        t_att = (time.perf_counter() - t1) / rows * self.m
        el = time.perf_counter() - t0
        cores = _blas_threads()
        what = (f"per-head selection of sequence 0 for {nh} of {self.H} heads, scaled to all heads, plus "
                f"attention for {rows} of {self.m} rows, scaled to the chunk")
        if self.m == 1:
            return {"value": (t_sel + t_att) * 1e6 * self.B, "unit": "us/step", "cores": cores, "kind": "oracle",
                    "sample": f"{what}, times {self.B} sequences; float64 numpy, one process; {el:.1f} s"}
        return {"value": self.m / (t_sel + t_att), "unit": "query-tokens/s", "cores": cores, "kind": "oracle",
                "sample": f"{what}; float64 numpy, BLAS threads for the matrix products, one process; {el:.1f} s"}


# ------------------------------------------------------- oracle on host cores
# The oracle baseline runs in worker processes, one per host core, forked at
# the start of main() before anything touches the GPU (they never do). The
# inputs they read are staged into .npy files under TMPDIR and memory-mapped,
# so every worker shares one page-cached copy. The box gives one GPU process
# 16 CPUs whatever the host reports.
_POOL = None
_POOL_N = 0
_STAGE_DIR = None


def _worker_init():
    os.environ["OMP_NUM_THREADS"] = "1"
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass
    # the oracle's modules, imported once per worker before any timed task
    import oracle.attention  # noqa: F401
    import oracle.esa  # noqa: F401
    import oracle.moba  # noqa: F401


def cpu_pool():
    global _POOL, _POOL_N
    if _POOL is None:
        import multiprocessing as mp
        _POOL_N = max(1, min(16, os.cpu_count() or 1))
        _POOL = mp.get_context("fork").Pool(_POOL_N, initializer=_worker_init)
    return _POOL, _POOL_N


def close_cpu_pool():
    global _POOL, _STAGE_DIR
    if _POOL is not None:
        _POOL.close()
        _POOL.join()
        _POOL = None
    if _STAGE_DIR is not None:
        import shutil
        shutil.rmtree(_STAGE_DIR, ignore_errors=True)
        _STAGE_DIR = None


def _stage(name, arr):
    """Writes arr (numpy) to a staging .npy file and returns its path."""
    global _STAGE_DIR
    import tempfile
    import numpy as np
    if _STAGE_DIR is None:
        _STAGE_DIR = tempfile.mkdtemp(prefix="qat_oracle_", dir=os.environ.get("TMPDIR", "/tmp"))
    path = os.path.join(_STAGE_DIR, name + ".npy")
    np.save(path, arr)
    return path


def _stage_gpu(name, t):
    """A device tensor staged as float32 (bf16 values widen exactly)."""
    return _stage(name, t.to(torch.float32).cpu().numpy())


def _run_parallel(task, items, budget_s, min_items=1):
    """Runs task(item) over the pool, keeping every worker busy until
    budget_s has passed (and at least min_items are done); returns (results
    in completion order, wall seconds)."""
    pool, n = cpu_pool()
    t0 = time.perf_counter()
    pending, results, nxt = [], [], 0
    while nxt < len(items) or pending:
        while (nxt < len(items) and len(pending) < 2 * n
               and (time.perf_counter() - t0 < budget_s or len(results) + len(pending) < min_items)):
            pending.append(pool.apply_async(task, (items[nxt],)))
            nxt += 1
        if not pending:
            break
        pending[0].wait()
        done = [p for p in pending if p.ready()]
        pending = [p for p in pending if not p.ready()]
        results.extend(p.get() for p in done)
    return results, time.perf_counter() - t0


def _moba_rows_task(a):
    """Oracle gating + attention of some query rows, all heads."""
    import numpy as np
    from oracle import attention as oatt
    from oracle import moba as omoba
    qp, kp, vp, kbar, rows, block, topk, scale = a
    q, k, v = (np.load(x, mmap_mode="r") for x in (qp, kp, vp))
    hq, hkv = q.shape[1], k.shape[1]
    for t in rows:
        qt = np.asarray(q[t], np.float64)
        for h in range(hq):
            g = omoba.kv_head(h, hq, hkv)
            blk, _ = omoba.select_row(qt[h], kbar[:, g], t, block, topk)
            idx = omoba.key_set(blk, t, block)
            oatt.attend(qt[h], np.asarray(k[idx, g], np.float64), np.asarray(v[idx, g], np.float64), scale)
    return len(rows)


class _ListedRows:
    """A K or V cache seen through the rows of listed positions only: x[i]
    holds position pos[i]; indexing by positions (and optionally heads)
    returns float64 rows."""

    def __init__(self, x, pos):
        self.x = x
        self.shape = x.shape
        self.where = {int(p): i for i, p in enumerate(pos)}

    def __getitem__(self, idx):
        import numpy as np
        rest = ()
        if isinstance(idx, tuple):
            idx, rest = idx[0], idx[1:]
        ii = [self.where[int(j)] for j in np.asarray(idx).reshape(-1)]
        return np.asarray(self.x[ii], np.float64)[(slice(None),) + rest]


def _esa_attend_task(a):
    """Oracle attention of some chunk rows (all heads) over one sequence's
    key list; kp / vp hold only the listed rows, pos their positions."""
    import numpy as np
    from oracle import esa as oesa
    qp, kp, vp, pos, sel, c0, n_init, W, scale, rows = a
    q = np.load(qp, mmap_mode="r")
    k, v = np.load(kp, mmap_mode="r"), np.load(vp, mmap_mode="r")
    qn = np.asarray(q, np.float64)
    oesa.attend(qn, _ListedRows(k, pos), _ListedRows(v, pos), sel, c0, n_init, W, scale, rows=list(rows))
    return len(rows)


def _esa_select_task(a):
    """Oracle step for one sequence of a decode batch up to the selection:
    compression of the new key into the cache, then the selection."""
    import numpy as np
    from oracle import esa as oesa
    qp, kcp, knewp, Wp, bi, c0, n_init, W, topk, radius, clip, correction = a
    q = np.asarray(np.load(qp, mmap_mode="r")[bi], np.float64)
    kc = np.asarray(np.load(kcp, mmap_mode="r")[bi], np.float64)
    Wn = np.load(Wp)
    kc[c0:c0 + 1] = oesa.key_cache(np.asarray(np.load(knewp, mmap_mode="r")[bi], np.float64), Wn)
    sel, _, _, _ = oesa.select(q, Wn, None, kc, c0, n_init, W, topk, radius, clip, correction=correction)
    return bi, sel


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        return 1


class _GpuRows:
    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, idx):
        import numpy as np
        rest = ()
        if isinstance(idx, tuple):   # rows, then an index into the remaining dimensions
            idx, rest = idx[0], idx[1:]
        ix = torch.as_tensor(np.asarray(idx), device=self.t.device, dtype=torch.long)
        return self.t.index_select(0, ix)[(slice(None),) + rest].to("cpu").to(torch.float64).numpy()


def make(name):
    if name == "moba_gqa_32k":
        return MobaWorkload(name, 2, 32768, 32, 8, 128, 512, 3, torch.bfloat16, planted=8)
    if name == "moba_fp32_4k":
        return MobaWorkload(name, 1, 4096, 4, 4, 64, 256, 3, torch.float32)
    if name == "moba_long_512k":
        return MobaWorkload(name, 5, 524288, 8, 8, 128, 8192, 3, torch.bfloat16, attn_rows=8192)
    if name == "moba_decode_128k":
        return MobaDecodeWorkload(name, 128, 16, 131072, 32, 8, 128, 512, 3, planted=8)
    if name == "moba_bwd_32k":
        return MobaBwdWorkload(name, 2, 32768, 32, 8, 128, 512, 3, planted=8)
    if name == "esa_prefill_64k":
        return EsaWorkload(name, 3, 1, 65536, 2048, 32, 128, 128, 128, 4096, 2048, 2, 48.0)
    if name == "esa_decode_128k":
        return EsaWorkload(name, 4, 16, 131072, 1, 32, 128, 128, 128, 4096, 2048, 2, 48.0, needles=16)
    if name == "cca_64k":
        return CcaWorkload(name, 6, 65536, 32, 128, 16, 1024)
    if name == "esa_bwd_64k":
        return EsaBwdWorkload(name, 3, 65536, 2048, 32, 128, 128, 128, 4096, 2048, 2, 48.0)
    if name == "esa_prefill_64k_votes":
        return EsaWorkload(name, 3, 1, 65536, 2048, 32, 128, 128, 128, 4096, 2048, 2, 48.0, correction="votes")
    if name == "esa_decode_128k_votes":
        return EsaWorkload(name, 4, 16, 131072, 1, 32, 128, 128, 128, 4096, 2048, 2, 48.0, needles=16,
                           correction="votes")
    if name == "esa_prefill_64k_heads":
        return EsaWorkload(name, 3, 1, 65536, 2048, 32, 128, 128, 128, 4096, 2048, 2, 48.0, per_head=True)
    if name == "esa_decode_128k_heads":
        return EsaWorkload(name, 4, 16, 131072, 1, 32, 128, 128, 128, 4096, 2048, 2, 48.0, needles=16,
                           per_head=True)
    raise SystemExit(f"unknown workload {name}")


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def measure(w, steps, warmup):
    """Times one workload: warmup, then `steps` timed steps (the library
    brackets only the dominant kernel with events, on the stream it runs on,
    so the roofline's launch time is measured live in this region), a second
    untimed pass with every stage bracketed, and the spread of single steps
    (for HBM-bound workloads also with L2 and the Infinity Cache flushed
    before each step). Returns the fields of the bench line."""
    qat = w.qat
    for _ in range(warmup):
        w.step()
    torch.cuda.synchronize()
    qat.timing_enable(True)
    qat.timing_select(w.dominant)
    qat.timing_reset()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        w.step()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    tot, n = qat.timing_query(w.dominant)
    dom_ms = round(tot / n, 4) if n else None
    # per-stage breakdown from a second, untimed pass with every stage bracketed
    qat.timing_select(None)
    qat.timing_reset()
    for _ in range(steps):
        w.step()
    torch.cuda.synchronize()
    qat.timing_enable(False)
    kernels = {}
    for name in STAGES:
        tot, n = qat.timing_query(name)
        if n:
            kernels[name] = round(tot / n, 4)
    qat.timing_reset()

    # spread of single steps (outside the timed region above): events around
    # each step; for the HBM-bound workloads also with L2 and the 256 MiB
    # Infinity Cache flushed before every step by reading 1 GiB of other data
    # (untimed; a read leaves clean lines, so the step pays no write-back)
    def step_times(flush):
        buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda") if flush else None
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in ev:
            if flush:
                buf.sum()
            a.record()
            w.step()
            b.record()
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in ev)

    def pct(t, q):
        return round(t[min(len(t) - 1, int(q * (len(t) - 1) + 0.5))], 4)

    warm = step_times(False)
    spread = {"p10": pct(warm, 0.1), "p50": pct(warm, 0.5), "p90": pct(warm, 0.9)}
    cold_dom_ms = None
    if w.bound == "hbm":
        # the dominant kernel's launches in these cold steps are timed too
        qat.timing_enable(True)
        qat.timing_select(w.dominant)
        qat.timing_reset()
        cold = step_times(True)
        tot, n = qat.timing_query(w.dominant)
        qat.timing_enable(False)
        qat.timing_reset()
        spread["cold_p50"] = pct(cold, 0.5)
        cold_dom_ms = round(tot / n, 4) if n else None
    work = w.dominant_work()
    if w.bound == "hbm":
        achieved = work / (dom_ms * 1e-3) / 1e9
        peak, unit = PEAK_HBM_GBS, "GB/s"
    elif w.bound == "mfma":
        achieved = work / (dom_ms * 1e-3) / 1e12
        peak, unit = PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        achieved = work / (dom_ms * 1e-3) / 1e12
        peak, unit = PEAK_F32_TFLOPS, "TFLOP/s"
    roof = {"kernel": w.dominant, "bound": w.bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic_for(w.dominant, w.name),
            "work_per_launch": work, "avg_launch_ms": dom_ms}
    if cold_dom_ms:
        # the same kernel with L2 and the Infinity Cache flushed before each step
        roof["cold_avg_launch_ms"] = cold_dom_ms
        roof["cold_frac"] = round(work / (cold_dom_ms * 1e-3) / 1e9 / peak, 4)
    return {"value": w.value(ms * 1e-3), "ms_per_step": ms, "roofline": roof, "kernels_avg_ms": kernels,
            "step_ms": spread}


STAGES = ("moba_meanpool", "moba_select", "moba_dispatch", "moba_past_attn", "moba_current_attn",
          "moba_generic_attn", "moba_decode_select", "moba_decode_attn", "moba_decode_combine",
          "moba_bwd_dq_past", "moba_bwd_dq", "moba_bwd_own", "moba_bwd_gated", "esa_bwd_dq", "esa_bwd_kv",
          "cca_pool", "cca_attn",
          "esa_compress", "esa_qcompress", "esa_scores", "esa_decode_scan", "esa_topk",
          "esa_prefill_attn", "esa_decode_attn", "esa_generic_attn")

# Workloads summarised in the default line beside moba_gqa_32k: the ESA
# decode step (the metric's decode half), ESA chunked prefill and MoBA's
# 512k fixed-sparsity case.
EXTRA = ("esa_decode_128k", "esa_prefill_64k", "moba_long_512k")


def summary(w, r):
    """Compact record of one extra workload's measurement."""
    roof = r["roofline"]
    out = {"workload": w.name, "value": round(r["value"], 3), "unit": w.unit,
           "ms_per_step": round(r["ms_per_step"], 4), "step_ms": r["step_ms"],
           "dominant": {k: roof[k] for k in ("kernel", "bound", "achieved", "unit", "frac", "avg_launch_ms",
                                             "traffic", "cold_frac", "cold_avg_launch_ms") if k in roof},
           "kernels_avg_ms": r["kernels_avg_ms"]}
    sb = getattr(w, "step_bytes", None)
    if sb is not None and w.bound == "hbm" and not getattr(w, "per_head", False):
        # HBM-bound step: algorithmic bytes of the whole step against its time
        b = sb()
        out["step_bytes"] = b
        out["step_hbm_frac"] = round(b / (r["ms_per_step"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        if "cold_p50" in r["step_ms"]:
            out["cold_step_hbm_frac"] = round(b / (r["step_ms"]["cold_p50"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
    sel = getattr(w, "selection_bytes", None)
    if sel is not None:   # MoBA gating over all rows: mean pool + block scores, HBM-bound
        b = sel()
        k = r["kernels_avg_ms"]
        t = k.get("moba_meanpool", 0.0) + k.get("moba_select", 0.0)
        if t > 0:
            out["selection"] = {"bytes": b, "ms": round(t, 4), "GBps": round(b / (t * 1e-3) / 1e9, 1),
                                "frac": round(b / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="moba_gqa_32k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="measure only --workload (the default line otherwise also summarises "
                         + ", ".join(EXTRA) + ")")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="run one plain device-to-device copy of BYTES before warmup (reference kernel for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--ingest-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: read the counter_collection.csv files of a FETCH_SIZE and a WRITE_SIZE "
                         "rocprofv3 run of --workload (made with --copy-calibration BYTES) and store the "
                         "per-launch HBM bytes of its stages in profiles/counters.json")
    ap.add_argument("--mfma-table", metavar="CSV",
                    help="no GPU work: print per-stage MFMA / VALU counter rows of one rocprofv3 run")
    args = ap.parse_args()
    if args.ingest_traffic:
        if not args.copy_calibration:
            raise SystemExit("--ingest-traffic needs the --copy-calibration size the runs used")
        for k, v in ingest_traffic(args.workload, *args.ingest_traffic, args.copy_calibration).items():
            print(k, json.dumps(v))
        return
    if args.mfma_table:
        print(mfma_table(args.mfma_table))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this library has no multi-GPU path (asked for --gpus {args.gpus}); "
              f"see DESIGN.md for how the path would shard.", file=sys.stderr)
        sys.exit(2)
    # the oracle's worker processes are forked before anything touches the GPU
    if not args.no_cpu_baseline:
        cpu_pool()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import query_aware_top_amd as qat
    qat.lib()
    w = make(args.workload)
    torch.cuda.synchronize()
    if args.copy_calibration:
        src = torch.ones(args.copy_calibration // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    r = measure(w, args.steps, args.warmup)
    line = {
        "metric": METRIC,
        "value": round(r["value"], 3),
        "unit": w.unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": w.higher_is_better,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) inputs generated on the GPU; see DESIGN.md for the recipe)",
        "config": w.config(),
        "roofline": r["roofline"],
        "kernels_avg_ms": r["kernels_avg_ms"],
        "step_ms": r["step_ms"],
    }
    if not args.no_cpu_baseline:
        cb = w.cpu_baseline()
        cb["sample"] += f"; host {_cpu_model()}, {os.cpu_count()} logical CPUs"
        line["cpu_baseline"] = cb
    if args.workload == "moba_gqa_32k" and not args.no_extra:
        del w
        torch.cuda.empty_cache()
        configs = {}
        for name in EXTRA:
            w2 = make(name)
            torch.cuda.synchronize()
            s2 = summary(w2, measure(w2, args.steps, args.warmup))
            s2["config"] = w2.config()
            if name == "esa_decode_128k":
                line["decode"] = s2
            else:
                configs[name] = s2
            del w2
            torch.cuda.empty_cache()
        line["configs"] = configs
    print(json.dumps(line), flush=True)
    close_cpu_pool()


if __name__ == "__main__":
    main()
