"""GPU parity of the MoBA path (moba_block_select + moba_sparse_attn through
the C ABI) against the float64 CPU oracle on the same seeded inputs."""
import math

import numpy as np
import pytest
import torch

import query_aware_top_amd as qat
import synth
from oracle import attention as oatt
from oracle import moba as omoba
from parity import BF16_TOL, F32_TOL, assert_close, moba_rows_ok, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run(q, k, v, block, topk, dtype, q_start=0, q_len=None, window=0):
    p = qat.moba_params(batch=q.shape[0], seq_len=q.shape[1], n_q_heads=q.shape[2], n_kv_heads=k.shape[2],
                        head_dim=q.shape[3], q_start=q_start, q_len=q_len, block=block, topk=topk,
                        window=window, dtype=dtype)
    blk = qat.moba_block_select(p, q, k)
    out, lse = qat.moba_sparse_attn(p, q, k, v, blk)
    torch.cuda.synchronize()
    return p, blk, out, lse


def check(q, k, v, block, topk, dtype, rows=None, q_start=0, q_len=None, window=0, tol=None):
    p, blk, out, lse = run(q, k, v, block, topk, dtype, q_start, q_len, window)
    tol = tol or (BF16_TOL if dtype == torch.bfloat16 else F32_TOL)
    lse_tol = 1e-3 if dtype == torch.bfloat16 else 1e-5
    if rows is None:
        rows = list(range(q_start, q_start + p.q_len))
    rel = [t - q_start for t in rows]
    total_swaps = 0
    for bi in range(q.shape[0]):
        qn, kn, vn = to64(q[bi]), to64(k[bi]), to64(v[bi])
        kbar = omoba.block_means(kn, block)
        blk_ref, sc = omoba.select(qn, kn, block, topk, rows, kbar)
        blk_g = blk[bi, rel].cpu().numpy()
        bad, swaps = moba_rows_ok(blk_g, blk_ref, sc, rows, block, topk)
        assert not bad, f"selection mismatch outside the tie band: {bad[:5]}"
        total_swaps += swaps
        o_ref, lse_ref = omoba.attend_rows(qn, kn, vn, block, blk_g, rows, p.scale, window)
        assert_close(to64(out[bi, rel]), o_ref, tol, "output")
        assert_close(to64(lse[bi, rel]), lse_ref, lse_tol, "lse")
    return blk, out, total_swaps


def test_moba_fp32_4k_parity_config():
    """MoBA block-sparse causal prefill, fp32: batch 1, 4 heads, d 64, N 4096,
    block 256, top-k 3 (and the 3-past + current reading k = 4)."""
    q, k, v, _ = synth.moba_inputs(1, 1, 4096, 4, 4, 64, torch.float32, DEV)
    for topk in (3, 4):
        print(f"[moba fp32 4k] topk={topk}", flush=True)
        check(q, k, v, 256, topk, torch.float32)


SMALL = [
    # batch, N, hq, hkv, d, block, topk, q_start, q_len, window, dtype
    (1, 1000, 4, 2, 128, 128, 3, 0, None, 0, torch.bfloat16),   # ragged N, GQA, several tiles
    (2, 777, 2, 2, 64, 64, 4, 100, 500, 0, torch.bfloat16),      # batch 2, offset rows, d 64
    (1, 600, 4, 1, 128, 64, 1, 0, None, 0, torch.bfloat16),      # k = 1: own block only
    (1, 512, 2, 2, 128, 64, 8, 0, None, 0, torch.bfloat16),      # k = all blocks: dense causal
    (1, 300, 2, 1, 64, 32, 3, 0, None, 40, torch.bfloat16),      # extra local window
    (1, 160, 2, 2, 64, 1, 5, 0, None, 0, torch.bfloat16),        # block 1: token-level gating
    (1, 700, 4, 2, 128, 64, 3, 0, None, 0, torch.float32),       # fp32, d 128
    (1, 520, 2, 2, 64, 100, 16, 0, None, 0, torch.bfloat16),     # topk 16 > blocks, block not /64
    (1, 300, 4, 2, 128, 512, 3, 0, None, 0, torch.bfloat16),     # N below one block: no past block exists
    (2, 200, 2, 2, 64, 256, 4, 50, 150, 0, torch.bfloat16),      # the same with batch 2 and offset rows
    (1, 700, 6, 2, 128, 128, 3, 0, None, 0, torch.bfloat16),     # 3 query heads per KV head (no head packing)
    (1, 600, 8, 1, 64, 64, 3, 0, None, 0, torch.bfloat16),       # 8 query heads per KV head
    (1, 1000, 4, 2, 128, 128, 3, 991, 9, 0, torch.bfloat16),     # 9 final rows: just past the decode kernels
    (1, 4500, 2, 1, 128, 2048, 2, 0, None, 0, torch.bfloat16),   # block 2048, one past block per row
]


@pytest.mark.parametrize("case", SMALL, ids=[f"c{i}" for i in range(len(SMALL))])
def test_moba_small_shapes(case):
    b, n, hq, hkv, d, block, topk, qs, ql, w, dt = case
    print(f"[moba small] {case}", flush=True)
    q, k, v, _ = synth.moba_inputs(10 + n, b, n, hq, hkv, d, dt, DEV)
    check(q, k, v, block, topk, dt, q_start=qs, q_len=ql, window=w)


def test_moba_all_blocks_is_dense_causal_on_gpu():
    n, h, d = 512, 2, 128
    q, k, v, _ = synth.moba_inputs(3, 1, n, h, h, d, torch.bfloat16, DEV)
    _, blk, out, _ = run(q, k, v, 64, 8, torch.bfloat16)
    ref = torch.nn.functional.scaled_dot_product_attention(
        q.float().transpose(1, 2), k.float().transpose(1, 2), v.float().transpose(1, 2), is_causal=True,
        scale=1 / math.sqrt(d)).transpose(1, 2)
    assert_close(to64(out), to64(ref), BF16_TOL, "dense")


def sample_rows(n, block, count, seed):
    r = np.random.default_rng(seed)
    rows = set(r.integers(0, n, count).tolist())
    rows |= {0, 1, block - 1, block, 2 * block + 7, n - 1}
    return sorted(t for t in rows if t < n)


def test_moba_gqa_32k_planted_full_size():
    """MoBA prefill at the 8B-style GQA shape, bf16: 32 query / 8 KV heads, d
    128, N 32768, block 512, top-k 3 with the forced block, 8 planted key
    blocks; sampled rows checked against the oracle, whole run twice for
    determinism."""
    n, hq, hkv, d, block = 32768, 32, 8, 128, 512
    q, k, v, info = synth.moba_inputs(2, 1, n, hq, hkv, d, torch.bfloat16, DEV, planted=8, block=block)
    rows = sample_rows(n, block, 40, 2)
    print(f"[moba 32k] rows={len(rows)}", flush=True)
    blk, out, swaps = check(q, k, v, block, 3, torch.bfloat16, rows=rows)
    _, blk2, out2, _ = run(q, k, v, block, 3, torch.bfloat16)
    assert torch.equal(blk, blk2) and torch.equal(out, out2), "two runs differ"
    # planted blocks dominate the gating (sanity of the workload, not parity)
    counts = torch.bincount(blk[blk >= 0].flatten().long(), minlength=n // block).cpu()
    past = counts.clone()
    past -= torch.bincount(torch.arange(n) // block, minlength=n // block) * hq
    top8 = set(torch.topk(past.float(), 8).indices.tolist())
    assert len(top8 & set(info["planted_blocks"])) >= 6


def test_moba_gqa_32k_planted_topk4():
    """The same 32k GQA planted shape under the other reading of "top-k 3 +
    forced current block": three past blocks plus the current one (k = 4);
    sampled rows against the oracle."""
    n, hq, hkv, d, block = 32768, 32, 8, 128, 512
    q, k, v, _ = synth.moba_inputs(2, 1, n, hq, hkv, d, torch.bfloat16, DEV, planted=8, block=block)
    rows = sample_rows(n, block, 40, 4)
    print(f"[moba 32k k=4] rows={len(rows)}", flush=True)
    blk, _, _ = check(q, k, v, block, 4, torch.bfloat16, rows=rows)
    # every row past the third block attends three past blocks and its own
    assert int((blk[0, 3 * block:] >= 0).sum(-1).min()) == 4


def test_moba_long_512k_full_size():
    """MoBA fixed sparsity, bf16: 8 heads x 128, N 524288 in 64 blocks of 8192,
    top-k 3 (95.31% sparsity); block gating over all queries, attention for
    the final 8192-query chunk; sampled rows against the oracle."""
    n, h, d, block, topk = 524288, 8, 128, 8192, 3
    q, k, v, _ = synth.moba_inputs(5, 1, n, h, h, d, torch.bfloat16, DEV)
    p_sel = qat.moba_params(batch=1, seq_len=n, n_q_heads=h, n_kv_heads=h, head_dim=d, block=block, topk=topk)
    blk = qat.moba_block_select(p_sel, q, k)
    qs = n - block
    p_att = qat.moba_params(batch=1, seq_len=n, n_q_heads=h, n_kv_heads=h, head_dim=d, q_start=qs, q_len=block,
                            block=block, topk=topk)
    out, lse = qat.moba_sparse_attn(p_att, q, k, v, blk[:, qs:].contiguous())
    torch.cuda.synchronize()
    print("[moba 512k] gpu done", flush=True)
    kn = to64(k[0])
    kbar = omoba.block_means(kn, block)
    rows_sel = sample_rows(n, block, 40, 5)
    qn = q[0].to("cpu")
    qsel = {t: qn[t].to(torch.float64).numpy() for t in rows_sel}
    blk_ref = np.zeros((len(rows_sel), h, topk), dtype=np.int64)
    sc = np.zeros((len(rows_sel), h, n // block))
    for r, t in enumerate(rows_sel):
        for hh in range(h):
            blk_ref[r, hh], sc[r, hh] = omoba.select_row(qsel[t][hh], kbar[:, hh], t, block, topk)
    bad, _ = moba_rows_ok(blk[0, rows_sel].cpu().numpy(), blk_ref, sc, rows_sel, block, topk)
    assert not bad, bad[:5]
    # 3 of 64 blocks attended by every query of the final chunk
    assert int((blk[0, qs:] >= 0).sum(-1).min()) == topk
    rows_att = sorted({qs, qs + 1, qs + 4095, n - 1} | set(np.random.default_rng(6).integers(qs, n, 10).tolist()))
    vn = to64(v[0])
    blk_g = blk[0, rows_att].cpu().numpy()
    o_ref = np.zeros((len(rows_att), h, d))
    lse_ref = np.zeros((len(rows_att), h))
    for r, t in enumerate(rows_att):
        qt = qn[t].to(torch.float64).numpy()
        for hh in range(h):
            idx = omoba.key_set(blk_g[r, hh], t, block)
            o_ref[r, hh], lse_ref[r, hh] = oatt.attend(qt[hh], kn[idx, hh], vn[idx, hh], p_att.scale)
    rel = [t - qs for t in rows_att]
    assert_close(to64(out[0, rel]), o_ref, BF16_TOL, "output")
    assert_close(to64(lse[0, rel]), lse_ref, 1e-3, "lse")


def test_moba_many_buckets_global_dispatch():
    """More than 4096 (sequence, KV head, block) buckets (8 KV heads x 515
    blocks of 64): the dispatch counts and places entries through global
    atomics and the tile table searches the tile prefix in global memory;
    the block means exceed the LDS budget of the resident scoring kernel,
    so the streaming one runs. Sampled rows against the oracle."""
    n, hq, hkv, d, block = 33000, 8, 8, 64, 64
    q, k, v, _ = synth.moba_inputs(31, 1, n, hq, hkv, d, torch.bfloat16, DEV)
    rows = sample_rows(n, block, 48, 31)
    check(q, k, v, block, 3, torch.bfloat16, rows=rows)
