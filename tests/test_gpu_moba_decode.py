"""GPU parity of the MoBA decode-step entry points (moba_block_means,
moba_decode_select, moba_decode_attn through the C ABI) against the float64
CPU oracle: a kept cache of complete-block means, gating of the newest
query rows against it, and split-key attention over the gated blocks plus
the partial current block."""
import numpy as np
import pytest
import torch

import query_aware_top_amd as qat
import synth
from oracle import attention as oatt
from oracle import moba as omoba
from parity import BF16_TOL, F32_TOL, assert_close, moba_rows_ok, to64
from query_aware_top_amd._binding import QAT_BF16

pytestmark = pytest.mark.gpu
DEV = "cuda"


def params(batch, n, hq, hkv, d, block, topk, q_len, dtype, window=0):
    return qat.moba_params(batch=batch, seq_len=n, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, q_start=n - q_len,
                           q_len=q_len, block=block, topk=topk, window=window, dtype=dtype)


def fill_cache(p, k, splits=2):
    """Means of every complete block, written in `splits` incremental calls."""
    nbc = p.seq_len // p.block
    kbar = torch.full((p.batch, nbc, p.n_kv_heads, p.head_dim), float("nan"), dtype=torch.float32, device=DEV)
    cuts = sorted({0, nbc} | {nbc * i // splits for i in range(1, splits)})
    for a, b in zip(cuts, cuts[1:]):
        qat.moba_block_means(p, k, a, b - a, kbar)
    return kbar


def check_cache(kbar, k, block, batches):
    for bi in batches:
        ref = omoba.block_means(to64(k[bi]), block)[: kbar.shape[1]]
        got = to64(kbar[bi])
        # float64 accumulation rounded once to float32: within one float32 ulp
        lim = np.abs(ref) * 2.0 ** -23 + 1e-30
        assert np.all(np.abs(got - ref) <= lim), f"block means: max err {np.abs(got - ref).max():.3e}"


def check_rows(p, q, k, v, kbar, blk, out, lse, batches, heads=None, window=0):
    """Selection (tie band) and output of the rows of `batches` against the oracle."""
    rows = list(range(p.q_start, p.q_start + p.q_len))
    tol = BF16_TOL if p.dtype == QAT_BF16 else F32_TOL
    lse_tol = 1e-3 if p.dtype == QAT_BF16 else 1e-5
    hq = p.n_q_heads
    heads = list(range(hq)) if heads is None else heads
    swaps = 0
    for bi in batches:
        kn, vn = to64(k[bi]), to64(v[bi])
        kb = omoba.block_means(kn, p.block)
        qn = to64(q[bi])   # [q_len, hq, d]
        blk_ref = np.zeros((len(rows), len(heads), p.topk), dtype=np.int64)
        sc = np.zeros((len(rows), len(heads), kb.shape[0]))
        for r, t in enumerate(rows):
            for j, h in enumerate(heads):
                blk_ref[r, j], sc[r, j] = omoba.select_row(qn[r, h], kb[:, omoba.kv_head(h, hq, p.n_kv_heads)],
                                                           t, p.block, p.topk)
        blk_g = blk[bi][:, heads].cpu().numpy()
        bad, n = moba_rows_ok(blk_g, blk_ref, sc, rows, p.block, p.topk)
        assert not bad, f"selection mismatch outside the tie band: {bad[:5]}"
        swaps += n
        o_ref = np.zeros((len(rows), len(heads), p.head_dim))
        lse_ref = np.zeros((len(rows), len(heads)))
        for r, t in enumerate(rows):
            for j, h in enumerate(heads):
                g = omoba.kv_head(h, hq, p.n_kv_heads)
                idx = omoba.key_set(blk_g[r, j], t, p.block, window)
                o_ref[r, j], lse_ref[r, j] = oatt.attend(qn[r, h], kn[idx, g], vn[idx, g], p.scale)
        assert_close(to64(out[bi][:, heads]), o_ref, tol, "output")
        assert_close(to64(lse[bi][:, heads]), lse_ref, lse_tol, "lse")
    return swaps


DECODE = [
    # batch, N, hq, hkv, d, block, topk, q_len, dtype
    (2, 5000, 8, 2, 128, 256, 3, 1, torch.bfloat16),     # ragged N: partial current block, GQA 4:1
    (1, 4097, 4, 4, 64, 256, 4, 1, torch.bfloat16),      # current block holds one key
    (3, 2048, 4, 1, 128, 512, 2, 1, torch.bfloat16),     # N on a block boundary; top-k 2
    (1, 3000, 4, 2, 128, 100, 16, 4, torch.bfloat16),    # 4 rows, block not /64, top-k 16 (15 past)
    (2, 1412, 4, 2, 64, 128, 3, 8, torch.float32),       # float32, 8 rows over a block boundary
    (1, 700, 2, 1, 128, 1000, 3, 1, torch.bfloat16),     # no complete block: own block only
    (1, 9000, 2, 2, 128, 1024, 5, 2, torch.bfloat16),    # 4 pieces per block
    (2, 3333, 24, 2, 128, 128, 4, 3, torch.bfloat16),    # 12 query heads per KV head: three rounds of four
    (1, 2600, 6, 1, 64, 256, 3, 1, torch.float32),       # 6 heads per KV head: a partial round of four
]


@pytest.mark.parametrize("case", DECODE, ids=[f"d{i}" for i in range(len(DECODE))])
def test_moba_decode_small(case):
    b, n, hq, hkv, d, block, topk, ql, dt = case
    print(f"[moba decode] {case}", flush=True)
    q, k, v, _ = synth.moba_decode_inputs(40 + n, b, n, ql, hq, hkv, d, dt, DEV)
    p = params(b, n, hq, hkv, d, block, topk, ql, dt)
    kbar = fill_cache(p, k)
    blk = qat.moba_decode_select(p, q, kbar)
    out, lse = qat.moba_decode_attn(p, q, k, v, blk)
    torch.cuda.synchronize()
    check_cache(kbar, k, block, range(b))
    check_rows(p, q, k, v, kbar, blk, out, lse, range(b))


def test_moba_decode_matches_full_layout_entry_points():
    """The decode entry points on the newest rows give what moba_block_select
    and moba_sparse_attn give for the same rows of a whole-sequence q: the
    same selection up to float32 near-ties, and bit-identical attention for
    the same selection."""
    b, n, hq, hkv, d, block, topk, ql = 2, 6000, 8, 2, 128, 512, 3, 3
    q, k, v, _ = synth.moba_inputs(77, b, n, hq, hkv, d, torch.bfloat16, DEV)
    p = params(b, n, hq, hkv, d, block, topk, ql, torch.bfloat16)
    qr = q[:, n - ql:].contiguous()
    kbar = fill_cache(p, k, splits=3)
    blk_d = qat.moba_decode_select(p, qr, kbar)
    blk_f = qat.moba_block_select(p, q, k)
    out_d, lse_d = qat.moba_decode_attn(p, qr, k, v, blk_f)
    out_f, lse_f = qat.moba_sparse_attn(p, q, k, v, blk_f)
    torch.cuda.synchronize()
    assert torch.equal(out_d, out_f) and torch.equal(lse_d, lse_f)
    check_rows(p, qr, k, v, kbar, blk_d, *qat.moba_decode_attn(p, qr, k, v, blk_d), range(b))
    assert (blk_d != blk_f).float().mean().item() < 0.05


def test_planned_calls_match_direct_calls():
    """qat.plan re-issues the marshalled C ABI calls: a planned decode step
    (cache update, gating, attention) gives bit-identical results to the
    direct calls, on repeated replays."""
    b, n, hq, hkv, d, block, topk = 3, 5000, 8, 2, 128, 256, 3
    q, k, v, _ = synth.moba_inputs(78, b, n, hq, hkv, d, torch.bfloat16, DEV)
    p = params(b, n, hq, hkv, d, block, topk, 1, torch.bfloat16)
    qr = q[:, n - 1:].contiguous()
    ws = torch.empty(qat.moba_workspace_size(p), dtype=torch.uint8, device=DEV)
    last = (n - 1) // block - 1
    kbar = qat.moba_block_means(p, k, 0, last, ws=ws)
    blk = torch.empty(b, 1, hq, topk, dtype=torch.int32, device=DEV)
    out = torch.empty(b, 1, hq, d, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(b, 1, hq, dtype=torch.float32, device=DEV)
    steps = [qat.plan(qat.moba_block_means, p, k, last, 1, kbar, ws=ws),
             qat.plan(qat.moba_decode_select, p, qr, kbar, blk=blk),
             qat.plan(qat.moba_decode_attn, p, qr, k, v, blk, out=out, lse=lse, ws=ws)]
    assert [s.calls for s in steps] == [["moba_block_means"], ["moba_decode_select"], ["moba_decode_attn"]]
    qat.moba_block_means(p, k, last, 1, kbar, ws=ws)
    blk_d = qat.moba_decode_select(p, qr, kbar)
    out_d, lse_d = qat.moba_decode_attn(p, qr, k, v, blk_d)
    for _ in range(3):
        out.zero_()
        for s in steps:
            s()
        torch.cuda.synchronize()
        assert torch.equal(blk, blk_d) and torch.equal(out, out_d) and torch.equal(lse, lse_d)


def test_moba_decode_window_and_generic_layout():
    """An extra local window takes the per-row kernel with the rows-only q."""
    b, n, hq, hkv, d, block, topk, ql, w = 1, 2500, 4, 2, 64, 128, 3, 2, 300
    q, k, v, _ = synth.moba_decode_inputs(91, b, n, ql, hq, hkv, d, torch.bfloat16, DEV)
    p = params(b, n, hq, hkv, d, block, topk, ql, torch.bfloat16, window=w)
    kbar = fill_cache(p, k)
    blk = qat.moba_decode_select(p, q, kbar)
    out, lse = qat.moba_decode_attn(p, q, k, v, blk)
    torch.cuda.synchronize()
    check_rows(p, q, k, v, kbar, blk, out, lse, range(b), window=w)


def test_moba_decode_incremental_cache_over_steps():
    """Token-by-token decode across a block boundary: the cache gains one
    block when the previous one completes; every step matches the oracle."""
    b, hq, hkv, d, block, topk = 1, 4, 2, 128, 64, 3
    n_total = 8 * block + 3
    q_all, k, v, _ = synth.moba_inputs(12, b, n_total, hq, hkv, d, torch.bfloat16, DEV)
    nbc_max = n_total // block
    kbar = torch.full((b, nbc_max, hkv, d), float("nan"), dtype=torch.float32, device=DEV)
    done = 0
    for n in range(7 * block - 2, n_total + 1):
        p_cache = params(b, n_total, hq, hkv, d, block, topk, 1, torch.bfloat16)
        if n // block > done:   # blocks completed since the last step
            qat.moba_block_means(p_cache, k, done, n // block - done, kbar)
            done = n // block
        # the step sees a cache of capacity n_total holding n tokens: rows at n - 1
        p = qat.moba_params(batch=b, seq_len=n_total, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, q_start=n - 1,
                            q_len=1, block=block, topk=topk, dtype=torch.bfloat16)
        qr = q_all[:, n - 1:n].contiguous()
        blk = qat.moba_decode_select(p, qr, kbar)
        out, lse = qat.moba_decode_attn(p, qr, k, v, blk)
        torch.cuda.synchronize()
        check_rows(p, qr, k, v, kbar, blk, out, lse, [0])


def test_moba_decode_128k_full_size():
    """The decode step at its full shape, bf16: 16 sequences of 131072 cached
    tokens, 32 query / 8 KV heads, d 128, block 512, top-k 3 (two gated
    blocks plus the partial current one), 8 planted blocks; the cache built
    in one call, selection and output checked on sampled sequences and
    heads, two runs bit-identical."""
    b, n, hq, hkv, d, block, topk = 16, 131072, 32, 8, 128, 512, 3
    q, k, v, info = synth.moba_decode_inputs(128, b, n, 1, hq, hkv, d, torch.bfloat16, DEV, planted=8, block=block)
    p = params(b, n, hq, hkv, d, block, topk, 1, torch.bfloat16)
    kbar = qat.moba_block_means(p, k, 0, n // block)
    blk = qat.moba_decode_select(p, q, kbar)
    out, lse = qat.moba_decode_attn(p, q, k, v, blk)
    blk2 = qat.moba_decode_select(p, q, kbar)
    out2, lse2 = qat.moba_decode_attn(p, q, k, v, blk2)
    torch.cuda.synchronize()
    print("[moba decode 128k] gpu done", flush=True)
    assert torch.equal(blk, blk2) and torch.equal(out, out2) and torch.equal(lse, lse2)
    # every row: two gated past blocks then the own block
    assert bool((blk[..., :2] >= 0).all()) and bool((blk[..., 2] == (n - 1) // block).all())
    check_cache(kbar, k, block, [0])
    swaps = check_rows(p, q, k, v, kbar, blk, out, lse, [0, 15], heads=[0, 1, 5, 13, 31])
    print(f"[moba decode 128k] near-tie swaps {swaps}", flush=True)
