"""GPU parity of the MoBA gradients (moba_sparse_attn_bwd through the C ABI)
against the float64 oracle (oracle.moba.backward_rows) on the GPU's own
selection, plus whole-tensor identities that hold at any size: every row's
probabilities sum to 1, so the dv rows of a KV head sum to the dO rows of its
query heads, and its ds sum to 0, so the dk rows of a KV head sum to 0."""
import numpy as np
import pytest
import torch

import query_aware_top_amd as qat
import synth
from oracle import moba as omoba
from parity import assert_close, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def forward_backward(q, k, v, block, topk, dtype, q_start=0, q_len=None, seed=0):
    p = qat.moba_params(batch=q.shape[0], seq_len=q.shape[1], n_q_heads=q.shape[2], n_kv_heads=k.shape[2],
                        head_dim=q.shape[3], q_start=q_start, q_len=q_len, block=block, topk=topk, dtype=dtype)
    blk = qat.moba_block_select(p, q, k)
    out, lse = qat.moba_sparse_attn(p, q, k, v, blk)
    do = synth.normal(seed, 7, (p.batch, p.q_len, p.n_q_heads, p.head_dim), dtype, DEV)
    dq, dk, dv = qat.moba_sparse_attn_bwd(p, q, k, v, blk, do, lse)
    torch.cuda.synchronize()
    return p, blk, do, dq, dk, dv


def check_identities(p, do, dk, dv):
    """sum over keys of dv[b, :, g] = sum of dO over the rows of g's query
    heads; sum over keys of dk[b, :, g] = 0 (float32 sums on the host)."""
    G = p.n_q_heads // p.n_kv_heads
    do64 = to64(do).reshape(p.batch, p.q_len, p.n_kv_heads, G, p.head_dim).sum(axis=(1, 3))
    dv_sum = to64(dv).sum(axis=1)
    dk_sum = to64(dk).sum(axis=1)
    scale_v = np.abs(to64(dv)).sum(axis=1) + 1e-30
    scale_k = np.abs(to64(dk)).sum(axis=1) + 1e-30
    assert np.all(np.abs(dv_sum - do64) <= 1e-4 * scale_v + 1e-4), np.abs(dv_sum - do64).max()
    assert np.all(np.abs(dk_sum) <= 1e-4 * scale_k + 1e-5), np.abs(dk_sum).max()


SMALL = [
    # batch, N, hq, hkv, d, block, topk, q_start, q_len, dtype
    (1, 1000, 4, 2, 128, 128, 3, 0, None, torch.bfloat16),     # ragged N, GQA, several tiles
    (2, 777, 2, 2, 64, 64, 4, 100, 500, torch.bfloat16),       # batch 2, offset rows, d 64
    (1, 600, 4, 1, 128, 64, 1, 0, None, torch.bfloat16),       # k = 1: own block only
    (1, 512, 2, 2, 128, 64, 8, 0, None, torch.bfloat16),       # k = all blocks: dense causal
    (1, 700, 4, 2, 128, 64, 3, 0, None, torch.float32),        # float32
    (1, 520, 2, 2, 64, 100, 16, 0, None, torch.bfloat16),      # block not a multiple of 64, k = 16
    (1, 300, 2, 1, 64, 1, 5, 0, None, torch.bfloat16),         # block 1: token-level gating
    (1, 3000, 8, 2, 128, 256, 3, 2990, 10, torch.bfloat16),    # a few rows at the end (decode-like)
    (1, 300, 4, 2, 128, 512, 3, 0, None, torch.bfloat16),      # N below one block: no past block exists
    (1, 700, 6, 2, 128, 128, 3, 0, None, torch.bfloat16),      # 3 query heads per KV head
]


@pytest.mark.parametrize("case", SMALL, ids=[f"b{i}" for i in range(len(SMALL))])
def test_moba_bwd_small_shapes(case):
    b, n, hq, hkv, d, block, topk, qs, ql, dt = case
    print(f"[moba bwd] {case}", flush=True)
    q, k, v, _ = synth.moba_inputs(60 + n, b, n, hq, hkv, d, dt, DEV)
    p, blk, do, dq, dk, dv = forward_backward(q, k, v, block, topk, dt, qs, ql, seed=61 + n)
    tol = 2e-3 if dt == torch.bfloat16 else 1e-4
    rows = list(range(p.q_start, p.q_start + p.q_len))
    for bi in range(b):
        dq_r, dk_r, dv_r = omoba.backward_rows(to64(q[bi]), to64(k[bi]), to64(v[bi]), block,
                                               blk[bi].cpu().numpy(), rows, p.scale, to64(do[bi]))
        assert_close(to64(dq[bi]), dq_r, tol, "dq")
        assert_close(to64(dk[bi]), dk_r, tol, "dk")
        assert_close(to64(dv[bi]), dv_r, tol, "dv")
    check_identities(p, do, dk, dv)


def test_moba_bwd_gqa_32k_full_size():
    """The 32k GQA prefill shape (32 query / 8 KV heads x 128, block 512,
    top-k 3, 8 planted blocks): dq on sampled rows; dk, dv of the last block
    (its own rows only) and of the earlier block with the fewest gating rows
    (all rows that attend it) against the oracle; the two identities over the
    whole tensors."""
    n, hq, hkv, d, block, topk = 32768, 32, 8, 128, 512, 3
    q, k, v, _ = synth.moba_inputs(2, 1, n, hq, hkv, d, torch.bfloat16, DEV, planted=8, block=block)
    p, blk, do, dq, dk, dv = forward_backward(q, k, v, block, topk, torch.bfloat16, seed=62)
    print("[moba bwd 32k] gpu done", flush=True)
    # reproducible: a second call gives the same bits (the dispatch places a
    # bucket's rows in row order for the gradient pass)
    out, lse = qat.moba_sparse_attn(p, q, k, v, blk)
    dq2, dk2, dv2 = qat.moba_sparse_attn_bwd(p, q, k, v, blk, do, lse)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2), "gradients differ between calls"
    check_identities(p, do, dk, dv)
    qn, kn, vn = to64(q[0]), to64(k[0]), to64(v[0])
    blk_g = blk[0].cpu().numpy()
    do_n = to64(do[0])
    rows = [0, 1, 511, 512, 4000, 20000, n - 1]
    dq_r, _, _ = omoba.backward_rows(qn, kn, vn, block, blk_g[rows], rows, p.scale, do_n[rows])
    assert_close(to64(dq[0, rows]), dq_r, 2e-3, "dq")
    nb = n // block
    # rows that attend block b: its own rows, and the rows that gated it
    gated = [(blk_g[:, :, :topk - 1] == b).any(axis=2).any(axis=1).sum() for b in range(nb)]
    b_mid = min(range(nb // 2, nb - 1), key=lambda b: gated[b])
    for b in (nb - 1, b_mid):
        attend = np.nonzero((blk_g[:, :, :topk - 1] == b).any(axis=2).any(axis=1))[0].tolist()
        rws = sorted(set(attend) | set(range(b * block, (b + 1) * block)))
        print(f"[moba bwd 32k] block {b}: {len(rws)} rows", flush=True)
        _, dk_r, dv_r = omoba.backward_rows(qn, kn, vn, block, blk_g[rws], rws, p.scale, do_n[rws])
        sl = slice(b * block, (b + 1) * block)
        assert_close(to64(dk[0, sl]), dk_r[sl], 2e-3, f"dk block {b}")
        assert_close(to64(dv[0, sl]), dv_r[sl], 2e-3, f"dv block {b}")
