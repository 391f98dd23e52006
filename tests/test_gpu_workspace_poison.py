"""Results must not depend on what a caller's workspace held before the call:
every entry point that takes a workspace runs twice on the same inputs, once
with the workspace zeroed and once filled with 0xFF bytes (NaN as bf16 and
float32), and the outputs must be bit-identical (and finite). A kernel that
reads a workspace region it never wrote (a partial of a block that was not
gated, a slot past a row's selection) fails here."""
import pytest
import torch

import query_aware_top_amd as qat
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _two_workspaces(nbytes):
    return (torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=DEV),
            torch.full((max(nbytes, 1),), 0xFF, dtype=torch.uint8, device=DEV))


def _same(a, b, what):
    torch.cuda.synchronize()
    assert torch.isfinite(a.float()).all(), f"{what}: non-finite values"
    assert torch.equal(a, b), f"{what}: depends on the workspace's prior contents"


@pytest.mark.parametrize("case", [
    # n, hq, hkv, d, block, topk: the smoke shape (all rows of the first block
    # without past partials), a ragged N, k = 4, d = 64, MHA, N below one
    # block (no past block exists, so no past-block pass runs)
    (1024, 4, 2, 128, 128, 3), (1000, 4, 2, 128, 128, 3), (1024, 4, 2, 128, 128, 4),
    (1024, 4, 2, 64, 128, 3), (2048, 4, 4, 128, 256, 3), (300, 4, 2, 128, 512, 3)])
def test_moba_prefill_ignores_stale_workspace(case):
    n, hq, hkv, d, block, topk = case
    print(f"[poison moba] {case}", flush=True)
    q, k, v, _ = synth.moba_inputs(31, 1, n, hq, hkv, d, torch.bfloat16, DEV)
    p = qat.moba_params(batch=1, seq_len=n, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, block=block, topk=topk)
    res = []
    for ws in _two_workspaces(qat.moba_workspace_size(p)):
        blk = qat.moba_block_select(p, q, k, ws=ws)
        out, lse = qat.moba_sparse_attn(p, q, k, v, blk, ws=ws)
        res.append((blk, out, lse))
    _same(res[0][0], res[1][0], "blk")
    _same(res[0][1], res[1][1], "out")
    _same(res[0][2], res[1][2], "lse")


def test_moba_decode_and_gradients_ignore_stale_workspace():
    n, hq, hkv, d, block, topk = 1024, 4, 2, 128, 128, 3
    q, k, v, _ = synth.moba_inputs(32, 1, n, hq, hkv, d, torch.bfloat16, DEV)
    pd = qat.moba_params(batch=1, seq_len=n, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, q_start=n - 1, q_len=1,
                         block=block, topk=topk)
    qr = q[:, n - 1:].contiguous()
    kbars, outs = [], []
    for ws in _two_workspaces(qat.moba_workspace_size(pd)):
        kbar = qat.moba_block_means(pd, k, 0, n // block, ws=ws)
        blk = qat.moba_decode_select(pd, qr, kbar)
        out, _ = qat.moba_decode_attn(pd, qr, k, v, blk, ws=ws)
        kbars.append(kbar)
        outs.append(out)
    _same(kbars[0], kbars[1], "decode kbar")
    _same(outs[0], outs[1], "decode out")
    p = qat.moba_params(batch=1, seq_len=n, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, block=block, topk=topk)
    blk = qat.moba_block_select(p, q, k)
    out, lse = qat.moba_sparse_attn(p, q, k, v, blk)
    do = synth.normal(33, 9, tuple(out.shape), torch.bfloat16, DEV)
    grads = []
    for ws in _two_workspaces(qat.moba_bwd_workspace_size(p)):
        grads.append(qat.moba_sparse_attn_bwd(p, q, k, v, blk, do, lse, ws=ws))
    for a, b, name in zip(grads[0], grads[1], ("dq", "dk", "dv")):
        _same(a, b, f"moba {name}")


@pytest.mark.parametrize("m", [256, 1])
def test_esa_select_attend_and_gradients_ignore_stale_workspace(m):
    T, H, d, d_c = 2048, 4, 64, 64
    c0 = T - m
    _, k, v, _ = synth.esa_inputs(34, 1, T, 1, H, d, torch.bfloat16, DEV)
    q = synth.normal(34, synth.gen.TID_Q, (1, m, H, d), torch.bfloat16, DEV, start=1 << 40)
    W = synth.compression_weights(34, d_c, H * d, device=DEV)
    kc = qat.esa_compress(k.view(T, H * d), W).view(1, T, d_c)
    pe = qat.esa_params(batch=1, n_heads=H, head_dim=d, d_c=d_c, ctx_len=T, chunk_start=c0, chunk_len=m,
                        n_init=16, window=256, topk=128, radius=2, clip=12.0)
    res = []
    for ws in _two_workspaces(qat.esa_workspace_size(pe)):
        sel, n_sel, _ = qat.esa_select(pe, q, W, None, kc, ws=ws)
        out, lse = qat.esa_sparse_attn(pe, q, k, v, sel, n_sel, ws=ws)
        res.append((sel, n_sel, out, lse))
    _same(res[0][1], res[1][1], "n_sel")
    _same(res[0][0], res[1][0], "sel")
    _same(res[0][2], res[1][2], "esa out")
    _same(res[0][3], res[1][3], "esa lse")
    sel, n_sel, out, lse = res[0]
    do = synth.normal(35, 9, tuple(out.shape), torch.bfloat16, DEV)
    grads = []
    for ws in _two_workspaces(qat.esa_bwd_workspace_size(pe)):
        grads.append(qat.esa_sparse_attn_bwd(pe, q, k, v, sel, n_sel, do, lse, ws=ws))
    for a, b, name in zip(grads[0], grads[1], ("dq", "dk", "dv")):
        _same(a, b, f"esa {name}")
