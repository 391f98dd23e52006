"""The entry point that allocates nothing (moba_decode_attn_noalloc, for
callers that cannot allocate device memory) against moba_decode_attn, which
takes a caller workspace, through the C ABI: two calls in a row, the second
with a smaller input, each bit-identical to the workspace entry point's
result on the same inputs (the same kernels run; only where their partials
live differs)."""
import pytest
import torch

import query_aware_top_amd as qat
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(seed, batch, n, hq, hkv, d, block, topk, q_len):
    q, k, v, _ = synth.moba_inputs(seed, batch, n, hq, hkv, d, torch.bfloat16, DEV, planted=2, block=block)
    p = qat.moba_params(batch=batch, seq_len=n, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, q_start=n - q_len,
                        q_len=q_len, block=block, topk=topk)
    kbar = qat.moba_block_means(p, k, 0, n // block)
    qr = q[:, n - q_len:].contiguous()
    blk = qat.moba_decode_select(p, qr, kbar)
    return p, qr, k, v, blk


def _compare(p, qr, k, v, blk):
    ref, ref_lse = qat.moba_decode_attn(p, qr, k, v, blk)
    out = torch.full_like(ref, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    qat.moba_decode_attn_noalloc(p, qr, k, v, blk, out, lse)
    torch.cuda.synchronize()
    assert torch.equal(out, ref), f"output differs: max {(out.float() - ref.float()).abs().max().item()}"
    assert torch.equal(lse, ref_lse), "lse differs"


def test_noalloc_decode_matches_workspace_entry_twice_second_smaller():
    # first call: 8 sequences x 2 new rows, 16 query / 4 KV heads, d 128, block 512, k 3
    print("[noalloc] call 1: batch 8, 2 rows, 16/4 heads x 128, 16384 keys", flush=True)
    big = _case(71, 8, 16384, 16, 4, 128, 512, 3, 2)
    _compare(*big)
    # second call, smaller: 2 sequences x 1 row, 4 / 2 heads x 64, block 256, k 4 (stale
    # partials of the first call are left in the shared array)
    print("[noalloc] call 2: batch 2, 1 row, 4/2 heads x 64, 3000 keys", flush=True)
    small = _case(72, 2, 3000, 4, 2, 64, 256, 4, 1)
    _compare(*small)


def test_noalloc_rejects_what_does_not_fit():
    """Cases outside the split-key path, or past the fixed array's size, are
    refused before any device work."""
    p = qat.moba_params(batch=1, seq_len=4096, n_q_heads=4, n_kv_heads=2, head_dim=64, q_start=0, q_len=4096,
                        block=256, topk=3)
    x = torch.zeros(1, 4096, 4, 64, dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros(1, 4096, 2, 64, dtype=torch.bfloat16, device=DEV)
    blk = torch.zeros(1, 4096, 4, 3, dtype=torch.int32, device=DEV)
    with pytest.raises(qat.QatError, match="split-key"):
        qat.moba_decode_attn_noalloc(p, x, kv, kv, blk, torch.empty_like(x))
    # 64 sequences x 8 rows x 32 heads, 6 pieces each: ~51 MB of partials, past the 16 MiB array
    p = qat.moba_params(batch=64, seq_len=1024, n_q_heads=32, n_kv_heads=8, head_dim=128, q_start=1016, q_len=8,
                        block=512, topk=3)
    q = torch.zeros(64, 8, 32, 128, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(64, 1024, 8, 128, dtype=torch.bfloat16, device=DEV)
    blk = torch.zeros(64, 8, 32, 3, dtype=torch.int32, device=DEV)
    with pytest.raises(qat.QatError, match="scratch"):
        qat.moba_decode_attn_noalloc(p, q, k, k, blk, torch.empty_like(q))
