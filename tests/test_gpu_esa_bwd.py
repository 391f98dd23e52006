"""GPU parity of the ESA gradients (esa_sparse_attn_bwd through the C ABI)
against the float64 oracle (oracle.esa.backward) on the GPU's own
selection, plus whole-tensor identities that hold at any size (per head: the
dv rows sum to the dO rows, the dk rows to 0)."""
import numpy as np
import pytest
import torch

import query_aware_top_amd as qat
import synth
from oracle import esa as oesa
from parity import assert_close, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_case(seed, B, T, c0, m, H, d, d_c, n_init, W, topk, radius, clip):
    _, k, v, _ = synth.esa_inputs(seed, B, T, 1, H, d, torch.bfloat16, DEV)
    q = synth.normal(seed, synth.gen.TID_Q, (B, m, H, d), torch.bfloat16, DEV, start=1 << 40)
    Wq = synth.compression_weights(seed, d_c, H * d, synth.gen.TID_W, torch.bfloat16, DEV)
    p = qat.esa_params(batch=B, n_heads=H, head_dim=d, d_c=d_c, ctx_len=T, chunk_start=c0, chunk_len=m,
                       n_init=n_init, window=W, topk=topk, radius=radius, clip=clip)
    kc = qat.esa_compress(k.view(B * T, H * d), Wq, out_dtype=torch.bfloat16).view(B, T, -1)
    sel, n_sel, _ = qat.esa_select(p, q, Wq, None, kc)
    _, lse = qat.esa_sparse_attn(p, q, k, v, sel, n_sel)
    do = synth.normal(seed, 7, (B, m, H, d), torch.bfloat16, DEV)
    dq, dk, dv = qat.esa_sparse_attn_bwd(p, q, k, v, sel, n_sel, do, lse)
    torch.cuda.synchronize()
    return p, q, k, v, sel, n_sel, do, dq, dk, dv


def check_identities(do, dk, dv):
    """Per sequence and head: sum over positions of dv = sum over queries of
    dO; sum over positions of dk = 0."""
    dv_sum = to64(dv).sum(axis=1)
    do_sum = to64(do).sum(axis=1)
    dk_sum = to64(dk).sum(axis=1)
    scale_v = np.abs(to64(dv)).sum(axis=1) + 1e-30
    scale_k = np.abs(to64(dk)).sum(axis=1) + 1e-30
    assert np.all(np.abs(dv_sum - do_sum) <= 1e-4 * scale_v + 1e-4), np.abs(dv_sum - do_sum).max()
    assert np.all(np.abs(dk_sum) <= 1e-4 * scale_k + 1e-5), np.abs(dk_sum).max()


SMALL = [
    # seed, B, T, c0, m, H, d, d_c, n_init, W, topk, radius, clip
    (71, 1, 2048, 1600, 300, 4, 128, 64, 16, 128, 100, 2, 12.0),   # several query and key tiles
    (72, 2, 1500, 1000, 257, 2, 64, 32, 8, 64, 50, 1, 6.0),        # batch 2, ragged chunk, d 64
    (73, 1, 300, 20, 100, 2, 64, 64, 32, 16, 10, 2, 4.0),          # chunk inside the initial part: M empty
    (74, 3, 3000, 2999, 1, 4, 128, 64, 32, 256, 300, 2, 24.0),     # decode: one query per sequence
    (75, 1, 600, 400, 130, 2, 64, 128, 16, 32, 1000, 2, 5.0),      # k >= |M|: dense causal
    (76, 1, 300, 0, 300, 2, 64, 64, 16, 32, 10, 1, 4.0),           # chunk at position 0: causal chunk keys only
    (77, 1, 1500, 1000, 200, 2, 64, 64, 0, 0, 100, 1, 6.0),        # no initial tokens, no window
]


@pytest.mark.parametrize("case", SMALL, ids=[f"e{i}" for i in range(len(SMALL))])
def test_esa_bwd_small(case):
    seed, B, T, c0, m, H, d, d_c, n_init, W, topk, radius, clip = case
    print(f"[esa bwd] {case}", flush=True)
    p, q, k, v, sel, n_sel, do, dq, dk, dv = run_case(*case)
    for bi in range(B):
        sg = sel[bi, :int(n_sel[bi])].cpu().numpy().astype(np.int64)
        dq_r, dk_r, dv_r = oesa.backward(to64(q[bi]), to64(k[bi]), to64(v[bi]), sg, c0, n_init, W, p.scale,
                                         to64(do[bi]))
        assert_close(to64(dq[bi]), dq_r, 2e-3, "dq")
        assert_close(to64(dk[bi]), dk_r, 2e-3, "dk")
        assert_close(to64(dv[bi]), dv_r, 2e-3, "dv")
    check_identities(do, dk, dv)


def test_esa_bwd_accumulates_over_calls():
    """dk, dv are added to: two calls give twice one call's gradients."""
    case = SMALL[1]
    p, q, k, v, sel, n_sel, do, dq, dk, dv = run_case(*case)
    _, lse = qat.esa_sparse_attn(p, q, k, v, sel, n_sel)
    dq2, dk2, dv2 = qat.esa_sparse_attn_bwd(p, q, k, v, sel, n_sel, do, lse, dk=dk.clone(), dv=dv.clone())
    torch.cuda.synchronize()
    assert torch.equal(dq2, dq)
    assert torch.allclose(dk2, 2 * dk, rtol=1e-6, atol=1e-7) and torch.allclose(dv2, 2 * dv, rtol=1e-6, atol=1e-7)


class _Rows:
    """Row view of a large GPU tensor for the oracle: x[idx] copies only the
    requested rows to the host as float64."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, idx):
        if isinstance(idx, tuple):
            rows, rest = idx[0], idx[1:]
            ix = torch.as_tensor(np.asarray(rows), device=self.t.device, dtype=torch.long)
            return to64(self.t.index_select(0, ix)[(slice(None),) + rest])
        ix = torch.as_tensor(np.asarray(idx), device=self.t.device, dtype=torch.long)
        return to64(self.t.index_select(0, ix))


def test_esa_bwd_prefill_64k_full_size():
    """The 64k chunked prefill shape (32 heads x 128, chunk 2048, 128 + 2048 +
    4096 gathered keys): dq of sampled queries (all heads), dk and dv of head
    0 at every position, and the identities over the whole tensors."""
    case = (3, 1, 65536, 63488, 2048, 32, 128, 128, 128, 4096, 2048, 2, 48.0)
    p, q, k, v, sel, n_sel, do, dq, dk, dv = run_case(*case)
    print("[esa bwd 64k] gpu done", flush=True)
    check_identities(do, dk, dv)
    c0, n_init, W = 63488, 128, 4096
    sg = sel[0, :int(n_sel[0])].cpu().numpy().astype(np.int64)
    qn, don = to64(q[0]), to64(do[0])
    K, V = _Rows(k[0]), _Rows(v[0])
    rows = [0, 1, 1000, 2047]
    dq_r, _, _ = oesa.backward(qn, K, V, sg, c0, n_init, W, p.scale, don[rows], rows=rows)
    assert_close(to64(dq[0, rows]), dq_r, 2e-3, "dq")
    # head 0, every query: its dk, dv over all positions
    idx = oesa.key_list(sg, c0, n_init, W, c0 + 2047)
    k0 = np.zeros((65536, 1, 128))
    v0 = np.zeros((65536, 1, 128))
    k0[idx, 0] = to64(k[0, torch.as_tensor(idx, device=DEV), 0])
    v0[idx, 0] = to64(v[0, torch.as_tensor(idx, device=DEV), 0])
    _, dk_r, dv_r = oesa.backward(qn[:, :1], k0, v0, sg, c0, n_init, W, p.scale, don[:, :1])
    print("[esa bwd 64k] oracle done", flush=True)
    assert_close(to64(dk[0, idx, 0]), dk_r[idx, 0], 2e-3, "dk head 0")
    assert_close(to64(dv[0, idx, 0]), dv_r[idx, 0], 2e-3, "dv head 0")
