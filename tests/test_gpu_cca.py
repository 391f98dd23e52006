"""GPU parity of the CCA-style core-token attention (cca_pool + cca_attn
through the C ABI) against the float64 oracle (oracle.cca)."""
import numpy as np
import pytest
import torch

import query_aware_top_amd as qat
import synth
from oracle import cca as occa
from parity import BF16_TOL, assert_close, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run(q, k, v, group, window, q_start=0, q_len=None):
    p = qat.cca_params(batch=q.shape[0], seq_len=q.shape[1], n_q_heads=q.shape[2], n_kv_heads=k.shape[2],
                       head_dim=q.shape[3], group=group, window=window, q_start=q_start, q_len=q_len)
    kc, vc = qat.cca_pool(p, q, k, v)
    out, lse = qat.cca_attn(p, q, k, v, kc, vc)
    torch.cuda.synchronize()
    return p, kc, vc, out, lse


def check(q, k, v, group, window, q_start=0, q_len=None, rows=None):
    p, kc, vc, out, lse = run(q, k, v, group, window, q_start, q_len)
    if rows is None:
        rows = list(range(p.q_start, p.q_start + p.q_len))
    rel = [t - p.q_start for t in rows]
    need = occa.window_start(p.q_start + p.q_len - 1, group, window) // group
    for bi in range(q.shape[0]):
        qn, kn, vn = to64(q[bi]), to64(k[bi]), to64(v[bi])
        kc_r, vc_r = occa.pool(qn, kn, vn, group, p.scale, need)
        # the core rows are stored in bfloat16: compare within bf16 rounding
        assert_close(to64(kc[bi, :need]), kc_r, 1e-2, "core keys")
        assert_close(to64(vc[bi, :need]), vc_r, 1e-2, "core values")
        o_ref, lse_ref = occa.attend_rows(qn, kn, vn, kc_r, vc_r, group, window, p.scale, rows)
        assert_close(to64(out[bi, rel]), o_ref, BF16_TOL, "output")
        assert_close(to64(lse[bi, rel]), lse_ref, 1e-3, "lse")


SMALL = [
    # batch, N, hq, hkv, d, group, window, q_start, q_len
    (1, 1000, 4, 2, 128, 16, 64, 0, None),      # ragged N, GQA, several tiles
    (2, 777, 2, 2, 64, 8, 30, 100, 500),        # batch 2, offset rows, window not a multiple of g
    (1, 600, 2, 1, 128, 1, 10, 0, None),        # g = 1: dense causal
    (1, 512, 2, 2, 64, 32, 0, 0, None),         # w = 0: own group only in the window
    (1, 300, 4, 4, 128, 7, 1000, 0, None),      # window beyond the sequence: dense causal
    (1, 2000, 2, 2, 128, 64, 256, 1500, 500),   # large groups, final chunk only
    (3, 3001, 8, 2, 128, 16, 1024, 3000, 1),    # one new row per sequence (decode-like), GQA 4:1
    (1, 1500, 2, 2, 64, 128, 64, 0, None),      # window shorter than a group
    (2, 4097, 4, 4, 128, 32, 512, 4000, 97),    # ragged tail rows over several tiles' worth of core tokens
    (1, 100, 2, 2, 128, 128, 64, 0, None),      # group longer than the sequence: no core token exists
    (1, 256, 2, 1, 64, 256, 0, 0, None),        # one group spanning the sequence, w = 0
    (1, 700, 8, 1, 64, 16, 100, 0, None),       # 8 query heads per KV head, d 64
    (1, 999, 4, 2, 128, 3, 17, 0, None),        # odd group size and window
]


@pytest.mark.parametrize("case", SMALL, ids=[f"c{i}" for i in range(len(SMALL))])
def test_cca_small(case):
    b, n, hq, hkv, d, g, w, qs, ql = case
    print(f"[cca] {case}", flush=True)
    q, k, v, _ = synth.moba_inputs(90 + n, b, n, hq, hkv, d, torch.bfloat16, DEV)
    check(q, k, v, g, w, qs, ql)


def test_cca_64k_full_size():
    """Core-token attention over a 65536-token prefill, 32 heads x 128,
    groups of 16, window 1024: sampled rows against the oracle (the core
    tokens of every group are pooled by the oracle for the sampled heads)."""
    n, h, d, g, w = 65536, 32, 128, 16, 1024
    q, k, v, _ = synth.moba_inputs(91, 1, n, h, h, d, torch.bfloat16, DEV)
    p, kc, vc, out, lse = run(q, k, v, g, w)
    print("[cca 64k] gpu done", flush=True)
    rows = [0, 15, 16, 1039, 1040, 1041, 30000, n - 1]
    heads = [0, 31]
    qn = to64(q[0][:, heads])
    kn, vn = to64(k[0][:, heads]), to64(v[0][:, heads])
    need = occa.window_start(n - 1, g, w) // g
    kc_r, vc_r = occa.pool(qn, kn, vn, g, p.scale, need)
    o_ref, lse_ref = occa.attend_rows(qn, kn, vn, kc_r, vc_r, g, w, p.scale, rows)
    assert_close(to64(out[0, rows][:, heads]), o_ref, BF16_TOL, "output")
    assert_close(to64(lse[0, rows][:, heads]), lse_ref, 1e-3, "lse")
