"""GPU parity of ESA's per-head selection (esa_select_heads, then
esa_sparse_attn and esa_sparse_attn_bwd with per_head = 1, through the C ABI)
against the float64 oracle (oracle.esa.select_heads / attend / backward with
one selection per head) on the same seeded inputs."""
import numpy as np
import pytest
import torch

import query_aware_top_amd as qat
import synth
from oracle import esa as oesa
from parity import BF16_TOL, assert_close, selection_ok, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


class _Rows:
    """Row view of a large GPU tensor for the oracle: x[rows] or x[rows, h]
    copies only those rows (of head h) to the host as float64."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, idx):
        rest = ()
        if isinstance(idx, tuple):
            idx, rest = idx[0], idx[1:]
        ix = torch.as_tensor(np.asarray(idx), device=self.t.device, dtype=torch.long)
        return to64(self.t.index_select(0, ix)[(slice(None),) + rest])


def run(seed, B, T, c0, m, H, d, n_init, W, topk, radius, clip, correction="clamp", planted=False):
    _, k, v, _ = synth.esa_inputs(seed, B, T, 1, H, d, torch.bfloat16, DEV)
    q = synth.normal(seed, synth.gen.TID_Q, (B, m, H, d), torch.bfloat16, DEV, start=1 << 40)
    pos = None
    if planted:   # head h of sequence b: one key at its own position along its queries
        if m > 1:   # all chunk queries of a head equal, so every query ranks the key first
            q[:] = q[:, :1]
        _, M, _ = oesa.partition(c0, n_init, W)
        g = np.random.default_rng(seed)
        pos = g.choice(M, size=(B, H), replace=False) if M.size >= B * H else None
        for bi in range(B):
            for h in range(H):
                k[bi, int(pos[bi, h]), h] = (q[bi, 0, h].to(torch.float64) * 0.375).to(torch.bfloat16)
    p = qat.esa_params(batch=B, n_heads=H, head_dim=d, d_c=128, ctx_len=T, chunk_start=c0, chunk_len=m,
                       n_init=n_init, window=W, topk=topk, radius=radius, clip=clip, correction=correction,
                       per_head=True)
    sel, n_sel, scores = qat.esa_select_heads(p, q, k, want_scores=True)
    out, lse = qat.esa_sparse_attn(p, q, k, v, sel, n_sel)
    torch.cuda.synchronize()
    return p, q, k, v, sel, n_sel, scores, out, lse, pos


def check_selection(p, q, k, sel, n_sel, scores, bi, heads, correction="clamp", K=None):
    c0, n_init, W = p.chunk_start, p.n_init, p.window
    _, M, _ = oesa.partition(c0, n_init, W)
    qn = to64(q[bi][:, heads])
    Kh = K if K is not None else to64(k[bi][:, heads])
    sels_ref, ups = oesa.select_heads(qn, Kh, c0, n_init, W, p.topk, p.radius, p.clip, correction=correction)
    swaps = 0
    for r, h in enumerate(heads):
        ns = int(n_sel[bi, h])
        assert ns == len(sels_ref[r])
        sg = sel[bi, h, :ns].cpu().numpy().astype(np.int64)
        assert np.all(np.diff(sg) > 0), "selection not ascending"
        assert np.all(sel[bi, h, ns:].cpu().numpy() == -1)
        ok, n = selection_ok(sg - n_init, sels_ref[r] - n_init, ups[r], p.topk)
        assert ok, f"sequence {bi} head {h}: selection differs outside the tie band"
        swaps += n
        if M.size:
            sc = to64(scores[bi, h, :M.size])
            if correction == "votes":
                err = np.abs(sc - ups[r]) / np.maximum(np.abs(ups[r]), 1e-30)
                assert np.max(err) < 1e-3, f"vote importance: max relative error {np.max(err):.3e}"
            else:
                assert_close(sc, ups[r], 1e-4, "importance scores")
    return swaps


def gpu_sels(sel, n_sel, bi, H):
    return [sel[bi, h, :int(n_sel[bi, h])].cpu().numpy().astype(np.int64) for h in range(H)]


SMALL = [
    # seed, B, T, c0, m, H, d, n_init, W, topk, radius, clip, correction
    (81, 1, 2048, 1600, 300, 4, 128, 16, 128, 100, 2, 12.0, "clamp"),   # several query and key tiles
    (82, 2, 1500, 1000, 257, 3, 64, 8, 64, 50, 1, 6.0, "clamp"),        # batch 2, ragged chunk, d 64
    (83, 1, 1800, 1500, 200, 2, 128, 16, 100, 64, 0, 48.0, "votes"),    # softmax-vote correction
    (84, 3, 3000, 2999, 1, 4, 128, 32, 256, 300, 2, 24.0, "clamp"),     # decode
    (85, 2, 2500, 2499, 1, 2, 64, 8, 128, 100, 1, 8.0, "votes"),        # decode, votes
    (86, 1, 300, 20, 100, 2, 64, 32, 16, 10, 2, 4.0, "clamp"),          # chunk inside the initial part: M empty
    (87, 1, 600, 400, 130, 2, 64, 16, 32, 1000, 2, 5.0, "clamp"),       # k >= |M|: dense causal
]


@pytest.mark.parametrize("case", SMALL, ids=[f"h{i}" for i in range(len(SMALL))])
def test_esa_heads_small(case):
    seed, B, T, c0, m, H, d, n_init, W, topk, radius, clip, corr = case
    print(f"[esa heads] {case}", flush=True)
    p, q, k, v, sel, n_sel, scores, out, lse, _ = run(seed, B, T, c0, m, H, d, n_init, W, topk, radius, clip, corr)
    for bi in range(B):
        check_selection(p, q, k, sel, n_sel, scores, bi, list(range(H)), corr)
        sels = gpu_sels(sel, n_sel, bi, H)
        o_ref, lse_ref = oesa.attend(to64(q[bi]), to64(k[bi]), to64(v[bi]), sels, c0, n_init, W, p.scale)
        assert_close(to64(out[bi]), o_ref, BF16_TOL, "output")
        assert_close(to64(lse[bi]), lse_ref, 1e-3, "lse")
    # gradients over the per-head lists
    do = synth.normal(seed, 7, (B, m, H, d), torch.bfloat16, DEV)
    dq, dk, dv = qat.esa_sparse_attn_bwd(p, q, k, v, sel, n_sel, do, lse)
    torch.cuda.synchronize()
    for bi in range(B):
        sels = gpu_sels(sel, n_sel, bi, H)
        dq_r, dk_r, dv_r = oesa.backward(to64(q[bi]), to64(k[bi]), to64(v[bi]), sels, c0, n_init, W, p.scale,
                                         to64(do[bi]))
        assert_close(to64(dq[bi]), dq_r, 2e-3, "dq")
        assert_close(to64(dk[bi]), dk_r, 2e-3, "dk")
        assert_close(to64(dv[bi]), dv_r, 2e-3, "dv")


def test_esa_heads_planted_needles_prefill():
    """A key planted per (sequence, head) along that head's first query is
    selected by its own head."""
    p, q, k, v, sel, n_sel, scores, out, lse, pos = run(88, 2, 4096, 3000, 64, 4, 128, 16, 256, 200, 0, 48.0,
                                                        planted=True)
    for bi in range(2):
        for h in range(4):
            assert int(pos[bi, h]) in set(sel[bi, h, :int(n_sel[bi, h])].cpu().tolist()), (bi, h)


def test_esa_heads_merged_and_per_head_disagree():
    """The per-head path really selects per head: with planted per-head keys
    the heads' selections differ from one another."""
    p, q, k, v, sel, n_sel, scores, out, lse, pos = run(89, 1, 4096, 4095, 1, 4, 128, 16, 256, 50, 0, 48.0,
                                                        planted=True)
    sets = [frozenset(sel[0, h, :int(n_sel[0, h])].cpu().tolist()) for h in range(4)]
    assert len(set(sets)) == 4


def test_esa_heads_prefill_64k_full_size():
    """The 64k chunked prefill shape (32 heads x 128, chunk 2048, top 2048 of
    59264 middle tokens per head, 128 + 2048 + 4096 gathered keys): the
    selection of heads 0 and 31 against the oracle, outputs of sampled rows
    (all heads, each over its own list)."""
    T, c0, m, H, d = 65536, 63488, 2048, 32, 128
    p, q, k, v, sel, n_sel, scores, out, lse, _ = run(3, 1, T, c0, m, H, d, 128, 4096, 2048, 2, 48.0)
    print("[esa heads 64k] gpu done", flush=True)
    K = _Rows(k[0])
    heads = [0, 31]

    class _Head:   # the oracle reads K[rows, h] with h indexing the sampled heads
        def __getitem__(self, idx):
            rows, r = idx
            return K[rows, heads[r]]

    check_selection(p, q, k, sel, n_sel, scores, 0, heads, K=_Head())
    print("[esa heads 64k] selection checked", flush=True)
    sels = gpu_sels(sel, n_sel, 0, H)
    rows = [0, 1, 1000, 2047]
    o_ref, lse_ref = oesa.attend(to64(q[0]), K, _Rows(v[0]), sels, c0, 128, 4096, p.scale, rows=rows)
    assert_close(to64(out[0, rows]), o_ref, BF16_TOL, "output")
    assert_close(to64(lse[0, rows]), lse_ref, 1e-3, "lse")


def test_esa_heads_decode_128k_full_size():
    """Decode at 128k context per head (4 sequences, 32 heads x 128, top
    2048): every (sequence, head) selects its own planted key; the selection
    of sampled (sequence, head) pairs against the oracle; outputs of all
    heads of two sequences."""
    B, T, H, d = 4, 131072, 32, 128
    p, q, k, v, sel, n_sel, scores, out, lse, pos = run(4, B, T, T - 1, 1, H, d, 128, 4096, 2048, 2, 48.0,
                                                        planted=True)
    print("[esa heads 128k] gpu done", flush=True)
    for bi in range(B):
        for h in range(H):
            assert int(pos[bi, h]) in set(sel[bi, h, :int(n_sel[bi, h])].cpu().tolist()), (bi, h)
    for bi, heads in ((0, [0, 17]), (3, [31])):
        K = _Rows(k[bi])

        class _Head:
            def __getitem__(self, idx, K=K, heads=heads):
                rows, r = idx
                return K[rows, heads[r]]

        check_selection(p, q, k, sel, n_sel, scores, bi, heads, K=_Head())
    for bi in (0, 3):
        sels = gpu_sels(sel, n_sel, bi, H)
        o_ref, lse_ref = oesa.attend(to64(q[bi]), _Rows(k[bi]), _Rows(v[bi]), sels, T - 1, 128, 4096, p.scale)
        assert_close(to64(out[bi]), o_ref, BF16_TOL, "output")
        assert_close(to64(lse[bi]), lse_ref, 1e-3, "lse")
