"""GPU parity of the ESA path (esa_compress, esa_select, esa_sparse_attn
through the C ABI) against the float64 CPU oracle on the same seeded inputs.

The compressed-key cache is computed on each side by its own code (GPU:
float64-accumulated compression kernel; oracle: float64 matmul and
round-to-nearest-even); the two must agree bit for bit before the selection
is compared.
"""
import math

import numpy as np
import pytest
import torch

import query_aware_top_amd as qat
import synth
from oracle import esa as oesa
from oracle.numerics import round_to_bf16
from parity import BF16_TOL, F32_TOL, assert_close, selection_ok, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def oracle_key_cache(k_seq: torch.Tensor, Wk: np.ndarray, chunk=8192) -> np.ndarray:
    """Oracle compression of one sequence's keys [T, H, d] (GPU tensor),
    streamed to the host in chunks."""
    T = k_seq.shape[0]
    out = np.zeros((T, Wk.shape[0]))
    for s in range(0, T, chunk):
        out[s:s + chunk] = oesa.key_cache(to64(k_seq[s:s + chunk]), Wk)
    return out


def gpu_key_cache(k: torch.Tensor, Wk: torch.Tensor) -> torch.Tensor:
    B, T, H, d = k.shape
    kc = qat.esa_compress(k.view(B * T, H * d), Wk, out_dtype=torch.bfloat16)
    return kc.view(B, T, -1)


def esa_case(seed, B, T, c0, m, H, d, d_c, n_init, W, topk, radius, clip, dtype=torch.bfloat16, needles=0,
             rows=None, seqs=None, correction="clamp", vote_tau=0.0):
    q_all, k, v, info = synth.esa_inputs(seed, B, T, 1, H, d, dtype, DEV)
    q = synth.normal(seed, synth.gen.TID_Q, (B, m, H, d), dtype, DEV, start=1 << 40)
    if needles:
        for bi in range(B):
            pos = synth.needle_positions(seed, bi, needles, n_init, max(n_init + 1, c0 - W), 2 * radius + 1)
            val = (q[bi, 0].to(torch.float64) * 0.375).to(dtype)
            for t in pos:
                k[bi, t] = val
            info.setdefault("needles", []).append(pos)
    # one shared random map for q and k (a Johnson-Lindenstrauss stand-in for
    # the trained compression): <Wq q, Wk k> tracks the head-summed <q, k>
    Wq = synth.compression_weights(seed, d_c, H * d, synth.gen.TID_W, dtype, DEV)
    Wk = Wq
    p = qat.esa_params(batch=B, n_heads=H, head_dim=d, d_c=d_c, ctx_len=T, chunk_start=c0, chunk_len=m,
                       n_init=n_init, window=W, topk=topk, radius=radius, clip=clip, dtype=dtype,
                       correction=correction, vote_tau=vote_tau)
    kc = gpu_key_cache(k, Wk)
    sel, n_sel, scores = qat.esa_select(p, q, Wq, None, kc, want_scores=True)
    out, lse = qat.esa_sparse_attn(p, q, k, v, sel, n_sel)
    torch.cuda.synchronize()
    print(f"[esa] gpu done B={B} T={T} m={m}", flush=True)
    if needles:   # every sequence, on the GPU's own output
        for bi in range(B):
            got = set(sel[bi, :int(n_sel[bi])].cpu().tolist())
            assert set(info["needles"][bi]) <= got, f"sequence {bi}: a planted needle was not selected"
    Wq_n, Wk_n = to64(Wq), to64(Wk)
    _, M, _ = oesa.partition(c0, n_init, W)
    tol = BF16_TOL if dtype == torch.bfloat16 else F32_TOL
    lse_tol = 1e-3 if dtype == torch.bfloat16 else 1e-5
    swaps = 0
    for bi in (seqs if seqs is not None else range(B)):
        kc_ref = oracle_key_cache(k[bi], Wk_n)
        kc_gpu = to64(kc[bi])
        assert np.array_equal(kc_gpu, kc_ref), f"compressed keys differ in {np.sum(kc_gpu != kc_ref)} entries"
        qn = to64(q[bi])
        sel_ref, up, _, _ = oesa.select(qn, Wq_n, None, kc_ref, c0, n_init, W, topk, radius, clip,
                                        correction=correction, tau=vote_tau if vote_tau > 0 else None)
        ns = int(n_sel[bi])
        assert ns == len(sel_ref)
        sg = sel[bi, :ns].cpu().numpy().astype(np.int64)
        assert np.all(np.diff(sg) > 0), "selection not ascending"
        assert np.all(sel[bi, ns:].cpu().numpy() == -1)
        ok, n = selection_ok(sg - n_init, sel_ref - n_init, up, topk)
        assert ok, f"sequence {bi}: selection differs outside the tie band"
        swaps += n
        if len(M):
            sc = to64(scores[bi, :len(M)])
            if correction == "votes":   # votes lie in (0, m]: relative comparison
                err = np.abs(sc - up) / np.maximum(np.abs(up), 1e-30)
                assert np.max(err) < 1e-3, f"vote importance: max relative error {np.max(err):.3e}"
            else:
                assert_close(sc, up, 1e-4, "importance scores")
        r = rows if rows is not None else list(range(m))
        o_ref, lse_ref = oesa.attend(qn, to64(k[bi]) if T * H * d < 2 ** 26 else _KV(k[bi]),
                                     to64(v[bi]) if T * H * d < 2 ** 26 else _KV(v[bi]), sg, c0, n_init, W,
                                     p.scale, rows=r)
        assert_close(to64(out[bi, r]), o_ref, tol, "output")
        assert_close(to64(lse[bi, r]), lse_ref, lse_tol, "lse")
        if needles:
            assert set(info["needles"][bi]) <= set(sg.tolist()), "a planted needle was not selected"
    return swaps


class _KV:
    """Row-gather view of a large GPU tensor for the oracle: K[idx] copies
    only the requested rows to the host as float64."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, idx):
        ix = torch.as_tensor(np.asarray(idx), device=self.t.device, dtype=torch.long)
        return to64(self.t.index_select(0, ix))


def test_compress_bf16_is_correctly_rounded():
    x = synth.normal(21, 1, (300, 1024), torch.bfloat16, DEV)
    W = synth.compression_weights(21, 64, 1024, dtype=torch.bfloat16, device=DEV)
    out = qat.esa_compress(x, W, out_dtype=torch.bfloat16)
    ref = round_to_bf16(to64(x) @ to64(W).T)
    assert np.array_equal(to64(out), ref)


def test_compress_f32_bias_and_strides():
    x = synth.normal(22, 1, (7, 50, 512), torch.float32, DEV)    # rows at stride 50*512
    W = synth.normal(22, 4, (32, 512), torch.float32, DEV, scale=0.05)
    bias = synth.normal(22, 5, (32,), torch.float32, DEV)
    base = torch.zeros(7, 3, 32, dtype=torch.float32, device=DEV)
    qat.esa_compress(x, W, bias, out=base, n=7, x_stride=50 * 512, out_stride=3 * 32)
    ref = to64(x[:, 0]) @ to64(W).T + to64(bias)
    got = to64(base[:, 0])
    assert np.all(np.abs(got - ref) <= 2.0 ** -23 * np.abs(ref) + 1e-30)
    assert torch.all(base[:, 1:] == 0)


SMALL = [
    # seed, B, T, c0, m, H, d, d_c, n_init, W, topk, radius, clip
    (1, 1, 2048, 1600, 300, 4, 128, 64, 16, 128, 100, 2, 12.0),
    (2, 2, 1500, 1000, 257, 2, 64, 32, 8, 64, 50, 1, 6.0),
    (3, 1, 600, 400, 130, 2, 64, 128, 16, 32, 1000, 2, 5.0),      # k >= |M|: everything selected
    (4, 1, 300, 20, 100, 2, 64, 64, 32, 16, 10, 2, 4.0),         # chunk inside the initial part: M empty
    (5, 1, 900, 700, 150, 2, 64, 64, 8, 64, 40, 0, math.inf),    # no correction, no neighbours
    (6, 1, 1200, 1000, 64, 2, 128, 256, 4, 100, 77, 3, 3.0),     # d_c 256, one partial tile
]


@pytest.mark.parametrize("case", SMALL, ids=[f"c{i}" for i in range(len(SMALL))])
def test_esa_chunk_small(case):
    print(f"[esa small] {case}", flush=True)
    esa_case(*case)


def test_esa_chunk_fp32():
    esa_case(7, 1, 1000, 800, 100, 2, 64, 64, 16, 64, 60, 2, 8.0, dtype=torch.float32)


@pytest.mark.parametrize("H,d", [(16, 128), (8, 64), (4, 64)])
def test_esa_decode_small(H, d):
    """One query per sequence (decode kernel when H*d is a multiple of 2048,
    the chunk kernel otherwise), planted needles."""
    T = 3000
    esa_case(8, 3, T, T - 1, 1, H, d, 64, 32, 256, 300, 2, 24.0, needles=4)


EDGES = [
    # seed, B, T, c0, m, H, d, d_c, n_init, W, topk, radius, clip
    (40, 2, 300, 299, 1, 16, 128, 64, 32, 300, 16, 1, 24.0),     # decode, window reaches the initial part: M empty
    (41, 2, 100, 99, 1, 16, 128, 64, 128, 64, 16, 1, 24.0),      # decode inside the initial part: no window either
    (42, 2, 900, 899, 1, 16, 128, 64, 16, 64, 2000, 2, 8.0),     # decode, k >= |M|: every middle token selected
    (43, 5, 5000, 4999, 1, 32, 64, 128, 100, 1000, 700, 3, 16.0),  # decode, d 64 with 32 heads, radius 3
    (44, 3, 3000, 2999, 1, 16, 128, 64, 32, 0, 300, 2, 24.0),    # decode, no local window
    (45, 3, 3000, 2999, 1, 16, 128, 64, 0, 256, 300, 2, 24.0),   # decode, no initial tokens
    (46, 2, 2000, 1999, 1, 64, 128, 64, 16, 128, 200, 1, 24.0),  # decode, 64 heads (32 elements per thread)
    (47, 1, 1500, 1000, 200, 2, 64, 64, 0, 0, 100, 1, 6.0),      # chunk, no initial tokens and no window
    (48, 1, 300, 0, 300, 2, 64, 64, 16, 32, 10, 1, 4.0),         # chunk at position 0: only causal chunk keys
]


@pytest.mark.parametrize("case", EDGES, ids=[f"e{i}" for i in range(len(EDGES))])
def test_esa_edge_cases(case):
    """Boundaries of the four-part split: an empty middle part, a query
    inside the initial part, no window, no initial tokens, everything
    selected, the widest decode rows, a chunk at the start of the sequence."""
    print(f"[esa edge] {case}", flush=True)
    esa_case(*case)


def test_esa_prefill_64k_full_size():
    """ESA token-level chunked prefill, bf16: 32 heads x 128, q/k compressed
    4096 -> 128 by a seeded random one-layer map, context 65536, final query
    chunk of 2048, 128 initial + 2048 selected + 4096 local tokens, neighbour
    radius 2, clip 48; full selection and sampled output rows."""
    rows = [0, 1, 127, 128, 1000, 2046, 2047]
    esa_case(3, 1, 65536, 63488, 2048, 32, 128, 128, 128, 4096, 2048, 2, 48.0, rows=rows)


def test_esa_decode_128k_full_size():
    """ESA decode step, bf16: batch 16, 32 heads x 128, KV context 131072 per
    sequence, one query token, compressed dim 128, 128 init + 2048 selected +
    4096 window tokens, 16 planted needles per sequence; oracle check on
    three sequences, needles checked on the GPU for all sixteen."""
    esa_case(4, 16, 131072, 131071, 1, 32, 128, 128, 128, 4096, 2048, 2, 48.0, needles=16, seqs=[0, 7, 15])


@pytest.mark.parametrize("T", [20000, 40000], ids=["split4", "split8"])
def test_esa_decode_topk_split_widths(T):
    """Sixteen-sequence decode at contexts where the top-k passes take 4
    (T = 20000) and 8 (T = 40000) candidates per thread (the full-size decode
    takes 16, the 64k prefill 2); selection and output against the oracle on
    three sequences."""
    esa_case(9, 16, T, T - 1, 1, 4, 64, 64, 32, 256, 300, 2, 24.0, seqs=[0, 2, 15])


def test_esa_key_list_beyond_lds():
    """A key list longer than the 16384 entries the chunk kernel stages in
    LDS (64 initial + 5000 selected + 12000 window + 128 chunk keys): the
    tile loads take their positions from global memory."""
    esa_case(10, 1, 40000, 36000, 128, 2, 64, 64, 64, 12000, 5000, 2, 12.0, rows=[0, 1, 63, 127])


# ---- the alternative correction reading: per-query softmax votes -----------
VOTES = [
    # seed, B, T, c0, m, H, d, d_c, n_init, W, topk, radius, clip(unused), vote_tau
    (31, 1, 2048, 1600, 300, 4, 128, 64, 16, 128, 100, 2, 1.0, 0.0),      # default temperature
    (32, 2, 1500, 1000, 257, 2, 64, 32, 8, 64, 50, 0, 1.0, 0.5),          # batch 2, ragged chunk, no neighbours
    (33, 1, 1200, 1000, 64, 2, 128, 256, 4, 100, 77, 3, 1.0, 0.05),      # d_c 256, one partial tile
    (34, 3, 3000, 2999, 1, 16, 128, 64, 32, 256, 300, 2, 1.0, 0.0),      # decode, three sequences
    (35, 16, 20000, 19999, 1, 4, 64, 64, 32, 256, 300, 1, 1.0, 0.2),     # decode, 16 sequences, wider top-k split
]


@pytest.mark.parametrize("case", VOTES, ids=[f"v{i}" for i in range(len(VOTES))])
def test_esa_votes_small(case):
    """ESA with the softmax-vote reading of the score correction: selection
    within the tie band, importance within 1e-3 relative, outputs within
    tolerance, against the oracle's vote reading."""
    *args, tau = case
    print(f"[esa votes] {case}", flush=True)
    seqs = [0, 7, 15] if args[1] == 16 else None
    esa_case(*args, correction="votes", vote_tau=tau, seqs=seqs)


def test_esa_votes_prefill_64k_full_size():
    """The 64k chunked prefill with the vote reading (default temperature
    1/sqrt(128)); full selection and sampled output rows."""
    rows = [0, 1, 1000, 2047]
    esa_case(3, 1, 65536, 63488, 2048, 32, 128, 128, 128, 4096, 2048, 2, 48.0, rows=rows, correction="votes")
