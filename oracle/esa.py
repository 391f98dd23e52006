"""ESA (Efficient Selective Attention): compression, importance, neighbour
influence, top-k token selection and attention over the fused parts.

Source: ESA write-up (hlszyjy.com/post/6872.html), the paragraphs on
token-level selection, the four-part token split with chunked prefill,
merging of heads, the one-layer compression MLP, score correction and
neighbour influence; the re-post (qqssy.cn) repeats them. The page's text
keeps the lead-in of each formula but drops the formulas themselves, so the
steps marked READING below are this library's stated definitions.

One sequence, chunk C = [c0, c0 + m) of queries (decode: m = 1, c0 = T - 1),
0-based positions:

1. Partition (four parts; READING): initial I = [0, min(n_init, c0)); local
   L = the W tokens just before the chunk, [max(n_init, c0 - W), c0); middle
   M = [n_init, max(n_init, c0 - W)); the chunk itself attends causally.
   Each query therefore sees at least W previous raw tokens, with the window
   aligned to the chunk (as the CCA write-up's locality module aligns its
   window to its group size).
2. Compression (one-layer MLP; READING: a single affine map, no activation):
   q~_i = Wq concat_h(q_i^h) + bq kept in float64; the compressed key cache
   holds k~_j = bf16(Wk concat_h(k_j^h) + bk), rounded to nearest even.
   Merging the heads into one 4096-wide vector is the write-up's head
   merging: one score, one selection for all heads.
3. Raw score s_ij = <q~_i, k~_j> for i in C, j in M.
4. Correction (READING; the formula is dropped, the text says it keeps the
   relative size of scores and stops one token from dominating):
   s^_ij = max(s_ij - max_j' s_ij', -clip).
   Alternative reading, behind a flag (correction="votes"): each query's
   scores become a softmax over the middle part at temperature tau,
   s^_ij = exp(tau s_ij) / sum_j' exp(tau s_ij'), so every query casts the
   same total vote of 1 (tau defaults to 1 / sqrt(d_c), the attention
   convention on the compressed width).
5. Importance u_j = sum_i s^_ij over all queries of the chunk ("takes every
   current query into account"); decode has one query.
6. Neighbour influence (READING; the formula is dropped, the text says a
   token's score is also shaped by the tokens around it and that a larger
   setting favours longer segments): u'_j = max{u_t : t in M, |t - j| <= r}.
7. Top-k: the min(k, |M|) largest u'_j, ties to the smaller position,
   returned in ascending order.
8. Attention: query t attends I u S u L u [c0, t], one joint softmax per
   head with the same S for every head (global part I u S and window part
   L u chunk fused, see oracle.attention.merge).

Per-head selection (the comparison arm of the write-up's ablation on head
merging; READING: with no per-head compression map on the page, each head h
scores the middle part with its own uncompressed q^h and k^h, s^h_ij =
<q_i^h, k_j^h>, then steps 4-7 run per head; in step 8 head h attends its
own selection). ``select_heads`` returns one selection per head and
``attend`` / ``backward`` take such a list in place of the shared one.

Parity: steps 1-3 and 5, 7, 8 are pinned by CPU tests (k >= |M| equals dense
causal attention; clip = inf and r = 0 reduce selection to one matrix-vector
product and a sort; exhaustive sort on tiny inputs; maximum_filter1d for the
neighbour step; bf16 rounding against torch). Steps 4 and 6 are pinned only
against this module's own READING (special cases clip -> 0, r = 0 and
plateau structure): their agreement with the original ESA formulas is
parity unpinned, since the pages do not carry those formulas.
"""
import numpy as np

from .attention import attend as attend_row
from .attention import attend_grad, attend_heads
from .numerics import round_to_bf16


def partition(c0, n_init, window):
    """Returns (I, M, L) as numpy index ranges for a chunk starting at c0."""
    I = np.arange(0, min(n_init, c0))
    if c0 > n_init:
        lstart = max(n_init, c0 - window)
        M = np.arange(n_init, lstart)
        L = np.arange(lstart, c0)
    else:
        M = np.arange(0)
        L = np.arange(0)
    return I, M, L


def compress(x, W, b=None):
    """x [n, D] (concatenated heads), W [d_c, D] -> [n, d_c] in float64."""
    out = np.asarray(x, np.float64) @ np.asarray(W, np.float64).T
    if b is not None:
        out = out + np.asarray(b, np.float64)
    return out


def key_cache(k, Wk, bk=None):
    """k [T, H, d] -> compressed key cache [T, d_c], rounded to bf16."""
    T = k.shape[0]
    return round_to_bf16(compress(np.asarray(k, np.float64).reshape(T, -1), Wk, bk))


def importance(qc, kc_mid, clip, row_chunk=256, correction="clamp", tau=None):
    """qc [m, d_c], kc_mid [n_M, d_c] -> (u [n_M], rowmax [m]).
    Steps 3-5: u_j = sum_i max(s_ij - max_j' s_ij', -clip); with
    correction="votes", u_j = sum_i softmax_j(tau s_i.)_j (tau: None means
    1 / sqrt(d_c))."""
    qc = np.asarray(qc, np.float64)
    kc_mid = np.asarray(kc_mid, np.float64)
    n_mid = kc_mid.shape[0]
    u = np.zeros(n_mid)
    rowmax = np.full(qc.shape[0], -np.inf)
    if n_mid == 0:
        return u, rowmax
    if correction == "votes" and tau is None:
        tau = 1.0 / np.sqrt(qc.shape[1])
    for i0 in range(0, qc.shape[0], row_chunk):
        s = qc[i0:i0 + row_chunk] @ kc_mid.T
        mrow = s.max(axis=1)
        rowmax[i0:i0 + row_chunk] = mrow
        if correction == "votes":
            # the row max is subtracted only to keep exp in range; the
            # softmax does not depend on it
            e = np.exp(tau * (s - mrow[:, None]))
            u += (e / e.sum(axis=1, keepdims=True)).sum(axis=0)
        else:
            u += np.maximum(s - mrow[:, None], -clip).sum(axis=0)
    return u, rowmax


def neighbour(u, radius):
    """Step 6: u'_j = max of u over the positions within distance r of j that
    lie inside the middle part."""
    u = np.asarray(u, np.float64)
    out = u.copy()
    n = u.shape[0]
    for off in range(1, radius + 1):
        if off >= n:
            break
        out[:-off] = np.maximum(out[:-off], u[off:])
        out[off:] = np.maximum(out[off:], u[:-off])
    return out


def top_k(scores, k):
    """Step 7: indices of the min(k, n) largest scores, ties to the smaller
    index, ascending. Full sort on (-score, index)."""
    scores = np.asarray(scores, np.float64)
    order = np.lexsort((np.arange(scores.shape[0]), -scores))
    return np.sort(order[:min(k, scores.shape[0])])


def select(q, Wq, bq, kc_cache, c0, n_init, window, topk, radius, clip, correction="clamp", tau=None):
    """Selection for one sequence and chunk.

    q [m, H, d] the chunk's queries, kc_cache [T, d_c] the compressed key
    cache (bf16 values). Returns (sel: absolute positions ascending,
    scores u' over M, importance u over M, rowmax [m]).
    """
    m = q.shape[0]
    _, M, _ = partition(c0, n_init, window)
    qc = compress(np.asarray(q, np.float64).reshape(m, -1), Wq, bq)
    u, rowmax = importance(qc, np.asarray(kc_cache, np.float64)[M], clip, correction=correction, tau=tau)
    up = neighbour(u, radius)
    sel = M[top_k(up, topk)] if M.size else np.zeros(0, dtype=np.int64)
    return sel, up, u, rowmax


def select_heads(q, K, c0, n_init, window, topk, radius, clip, correction="clamp", tau=None):
    """Per-head selection for one sequence and chunk. q [m, H, d] the chunk's
    queries, K [T, H, d] the key cache (or a view whose K[rows, h] returns
    those rows of head h). Returns (sels: H ascending position arrays,
    ups [H, |M|] the per-head u')."""
    m, H, d = q.shape
    _, M, _ = partition(c0, n_init, window)
    q = np.asarray(q, np.float64)
    sels, ups = [], np.zeros((H, M.size))
    for h in range(H):
        if M.size == 0:
            sels.append(np.zeros(0, dtype=np.int64))
            continue
        u, _ = importance(q[:, h], np.asarray(K[M, h], np.float64), clip, correction=correction, tau=tau)
        ups[h] = neighbour(u, radius)
        sels.append(M[top_k(ups[h], topk)])
    return sels, ups


def _per_head(sel):
    """A list / tuple of arrays is one selection per head; anything else is
    the selection shared by every head."""
    return isinstance(sel, (list, tuple))


def key_list(sel, c0, n_init, window, t):
    I, _, L = partition(c0, n_init, window)
    return np.concatenate([I, np.asarray(sel, np.int64), L, np.arange(c0, t + 1)])


def attend(q, K, V, sel, c0, n_init, window, scale, rows=None):
    """Step 8 for one sequence. q [m, H, d] (chunk rows), K/V [T, H, d].
    rows: chunk-relative query indices (default all); sel: the shared
    selection, or a list of one per head. Returns o [len(rows), H, d],
    lse [len(rows), H]."""
    m, H, d = q.shape
    if rows is None:
        rows = list(range(m))
    o = np.zeros((len(rows), H, V.shape[2]))
    lse = np.zeros((len(rows), H))
    for r, i in enumerate(rows):
        if _per_head(sel):
            for h in range(H):
                idx = key_list(sel[h], c0, n_init, window, c0 + i)
                o[r, h], lse[r, h] = attend_row(np.asarray(q[i, h], np.float64),
                                                np.asarray(K[idx, h], np.float64),
                                                np.asarray(V[idx, h], np.float64), scale)
            continue
        idx = key_list(sel, c0, n_init, window, c0 + i)
        o[r], lse[r] = attend_heads(np.asarray(q[i], np.float64),
                                    np.asarray(K[idx], np.float64),
                                    np.asarray(V[idx], np.float64), scale)
    return o, lse


def backward(q, K, V, sel, c0, n_init, window, scale, do, rows=None, heads=None):
    """Gradients of step 8 with the selection held fixed (a discrete top-k):
    q [m, H, d] chunk rows, K/V [T, H, d], do [len(rows), H, d]. Returns
    dq [len(rows), H, d] and dK, dV [T, H, d] with every listed row's
    contribution added (heads: the heads to compute, default all; the others
    stay zero)."""
    m, H, d = q.shape
    if rows is None:
        rows = list(range(m))
    if heads is None:
        heads = list(range(H))
    dq = np.zeros((len(rows), H, d))
    dK = np.zeros(K.shape)
    dV = np.zeros(V.shape)
    for r, i in enumerate(rows):
        for h in heads:
            idx = key_list(sel[h] if _per_head(sel) else sel, c0, n_init, window, c0 + i)
            dq[r, h], gk, gv = attend_grad(q[i, h], np.asarray(K[idx, h], np.float64),
                                           np.asarray(V[idx, h], np.float64), scale, do[r, h])
            dK[idx, h] += gk
            dV[idx, h] += gv
    return dq, dK, dV
