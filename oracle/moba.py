"""MoBA (Mixture of Block Attention): block scoring, gating and attention.

Source: MoBA write-up, section 3 ("block partition and selection") and
section 2 (attention restricted to the selected set).

Definitions, one sequence at a time, 0-based positions:

* block b holds keys [b*B, (b+1)*B) -- the write-up's 1-based range
  I_i = [(i-1)B + 1, iB] shifted to 0-based; a trailing partial block holds
  the remaining keys;
* affinity s_b = <q, mean_pool(K[block b])>, an unscaled inner product of
  the query with the block's mean key (section 3, affinity equation);
* causality: blocks that are not strictly earlier than the query's own block
  cur(t) = floor(t / B) get s_b = -inf and are never gated in (reading of
  the rule "s_i = -inf, g_i = 0 if pos(q) < i*B": the current block never
  competes because it is forced in anyway);
* gating: the top (k - 1) earlier blocks by s_b, ties to the smaller block
  index, plus the forced current block (section 3, "force q to attend its
  current block, with a causal mask"); k counts the forced block (reading
  that matches both 95.31% = 1 - 3/64 sparsity in the experiments section
  and k = 1 giving current-block-only attention);
* keys of query t: the union of the gated earlier blocks, the causal part
  [cur(t)*B, t] of its own block and, if window w > 0, the extra local keys
  [max(0, t - w + 1), t]; each key counted once;
* grouped-query attention: query head h reads KV head h // (Hq / Hkv)
  (attention blog, section on MQA/GQA head grouping; the contiguous mapping
  is this library's convention).

Pins: tests/test_oracle_pins.py -- k >= number of blocks equals dense causal
attention; k = 1 equals block-diagonal causal attention; B = 1 equals a
brute-force token top-(k-1) by full sort; mean pool of constant blocks; GQA
equals MHA with the KV heads repeated; exhaustive-sort selection on tiny
inputs; 3 of 64 blocks gives the printed 95.31% sparsity.
"""
import numpy as np

from .attention import attend, attend_grad


def block_means(k, block):
    """k [N, Hkv, d] -> [nb, Hkv, d] block means, nb = ceil(N / block)."""
    k = np.asarray(k, np.float64)
    n = k.shape[0]
    nb = -(-n // block)
    out = np.zeros((nb, k.shape[1], k.shape[2]))
    for b in range(nb):
        out[b] = k[b * block:min(n, (b + 1) * block)].mean(axis=0)
    return out


def kv_head(h, hq, hkv):
    return h // (hq // hkv)


def select_row(q_th, kbar_g, t, block, topk):
    """Gate one (query token t, head) row.

    q_th [d], kbar_g [nb, d] (block means of this head's KV head).
    Returns (blk [topk] ascending, -1 padded; scores [nb] with -inf where
    not a candidate).
    """
    nb = kbar_g.shape[0]
    cur = t // block
    scores = np.full(nb, -np.inf)
    scores[:cur] = kbar_g[:cur] @ np.asarray(q_th, np.float64)
    # full sort of the candidates on (-score, block index)
    order = np.lexsort((np.arange(cur), -scores[:cur]))
    picked = sorted(order[:max(0, topk - 1)].tolist() + [cur])
    blk = np.full(topk, -1, dtype=np.int64)
    blk[:len(picked)] = picked
    return blk, scores


def select(q, k, block, topk, rows, kbar=None):
    """q [N, Hq, d], k [N, Hkv, d]; rows = token positions.
    Returns blk [len(rows), Hq, topk] and scores [len(rows), Hq, nb]."""
    q = np.asarray(q, np.float64)
    hq, hkv = q.shape[1], k.shape[1]
    if kbar is None:
        kbar = block_means(k, block)
    nb = kbar.shape[0]
    blk = np.zeros((len(rows), hq, topk), dtype=np.int64)
    sc = np.zeros((len(rows), hq, nb))
    for r, t in enumerate(rows):
        for h in range(hq):
            blk[r, h], sc[r, h] = select_row(q[t, h], kbar[:, kv_head(h, hq, hkv)],
                                             t, block, topk)
    return blk, sc


def key_set(blk_row, t, block, window=0):
    """Sorted key positions attended by query t given its gated blocks."""
    cur = t // block
    parts = [np.arange(cur * block, t + 1)]
    for b in blk_row:
        if b >= 0 and b != cur:
            parts.append(np.arange(b * block, (b + 1) * block))
    if window > 0:
        parts.append(np.arange(max(0, t - window + 1), t + 1))
    return np.unique(np.concatenate(parts))


def attend_rows(q, k, v, block, blk, rows, scale, window=0):
    """Attention of the given rows over their gated key sets.
    blk [len(rows), Hq, topk]. Returns o [len(rows), Hq, d], lse [len(rows), Hq]."""
    q = np.asarray(q, np.float64)
    hq, hkv = q.shape[1], k.shape[1]
    o = np.zeros((len(rows), hq, v.shape[2]))
    lse = np.zeros((len(rows), hq))
    for r, t in enumerate(rows):
        for h in range(hq):
            idx = key_set(blk[r, h], t, block, window)
            g = kv_head(h, hq, hkv)
            o[r, h], lse[r, h] = attend(q[t, h], np.asarray(k[idx, g], np.float64),
                                        np.asarray(v[idx, g], np.float64), scale)
    return o, lse


def forward(q, k, v, block, topk, scale, window=0, rows=None):
    """Selection then attention for one sequence. Returns (blk, scores, o, lse)."""
    if rows is None:
        rows = list(range(q.shape[0]))
    blk, sc = select(q, k, block, topk, rows)
    o, lse = attend_rows(q, k, v, block, blk, rows, scale, window)
    return blk, sc, o, lse


def backward_rows(q, k, v, block, blk, rows, scale, do, window=0):
    """Gradients of the attention of the given rows (gating held fixed: the
    gated sets blk are a discrete choice, as in the write-up's training,
    where the gate has no parameters of its own).

    q [N, Hq, d], k/v [N, Hkv, d], blk [len(rows), Hq, topk], do
    [len(rows), Hq, d]. Returns dq [len(rows), Hq, d] and dk, dv [N, Hkv, d]
    with every row's and head's contribution added (GQA: the query heads of
    a KV head add into it)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    hq, hkv = q.shape[1], k.shape[1]
    dq = np.zeros((len(rows), hq, q.shape[2]))
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for r, t in enumerate(rows):
        for h in range(hq):
            idx = key_set(blk[r, h], t, block, window)
            g = kv_head(h, hq, hkv)
            dq[r, h], dK, dV = attend_grad(q[t, h], k[idx, g], v[idx, g], scale, do[r, h])
            dk[idx, g] += dK
            dv[idx, g] += dV
    return dq, dk, dv
