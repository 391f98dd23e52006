"""CCA-style core-token attention: query-aware group pooling plus a
group-aligned local window, fused in one softmax.

Test infrastructure only (the library's GPU path never imports it).

Source: CCA-Attention ICML 2025 write-up (m.jxzklqfsx.com/article/817694.html),
sections on the global-aware pooling module, the locality-preserving module
and the global-local fusion; the page drops every equation, so the steps
below are this oracle's stated READINGS (listed with the library's readings
of the pages):

1. Groups: the sequence is cut into non-overlapping groups of g tokens,
   group i = positions [i g, (i + 1) g); only complete groups are pooled.
2. Core token of group i (per query head h): the group's LAST token's query
   scores the group's keys, a_j = softmax_j(scale <q_{(i+1)g-1,h}, k_j>), and
   the core key / value are the a-weighted sums of the group's keys / values
   (READING: the pooled token goes through the same linear K / V maps as the
   raw tokens -- the page says the two modules share their linear
   transforms -- so pooling the token and then projecting equals pooling the
   projected keys and values; no learned parameters enter).
3. Local window (READING of "at least w previous raw tokens, window aligned
   to the group size"): query t sees the raw tokens [ls(t), t] with
   ls(t) = max(0, floor(t / g) g - ceil(w / g) g), so the window starts on a
   group boundary and holds at least min(t, w) earlier tokens.
4. Global part: the core tokens of the groups that end at or before ls(t),
   i < ls(t) / g (all of them precede the window; causal by construction).
5. Fusion: one softmax over the union of the core tokens and the window
   (the page's unified K / V), computed as one attention over the
   concatenation.

Pins (tests/test_oracle_pins.py): g = 1 equals dense causal attention for any
w; w >= t equals dense causal attention; identical keys in a group give that
key and the group's mean value; the core depends on the group's last query
only; the window start equals the latest group boundary, found by search,
from which every query of the group still sees >= min(t, w) earlier tokens
(a window one group wider or narrower fails); the rows equal attention over
a key set enumerated position by position; with Hq = 4 over Hkv = 2 the
result equals MHA with each KV head repeated in place (an interleaved head
map fails).
"""
import numpy as np

from .attention import attend


def kv_head(h, hq, hkv):
    return h // (hq // hkv)


def window_start(t, g, w):
    """ls(t): first raw position query t sees (step 3)."""
    wg = -(-w // g) * g
    return max(0, (t // g) * g - wg)


def pool(q, k, v, g, scale, n_groups=None):
    """Core keys / values (step 2). q [N, Hq, d], k/v [N, Hkv, d] -> kc, vc
    [n_groups, Hq, d] for the first n_groups complete groups."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n, hq, d = q.shape
    hkv = k.shape[1]
    if n_groups is None:
        n_groups = n // g
    kc = np.zeros((n_groups, hq, d))
    vc = np.zeros((n_groups, hq, v.shape[2]))
    for i in range(n_groups):
        sl = slice(i * g, (i + 1) * g)
        for h in range(hq):
            gh = kv_head(h, hq, hkv)
            s = scale * (k[sl, gh] @ q[(i + 1) * g - 1, h])
            a = np.exp(s - s.max())
            a /= a.sum()
            kc[i, h] = a @ k[sl, gh]
            vc[i, h] = a @ v[sl, gh]
    return kc, vc


def attend_rows(q, k, v, kc, vc, g, w, scale, rows):
    """Steps 3-5 for the given positions. Returns o [len(rows), Hq, d] and
    lse [len(rows), Hq]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    hq, hkv = q.shape[1], k.shape[1]
    o = np.zeros((len(rows), hq, v.shape[2]))
    lse = np.zeros((len(rows), hq))
    for r, t in enumerate(rows):
        ls = window_start(t, g, w)
        nc = ls // g
        for h in range(hq):
            gh = kv_head(h, hq, hkv)
            K = np.concatenate([kc[:nc, h], k[ls:t + 1, gh]])
            V = np.concatenate([vc[:nc, h], v[ls:t + 1, gh]])
            o[r, h], lse[r, h] = attend(q[t, h], K, V, scale)
    return o, lse
