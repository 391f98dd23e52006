"""Exact softmax attention over an explicit key set, and log-sum-exp merge.

Sources:
* MoBA write-up, section 1 (standard attention): Attn(q, K, V) =
  Softmax(q K^T) V for one query token against its keys; section 2: the same
  with K, V restricted to a selected index set I.
* Softmax scale: the pages' formulas carry no 1/sqrt(d) factor; the oracle
  takes the scale as a parameter (reading: standard scaled attention, all
  workloads use 1/sqrt(d)).
* Fusion of parts: the ESA write-up fuses "global" (initial + selected) and
  "window" (local) attention into one output; the CCA write-up (global-local
  fusion section) builds one unified K, V from both parts and runs a single
  softmax. Reading: the fused output is one joint softmax over the union of
  the parts, which is what ``merge`` reproduces from per-part (o, lse).

Pins (tests/test_oracle_pins.py): torch scaled_dot_product_attention in
float64 for dense causal attention; closed forms (identical keys -> mean of
V, scale 0 -> mean of V, one dominant key -> its value row, lse of a zero
query = log n); merge of random disjoint splits equals attention on the
union.
"""
import numpy as np


def attend(q, K, V, scale):
    """One query row q [d] against keys K [n, d] and values V [n, dv].

    Returns (o [dv], lse) with lse = log sum_j exp(scale * q.k_j), computed
    with the running maximum subtracted before exponentiation. An empty key
    set gives o = 0 and lse = -inf.
    """
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    if K.shape[0] == 0:
        return np.zeros(V.shape[1]), -np.inf
    s = scale * (K @ q)
    mx = s.max()
    w = np.exp(s - mx)
    l = w.sum()
    return (w @ V) / l, mx + np.log(l)


def attend_grad(q, K, V, scale, do):
    """Gradient of o = attend(q, K, V, scale)[0] against an upstream
    gradient do [dv]: returns (dq [d], dK [n, d], dV [n, dv]).

    With s = scale K q, P = softmax(s), o = P V (the definition of
    ``attend``): dV = P do^T, dP_j = do . v_j, D = sum_j P_j dP_j,
    dS_j = P_j (dP_j - D), dq = scale sum_j dS_j k_j, dK_j = scale dS_j q.
    An empty key set has zero gradients.
    """
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    do = np.asarray(do, np.float64)
    if K.shape[0] == 0:
        return np.zeros_like(q), np.zeros_like(K), np.zeros_like(V)
    s = scale * (K @ q)
    w = np.exp(s - s.max())
    P = w / w.sum()
    dV = np.outer(P, do)
    dP = V @ do
    dS = P * (dP - P @ dP)
    return scale * (dS @ K), scale * np.outer(dS, q), dV


def attend_heads(Q, K, V, scale):
    """Per-head attention of one query position: Q [H, d], K/V [n, H, d]
    -> o [H, d], lse [H]. Same definition as ``attend`` for every head."""
    H = Q.shape[0]
    o = np.zeros((H, V.shape[2]))
    lse = np.full(H, -np.inf)
    for h in range(H):
        o[h], lse[h] = attend(Q[h], K[:, h, :], V[:, h, :], scale)
    return o, lse


def merge(parts):
    """Join partial results [(o_i, lse_i)] over disjoint key sets into the
    result over their union: lse = log sum_i exp(lse_i),
    o = sum_i exp(lse_i - lse) o_i. Parts with lse = -inf (empty sets) add
    nothing."""
    lses = np.array([p[1] for p in parts], dtype=np.float64)
    if np.all(np.isneginf(lses)):
        return np.zeros_like(np.asarray(parts[0][0], np.float64)), -np.inf
    mx = lses.max()
    lse = mx + np.log(np.exp(lses - mx).sum())
    o = sum(np.exp(l - lse) * np.asarray(o_, np.float64)
            for o_, l in parts if not np.isneginf(l))
    return o, lse
