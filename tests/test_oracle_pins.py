"""Pins of the CPU oracle against things other than itself.

Each test ties one oracle function to a closed form, a special case that
reduces to a library routine (torch's float64 scaled_dot_product_attention,
numpy sorts, scipy's maximum filter, torch's bfloat16 cast), a brute-force
property check on tiny inputs, or a number printed on the source pages
(tests/golden/pages_numbers.json). No GPU is needed.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.ndimage as ndi
import torch
import torch.nn.functional as F

import oracle
import synth
from oracle import attention as oatt
from oracle import cca as occa
from oracle import esa as oesa
from oracle import moba as omoba
from oracle.numerics import round_to_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")


def rng(seed):
    return np.random.default_rng(seed)


def sdpa_causal(q, k, v, scale):
    """Library dense causal attention in float64. q [N,H,d], k/v [N,Hkv,d]
    (KV heads repeated contiguously for grouped queries)."""
    hq, hkv = q.shape[1], k.shape[1]
    rep = hq // hkv
    Q = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]
    K = torch.from_numpy(np.ascontiguousarray(np.repeat(k, rep, axis=1).transpose(1, 0, 2)))[None]
    V = torch.from_numpy(np.ascontiguousarray(np.repeat(v, rep, axis=1).transpose(1, 0, 2)))[None]
    o = F.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=scale)
    return o[0].numpy().transpose(1, 0, 2)


def sdpa_masked(q, k, v, mask, scale):
    """mask [H, N, N] boolean (True = attend)."""
    hq, hkv = q.shape[1], k.shape[1]
    rep = hq // hkv
    Q = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]
    K = torch.from_numpy(np.ascontiguousarray(np.repeat(k, rep, axis=1).transpose(1, 0, 2)))[None]
    V = torch.from_numpy(np.ascontiguousarray(np.repeat(v, rep, axis=1).transpose(1, 0, 2)))[None]
    o = F.scaled_dot_product_attention(Q, K, V, attn_mask=torch.from_numpy(mask)[None], scale=scale)
    return o[0].numpy().transpose(1, 0, 2)


# ------------------------------------------------------------------ generator
def test_generator_torch_matches_numpy_integer_stream():
    base = synth.gen.stream_base(7, 3)
    c = np.arange(1000, 6000, dtype=np.uint64)
    ref = synth.splitmix64_np(base, c).view(np.int64)
    t = torch.from_numpy(c.astype(np.int64))
    got = synth.gen._mix_t(synth.gen._signed(base) + (t + 1) * synth.gen._signed(synth.gen.GOLDEN))
    assert np.array_equal(ref, got.numpy())


def test_generator_known_splitmix_value():
    # splitmix64 of state 0 after one increment: first output of the
    # published generator seeded with 0 is 0xE220A8397B1DCDAF.
    assert int(synth.splitmix64_np(0, np.array([0], dtype=np.uint64))[0]) == 0xE220A8397B1DCDAF


def test_generator_rounded_outputs_agree_and_are_normal():
    a = synth.normal_np(11, 2, 200000, start=99)
    b = synth.normal(11, 2, (200000,), torch.float32, start=99).numpy().astype(np.float64)
    assert np.array_equal(a.astype(np.float32).astype(np.float64), b)
    assert abs(a.mean()) < 0.01 and abs(a.std() - 1) < 0.01


# ------------------------------------------------------------------ rounding
def test_round_to_bf16_matches_torch_on_f32_exact_values():
    x = rng(0).standard_normal(100000).astype(np.float32)
    # include exact ties at bf16 half-ulp
    ties = (np.arange(1, 2000, dtype=np.float32) * 2 + 1) * np.float32(2.0 ** -9) + 1
    x = np.concatenate([x, ties.astype(np.float32), -ties.astype(np.float32), [0.0]])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = round_to_bf16(x.astype(np.float64))
    assert np.array_equal(ref, got)


# ------------------------------------------------------------------ attention
def test_attend_matches_library_dense_causal():
    r = rng(1)
    N, H, d = 37, 3, 16
    q, k, v = (r.standard_normal((N, H, d)) for _ in range(3))
    ref = sdpa_causal(q, k, v, 0.3)
    for t in range(N):
        o, _ = oatt.attend_heads(q[t], k[:t + 1], v[:t + 1], 0.3)
        np.testing.assert_allclose(o, ref[t], rtol=1e-12, atol=1e-12)


def test_attend_closed_forms():
    r = rng(2)
    V = r.standard_normal((9, 5))
    q = r.standard_normal(4)
    K = np.tile(r.standard_normal(4), (9, 1))          # identical keys
    o, lse = oatt.attend(q, K, V, 0.7)
    np.testing.assert_allclose(o, V.mean(0), atol=1e-13)
    np.testing.assert_allclose(lse, 0.7 * K[0] @ q + math.log(9), atol=1e-12)
    o, lse = oatt.attend(q, r.standard_normal((9, 4)), V, 0.0)   # scale 0
    np.testing.assert_allclose(o, V.mean(0), atol=1e-13)
    np.testing.assert_allclose(lse, math.log(9), atol=1e-13)
    K = r.standard_normal((9, 4)) * 1e-3
    K[4] = q * 1e3                                      # one dominant key
    o, _ = oatt.attend(q, K, V, 1.0)
    np.testing.assert_allclose(o, V[4], atol=1e-12)
    o, lse = oatt.attend(q, np.zeros((0, 4)), V[:0], 1.0)
    assert np.isneginf(lse) and np.all(o == 0)


def test_merge_of_disjoint_splits_equals_union():
    r = rng(3)
    q = r.standard_normal(8)
    K = r.standard_normal((50, 8))
    V = r.standard_normal((50, 6))
    full = oatt.attend(q, K, V, 0.5)
    for trial in range(5):
        perm = r.permutation(50)
        cuts = sorted(r.choice(np.arange(1, 50), size=3, replace=False))
        parts = [oatt.attend(q, K[s], V[s], 0.5) for s in np.split(perm, cuts)]
        parts.append(oatt.attend(q, K[:0], V[:0], 0.5))   # an empty part
        o, lse = oatt.merge(parts)
        np.testing.assert_allclose(o, full[0], atol=1e-12)
        np.testing.assert_allclose(lse, full[1], atol=1e-12)


# ------------------------------------------------------------------ MoBA
def test_moba_block_means_closed_form():
    N, B = 40, 8
    k = np.zeros((N, 2, 3))
    for t in range(N):
        k[t, 0, :] = t // B            # constant per block
        k[t, 1, :] = t                 # arithmetic progression
    kb = omoba.block_means(k, B)
    for b in range(N // B):
        np.testing.assert_allclose(kb[b, 0], b)
        np.testing.assert_allclose(kb[b, 1], b * B + (B - 1) / 2)
    kb = omoba.block_means(k[:37], B)   # trailing partial block
    np.testing.assert_allclose(kb[4, 1], np.mean(np.arange(32, 37)))


def _moba_full(q, k, v, B, topk, scale, window=0):
    blk, sc, o, lse = omoba.forward(q, k, v, B, topk, scale, window)
    return blk, sc, o


@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 2)])
def test_moba_all_blocks_equals_dense_causal(hq, hkv):
    r = rng(4)
    N, d, B = 48, 8, 8
    q = r.standard_normal((N, hq, d))
    k = r.standard_normal((N, hkv, d))
    v = r.standard_normal((N, hkv, d))
    _, _, o = _moba_full(q, k, v, B, topk=N // B, scale=0.35)
    np.testing.assert_allclose(o, sdpa_causal(q, k, v, 0.35), atol=1e-12)


def test_moba_k1_equals_block_diagonal_causal():
    r = rng(5)
    N, H, d, B = 40, 2, 8, 8
    q, k, v = (r.standard_normal((N, H, d)) for _ in range(3))
    _, _, o = _moba_full(q, k, v, B, topk=1, scale=0.4)
    mask = np.zeros((H, N, N), dtype=bool)
    for t in range(N):
        mask[:, t, (t // B) * B:t + 1] = True
    np.testing.assert_allclose(o, sdpa_masked(q, k, v, mask, 0.4), atol=1e-12)


def test_moba_block1_equals_token_topk_bruteforce():
    r = rng(6)
    N, H, d, topk = 30, 2, 6, 4
    q, k, v = (r.standard_normal((N, H, d)) for _ in range(3))
    blk, _, o = _moba_full(q, k, v, 1, topk=topk, scale=0.5)
    mask = np.zeros((H, N, N), dtype=bool)
    for t in range(N):
        for h in range(H):
            s = [(-(q[t, h] @ k[j, h]), j) for j in range(t)]
            chosen = sorted(j for _, j in sorted(s)[:topk - 1]) + [t]
            got = [b for b in blk[t, h] if b >= 0]
            assert got == sorted(chosen)
            mask[h, t, chosen] = True
    np.testing.assert_allclose(o, sdpa_masked(q, k, v, mask, 0.5), atol=1e-12)


def test_moba_gqa_equals_mha_with_repeated_kv():
    r = rng(7)
    N, d, B = 32, 8, 4
    q = r.standard_normal((N, 6, d))
    k = r.standard_normal((N, 2, d))
    v = r.standard_normal((N, 2, d))
    blk_g, _, o_g = _moba_full(q, k, v, B, 3, 0.3)
    blk_m, _, o_m = _moba_full(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), B, 3, 0.3)
    assert np.array_equal(blk_g, blk_m)
    np.testing.assert_allclose(o_g, o_m, atol=1e-13)


def test_moba_selection_exhaustive_with_ties():
    """Every (k-1)-subset of the candidates is tried; the gated set must be
    the one whose members all beat every non-member on (score, -index)."""
    r = rng(8)
    N, H, d, B, topk = 24, 1, 4, 2, 4
    # small integer entries make exact score ties common
    q = r.integers(-1, 2, (N, H, d)).astype(np.float64)
    k = r.integers(-1, 2, (N, H, d)).astype(np.float64)
    kb = omoba.block_means(k, B)
    ties_seen = 0
    for t in range(N):
        cur = t // B
        blk, sc = omoba.select_row(q[t, 0], kb[:, 0], t, B, topk)
        s = [q[t, 0] @ kb[b, 0] for b in range(cur)]
        ties_seen += len(s) - len(set(s))
        want = None
        for sub in itertools.combinations(range(cur), min(topk - 1, cur)):
            rest = [b for b in range(cur) if b not in sub]
            if all((s[a] > s[b]) or (s[a] == s[b] and a < b) for a in sub for b in rest):
                assert want is None
                want = sorted(sub)
        want = sorted(want + [cur])
        assert [b for b in blk if b >= 0] == want
        assert list(blk[len(want):]) == [-1] * (topk - len(want))
        assert np.all(np.isneginf(sc[cur:]))
    assert ties_seen > 0


# ---- MoBA backward (gradients with the gating held fixed) -----------------
def _moba_bwd_case(seed, n=12, hq=2, hkv=1, d=3, block=4, topk=2):
    r = rng(seed)
    q, k, v = (r.standard_normal((n, h, d)) for h in (hq, hkv, hkv))
    rows = list(range(n))
    blk, _ = omoba.select(q, k, block, topk, rows)
    do = r.standard_normal((n, hq, d))
    return q, k, v, blk, rows, do


def test_moba_backward_matches_finite_differences():
    """L = sum_rows,heads do . o(q, k, v) with the gated sets fixed: the
    oracle's gradients equal central differences of the oracle forward."""
    q, k, v, blk, rows, do = _moba_bwd_case(50)
    scale, block = 0.6, 4

    def loss(q_, k_, v_):
        o, _ = omoba.attend_rows(q_, k_, v_, block, blk, rows, scale)
        return float(np.sum(o * do))

    dq, dk, dv = omoba.backward_rows(q, k, v, block, blk, rows, scale, do)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for i in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[i] += eps
            xm[i] -= eps
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            num[i] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        assert np.allclose(g, num, rtol=0, atol=2e-8), (name, np.abs(g - num).max())


def test_moba_backward_matches_torch_autograd_on_masked_dense():
    """Same gradients from torch autograd (float64, CPU) of a dense masked
    softmax attention whose mask is each row's MoBA key set, GQA by repeating
    the KV heads in the graph."""
    n, hq, hkv, d, block, topk = 40, 4, 2, 5, 8, 3
    q, k, v, blk, rows, do = _moba_bwd_case(51, n, hq, hkv, d, block, topk)
    scale = 0.45
    dq, dk, dv = omoba.backward_rows(q, k, v, block, blk, rows, scale, do)
    mask = np.full((hq, n, n), -np.inf)
    for t in rows:
        for h in range(hq):
            mask[h, t, omoba.key_set(blk[t, h], t, block)] = 0.0
    Q = torch.tensor(q, requires_grad=True)
    Kt = torch.tensor(k, requires_grad=True)
    Vt = torch.tensor(v, requires_grad=True)
    rep = hq // hkv
    Kr = Kt.repeat_interleave(rep, dim=1)
    Vr = Vt.repeat_interleave(rep, dim=1)
    s = torch.einsum("thd,jhd->htj", Q, Kr) * scale + torch.tensor(mask)
    o = torch.einsum("htj,jhd->thd", torch.softmax(s, dim=-1), Vr)
    o.backward(torch.tensor(do))
    assert np.allclose(dq, Q.grad.numpy(), atol=1e-12)
    assert np.allclose(dk, Kt.grad.numpy(), atol=1e-12)
    assert np.allclose(dv, Vt.grad.numpy(), atol=1e-12)


def test_esa_backward_matches_finite_differences():
    """ESA attention with the selection fixed: gradients equal central
    differences of the oracle forward (tiny chunk, all four parts present)."""
    r = rng(52)
    T, m, H, d = 30, 4, 2, 3
    q = r.standard_normal((m, H, d))
    K, V = r.standard_normal((T, H, d)), r.standard_normal((T, H, d))
    c0, n_init, W, scale = T - m, 3, 5, 0.7
    _, M, _ = oesa.partition(c0, n_init, W)
    sel = np.sort(r.choice(M, 6, replace=False))
    do = r.standard_normal((m, H, d))

    def loss(q_, K_, V_):
        o, _ = oesa.attend(q_, K_, V_, sel, c0, n_init, W, scale)
        return float(np.sum(o * do))

    dq, dK, dV = oesa.backward(q, K, V, sel, c0, n_init, W, scale, do)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", K, dK), ("v", V, dV)):
        num = np.zeros_like(x)
        for i in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[i] += eps
            xm[i] -= eps
            args_p = {"q": (xp, K, V), "k": (q, xp, V), "v": (q, K, xp)}[name]
            args_m = {"q": (xm, K, V), "k": (q, xm, V), "v": (q, K, xm)}[name]
            num[i] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        assert np.allclose(g, num, rtol=0, atol=2e-8), (name, np.abs(g - num).max())
    # keys outside the four parts get no gradient
    outside = np.setdiff1d(np.arange(T), np.concatenate([np.arange(n_init), sel, np.arange(c0 - W, T)]))
    assert np.all(dK[outside] == 0) and np.all(dV[outside] == 0)


def test_esa_backward_matches_torch_autograd_on_masked_dense():
    r = rng(53)
    T, m, H, d = 60, 8, 3, 4
    q = r.standard_normal((m, H, d))
    K, V = r.standard_normal((T, H, d)), r.standard_normal((T, H, d))
    c0, n_init, W, scale = T - m, 4, 10, 0.5
    _, M, _ = oesa.partition(c0, n_init, W)
    sel = np.sort(r.choice(M, 12, replace=False))
    do = r.standard_normal((m, H, d))
    dq, dK, dV = oesa.backward(q, K, V, sel, c0, n_init, W, scale, do)
    mask = np.full((m, T), -np.inf)
    for i in range(m):
        mask[i, oesa.key_list(sel, c0, n_init, W, c0 + i)] = 0.0
    Q, Kt, Vt = (torch.tensor(x, requires_grad=True) for x in (q, K, V))
    s = torch.einsum("ihd,jhd->hij", Q, Kt) * scale + torch.tensor(mask)[None]
    o = torch.einsum("hij,jhd->ihd", torch.softmax(s, dim=-1), Vt)
    o.backward(torch.tensor(do))
    assert np.allclose(dq, Q.grad.numpy(), atol=1e-12)
    assert np.allclose(dK, Kt.grad.numpy(), atol=1e-12)
    assert np.allclose(dV, Vt.grad.numpy(), atol=1e-12)


# ---- CCA-style core-token attention --------------------------------------
def _cca_case(seed, n=40, hq=2, hkv=1, d=4):
    r = rng(seed)
    return r.standard_normal((n, hq, d)), r.standard_normal((n, hkv, d)), r.standard_normal((n, hkv, d))


@pytest.mark.parametrize("w", [0, 3, 10])
def test_cca_group1_equals_dense_causal(w):
    """g = 1: a group's core token is the token itself, so the core tokens
    plus the window are all earlier tokens."""
    q, k, v = _cca_case(60)
    kc, vc = occa.pool(q, k, v, 1, 0.5)
    rows = list(range(40))
    o, lse = occa.attend_rows(q, k, v, kc, vc, 1, w, 0.5, rows)
    for t in rows:
        for h in range(2):
            o_ref, l_ref = oatt.attend(q[t, h], k[:t + 1, 0], v[:t + 1, 0], 0.5)
            assert np.allclose(o[t, h], o_ref, atol=1e-12) and abs(lse[t, h] - l_ref) < 1e-12


def test_cca_wide_window_equals_dense_causal():
    q, k, v = _cca_case(61)
    kc, vc = occa.pool(q, k, v, 4, 0.3)
    o, _ = occa.attend_rows(q, k, v, kc, vc, 4, 64, 0.3, list(range(40)))
    for t in range(40):
        o_ref, _ = oatt.attend(q[t, 1], k[:t + 1, 0], v[:t + 1, 0], 0.3)
        assert np.allclose(o[t, 1], o_ref, atol=1e-12)


def test_cca_pool_closed_forms():
    """Identical keys in a group: the core key is that key and the core value
    the group's mean value; the core depends on the group's last query only."""
    q, k, v = _cca_case(62, n=16, hq=1)
    k[4:8, 0] = k[4, 0]
    kc, vc = occa.pool(q, k, v, 4, 0.7)
    assert np.allclose(kc[1, 0], k[4, 0], atol=1e-14)
    assert np.allclose(vc[1, 0], v[4:8, 0].mean(axis=0), atol=1e-14)
    q2 = q.copy()
    q2[8:11] += 5.0        # not the last query of group 2
    kc2, _ = occa.pool(q2, k, v, 4, 0.7)
    assert np.array_equal(kc2, kc)
    q2[11] += 1.0          # the last query of group 2
    kc3, _ = occa.pool(q2, k, v, 4, 0.7)
    assert not np.allclose(kc3[2], kc[2])


def test_cca_window_is_group_aligned_and_long_enough():
    for g in (1, 3, 4, 16):
        for w in (0, 1, 5, 16, 33):
            for t in range(200):
                ls = occa.window_start(t, g, w)
                assert ls % g == 0 and 0 <= ls <= t
                assert t - ls >= min(t, w)


def _window_start_by_search(t, g, w):
    """The window start found by search from the locality module's two
    requirements alone: it is a group boundary, every query of t's group sees
    at least min(t', w) earlier raw tokens from it, and no later boundary
    would do (the window is the shortest such one, shared by the group)."""
    grp0 = (t // g) * g
    members = range(grp0, grp0 + g)
    best = None
    for s in range(0, grp0 + 1, g):
        if all(tp - s >= min(tp, w) for tp in members):
            best = s
    return best


def test_cca_window_start_is_the_latest_boundary_that_keeps_w_tokens():
    """Pins window_start itself: a window one group wider (or narrower) than
    the shortest group-aligned one with >= w tokens for every query of the
    group fails here."""
    for g in (1, 2, 3, 4, 16):
        for w in (0, 1, 2, 5, 16, 17, 33):
            for t in range(160):
                assert occa.window_start(t, g, w) == _window_start_by_search(t, g, w), (t, g, w)


def test_cca_rows_attend_the_enumerated_key_set():
    """attend_rows against attention over a key set enumerated position by
    position: the core token of every complete group that lies wholly before
    the searched window start, then every raw token from that start to t."""
    q, k, v = _cca_case(63, n=48, hq=2, hkv=1)
    g, w, scale = 4, 6, 0.4
    kc, vc = occa.pool(q, k, v, g, scale)
    rows = list(range(48))
    o, lse = occa.attend_rows(q, k, v, kc, vc, g, w, scale, rows)
    for t in rows:
        s = _window_start_by_search(t, g, w)
        cores = [i for i in range(48 // g) if (i + 1) * g <= s]
        raw = [j for j in range(48) if s <= j <= t]
        for h in range(2):
            K = np.array([kc[i, h] for i in cores] + [k[j, 0] for j in raw]).reshape(-1, k.shape[2])
            V = np.array([vc[i, h] for i in cores] + [v[j, 0] for j in raw]).reshape(-1, v.shape[2])
            o_ref, l_ref = oatt.attend(q[t, h], K, V, scale)
            assert np.allclose(o[t, h], o_ref, atol=1e-12) and abs(lse[t, h] - l_ref) < 1e-12


def test_cca_gqa_equals_mha_with_repeated_kv():
    """Hq = 4 query heads over Hkv = 2 KV heads: heads 0, 1 use KV head 0 and
    heads 2, 3 KV head 1 (contiguous groups), so the result equals the
    one-KV-head-per-query-head case with each KV head repeated in place."""
    q, k, v = _cca_case(64, n=40, hq=4, hkv=2)
    g, w, scale = 4, 5, 0.35
    kr, vr = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)
    kc, vc = occa.pool(q, k, v, g, scale)
    kc_r, vc_r = occa.pool(q, kr, vr, g, scale)
    assert np.allclose(kc, kc_r, atol=1e-14) and np.allclose(vc, vc_r, atol=1e-14)
    rows = list(range(40))
    o, lse = occa.attend_rows(q, k, v, kc, vc, g, w, scale, rows)
    o_r, lse_r = occa.attend_rows(q, kr, vr, kc_r, vc_r, g, w, scale, rows)
    assert np.allclose(o, o_r, atol=1e-13) and np.allclose(lse, lse_r, atol=1e-13)
    # the interleaved map (head h -> KV head h % Hkv) gives a different result
    ki, vi = np.tile(k, (1, 2, 1)), np.tile(v, (1, 2, 1))
    kc_i, vc_i = occa.pool(q, ki, vi, g, scale)
    assert not np.allclose(kc, kc_i)


def test_moba_is_causal():
    r = rng(9)
    N, H, d, B = 32, 2, 8, 4
    q, k, v = (r.standard_normal((N, H, d)) for _ in range(3))
    _, _, o1 = _moba_full(q, k, v, B, 3, 0.3)
    k2, v2 = k.copy(), v.copy()
    k2[20:] = r.standard_normal(k2[20:].shape)
    v2[20:] = r.standard_normal(v2[20:].shape)
    _, _, o2 = _moba_full(q, k2, v2, B, 3, 0.3)
    np.testing.assert_array_equal(o1[:20], o2[:20])


def test_moba_window_adds_local_keys_once():
    r = rng(10)
    N, H, d, B, w = 24, 1, 4, 8, 5
    q, k, v = (r.standard_normal((N, H, d)) for _ in range(3))
    blk, _, o = _moba_full(q, k, v, B, 2, 0.5, window=w)
    for t in range(N):
        keys = omoba.key_set(blk[t, 0], t, B, w)
        assert len(keys) == len(set(keys.tolist()))
        want = set(range((t // B) * B, t + 1)) | set(range(max(0, t - w + 1), t + 1))
        for b in blk[t, 0]:
            if 0 <= b < t // B:
                want |= set(range(b * B, (b + 1) * B))
        assert set(keys.tolist()) == want


def test_moba_sparsity_matches_page():
    g = json.load(open(GOLDEN))["moba_fixed_sparsity"]
    nb, topk = g["shape"]["n_blocks"], g["shape"]["topk"]
    # a late query of a 64-block sequence gates exactly topk blocks
    r = rng(11)
    B = 2
    q = r.standard_normal((nb * B, 1, 4))
    k = r.standard_normal((nb * B, 1, 4))
    blk, _ = omoba.select(q, k, B, topk, rows=[nb * B - 1])
    attended = int((blk[0, 0] >= 0).sum())
    assert attended == topk
    assert abs((1 - attended / nb) - g["value"]) <= g["abs_tol"]
    assert abs(oracle.cost.moba_sparsity(nb, topk) - g["value"]) <= g["abs_tol"]


# ------------------------------------------------------------------ ESA
def test_esa_partition_covers_prefix_disjointly():
    for c0, n_init, W in [(0, 4, 8), (3, 4, 8), (10, 4, 8), (13, 4, 8), (100, 4, 8), (63488, 128, 4096)]:
        I, M, L = oesa.partition(c0, n_init, W)
        allp = np.concatenate([I, M, L])
        assert np.array_equal(np.sort(allp), np.arange(c0))
        assert len(L) <= W
    I, M, L = oesa.partition(63488, 128, 4096)
    assert (len(I), len(M), len(L)) == (128, 59264, 4096)
    I, M, L = oesa.partition(131071, 128, 4096)
    assert len(M) == 126847 and len(I) + 2048 + len(L) + 1 == 6273


def test_esa_compress_concatenates_heads_in_order():
    r = rng(12)
    H, d, d_c = 3, 4, 5
    x = r.standard_normal((7, H, d))
    W = np.zeros((d_c, H * d))
    picks = [(0, 1), (2, 3), (1, 0), (2, 0), (0, 3)]
    for c, (h, j) in enumerate(picks):
        W[c, h * d + j] = 1.0
    out = oesa.compress(x.reshape(7, -1), W, np.arange(d_c, dtype=np.float64))
    for c, (h, j) in enumerate(picks):
        np.testing.assert_array_equal(out[:, c], x[:, h, j] + c)


def test_esa_key_cache_is_rounded_compression():
    r = rng(13)
    k = r.standard_normal((20, 2, 4)).astype(np.float32).astype(np.float64)
    W = np.eye(3, 8)                      # picks exact float32 values
    kc = oesa.key_cache(k, W)
    ref = torch.from_numpy(k.reshape(20, 8)[:, :3].astype(np.float32)).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(kc, ref)


def test_esa_neighbour_matches_library_filter():
    r = rng(14)
    for n, rad in [(1, 2), (2, 2), (7, 0), (50, 1), (50, 2), (50, 7), (5, 9)]:
        u = r.integers(-5, 5, n).astype(np.float64)
        ref = ndi.maximum_filter1d(u, size=2 * rad + 1, mode="constant", cval=-np.inf)
        np.testing.assert_array_equal(oesa.neighbour(u, rad), ref)


def test_esa_topk_exhaustive_with_ties():
    r = rng(15)
    for trial in range(30):
        n = int(r.integers(1, 9))
        k = int(r.integers(1, 10))
        s = r.integers(-2, 3, n).astype(np.float64)
        got = oesa.top_k(s, k)
        kk = min(k, n)
        wants = [sorted(sub) for sub in itertools.combinations(range(n), kk)
                 if all((s[a] > s[b]) or (s[a] == s[b] and a < b)
                        for a in sub for b in range(n) if b not in sub)]
        assert len(wants) == 1 and list(got) == wants[0]


def test_esa_no_clip_no_radius_reduces_to_summed_query():
    """clip = inf, r = 0: u_j = <sum_i q~_i, k~_j> - const, so the selection is
    a sort of one matrix-vector product."""
    r = rng(16)
    m, H, d, T, d_c = 6, 2, 8, 90, 5
    q = r.standard_normal((m, H, d))
    Wq = r.standard_normal((d_c, H * d))
    kc = round_to_bf16(r.standard_normal((T, d_c)))
    c0, n_init, W, topk = 84, 4, 10, 9
    sel, up, u, _ = oesa.select(q, Wq, None, kc, c0, n_init, W, topk, radius=0, clip=np.inf)
    _, M, _ = oesa.partition(c0, n_init, W)
    qsum = (q.reshape(m, -1) @ Wq.T).sum(0)
    score = kc[M] @ qsum
    want = np.sort(M[np.argsort(-score, kind="stable")[:topk]])
    assert np.array_equal(sel, want)


def test_esa_zero_clip_gives_all_ties_lowest_positions():
    r = rng(17)
    q = r.standard_normal((3, 2, 4))
    kc = r.standard_normal((60, 5))
    Wq = r.standard_normal((5, 8))
    sel, up, _, _ = oesa.select(q, Wq, None, kc, 55, 3, 6, 7, radius=2, clip=0.0)
    assert np.all(up == 0)
    assert np.array_equal(sel, np.arange(3, 10))


def test_esa_decode_monotone_correction_keeps_raw_ranking():
    r = rng(18)
    T, H, d, d_c = 300, 2, 4, 6
    q = r.standard_normal((1, H, d))
    Wq = r.standard_normal((d_c, H * d))
    kc = round_to_bf16(r.standard_normal((T, d_c)))
    c0 = T - 1
    sel, _, _, _ = oesa.select(q, Wq, None, kc, c0, 5, 20, 12, radius=0, clip=1e9)
    _, M, _ = oesa.partition(c0, 5, 20)
    raw = kc[M] @ (q.reshape(1, -1) @ Wq.T)[0]
    assert np.array_equal(sel, np.sort(M[np.argsort(-raw, kind="stable")[:12]]))


# ---- per-head selection (the head-merging ablation's other arm) ----------
def test_esa_per_head_single_head_is_merged_with_identity_map():
    """H = 1 with the identity as compression map (d_c = d, k bf16 so the
    rounded cache is k itself): per-head selection = the merged selection,
    for both correction readings."""
    r = rng(60)
    T, d, m = 160, 8, 5
    q = round_to_bf16(r.standard_normal((m, 1, d)))
    k = round_to_bf16(r.standard_normal((T, 1, d)))
    eye = np.eye(d)
    kc = oesa.key_cache(k, eye)
    assert np.array_equal(kc, k[:, 0])
    c0, n_init, W = T - m, 6, 20
    for corr in ("clamp", "votes"):
        sel, up, _, _ = oesa.select(q, eye, None, kc, c0, n_init, W, 9, radius=1, clip=2.5, correction=corr)
        sels, ups = oesa.select_heads(q, k, c0, n_init, W, 9, radius=1, clip=2.5, correction=corr)
        assert len(sels) == 1
        assert np.array_equal(sels[0], sel)
        np.testing.assert_allclose(ups[0], up, rtol=1e-12, atol=1e-12)


def test_esa_per_head_planted_needles_are_per_head():
    """Head h's queries all point along a_h and head h's key at p_h is
    3 a_h (other heads' keys at p_h are noise): with top-1 and radius 0,
    head h selects exactly p_h -- a transposed head index selects another
    head's needle."""
    r = rng(61)
    T, H, d, m = 200, 4, 16, 3
    k = 0.1 * r.standard_normal((T, H, d))
    q = np.zeros((m, H, d))
    pos = [30, 77, 101, 140]
    for h in range(H):
        a = r.standard_normal(d)
        a /= np.linalg.norm(a)
        q[:, h] = a
        k[pos[h], h] = 3 * a
    sels, _ = oesa.select_heads(q, k, T - m, 4, 16, 1, radius=0, clip=48.0)
    assert [list(s) for s in sels] == [[p] for p in pos]


def test_esa_per_head_heads_are_independent():
    """Changing one head's keys leaves the other heads' selections alone, and
    head h's selection is the single-head selection of its own slice."""
    r = rng(62)
    T, H, d, m = 180, 3, 8, 4
    q = r.standard_normal((m, H, d))
    k = r.standard_normal((T, H, d))
    args = (T - m, 5, 24, 11)
    sels, _ = oesa.select_heads(q, k, *args, radius=2, clip=3.0)
    k2 = k.copy()
    k2[:, 2] = r.standard_normal((T, d))
    sels2, _ = oesa.select_heads(q, k2, *args, radius=2, clip=3.0)
    assert np.array_equal(sels[0], sels2[0]) and np.array_equal(sels[1], sels2[1])
    for h in range(H):
        one, _ = oesa.select_heads(q[:, h:h + 1], k[:, h:h + 1], *args, radius=2, clip=3.0)
        assert np.array_equal(one[0], sels[h])


def test_esa_per_head_attention_reduces_to_shared_and_single_head():
    """Per-head lists that are all equal give the shared-selection attention;
    with different lists, head h's output is the single-head attention over
    its own list. Gradients reduce the same way."""
    r = rng(63)
    T, H, d, m = 120, 3, 8, 5
    c0, n_init, W, scale = T - m, 4, 12, 0.35
    q = r.standard_normal((m, H, d))
    K = r.standard_normal((T, H, d))
    V = r.standard_normal((T, H, d))
    _, M, _ = oesa.partition(c0, n_init, W)
    shared = np.sort(r.choice(M, 9, replace=False))
    o1, l1 = oesa.attend(q, K, V, shared, c0, n_init, W, scale)
    o2, l2 = oesa.attend(q, K, V, [shared] * H, c0, n_init, W, scale)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=1e-12, atol=1e-12)
    sels = [np.sort(r.choice(M, 9, replace=False)) for _ in range(H)]
    o, lse = oesa.attend(q, K, V, sels, c0, n_init, W, scale)
    do = r.standard_normal((m, H, d))
    dq, dK, dV = oesa.backward(q, K, V, sels, c0, n_init, W, scale, do)
    for h in range(H):
        sl = slice(h, h + 1)
        oh, lh = oesa.attend(q[:, sl], K[:, sl], V[:, sl], sels[h], c0, n_init, W, scale)
        np.testing.assert_allclose(o[:, sl], oh, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[:, sl], lh, rtol=1e-12, atol=1e-12)
        gq, gK, gV = oesa.backward(q[:, sl], K[:, sl], V[:, sl], sels[h], c0, n_init, W, scale, do[:, sl])
        np.testing.assert_allclose(dq[:, sl], gq, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dK[:, sl], gK, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dV[:, sl], gV, rtol=1e-12, atol=1e-12)


# ---- alternative correction reading: per-query softmax votes -------------
def _votes_case(seed, m, n_mid, d_c=6):
    r = rng(seed)
    return r.standard_normal((m, d_c)), round_to_bf16(r.standard_normal((n_mid, d_c)))


def test_esa_votes_each_query_casts_one_vote():
    """Every query's votes sum to 1, so the importances sum to m."""
    qc, kc = _votes_case(40, 7, 50)
    for tau in (None, 0.3, 2.0):
        u, _ = oesa.importance(qc, kc, np.inf, correction="votes", tau=tau)
        assert abs(u.sum() - 7) < 1e-12
        assert np.all(u > 0)


def test_esa_votes_two_tokens_are_logistic():
    """One query, two middle tokens: the votes are sigma(+-tau (s0 - s1))."""
    qc, kc = _votes_case(41, 1, 2)
    tau = 0.7
    s = kc @ qc[0]
    u, _ = oesa.importance(qc, kc, np.inf, correction="votes", tau=tau)
    want0 = 1.0 / (1.0 + math.exp(-tau * (s[0] - s[1])))
    assert abs(u[0] - want0) < 1e-14 and abs(u[1] - (1.0 - want0)) < 1e-14


def test_esa_votes_temperature_limits():
    """tau -> 0: every token gets m / n_M; tau -> inf: each query's whole vote
    goes to its own arg-max token (brute-force count)."""
    m, n_mid = 9, 40
    qc, kc = _votes_case(42, m, n_mid)
    u0, _ = oesa.importance(qc, kc, np.inf, correction="votes", tau=1e-13)
    assert np.allclose(u0, m / n_mid, rtol=0, atol=1e-9)
    uinf, _ = oesa.importance(qc, kc, np.inf, correction="votes", tau=1e6)
    counts = np.zeros(n_mid)
    for i in range(m):
        best = max(range(n_mid), key=lambda j: (float(np.dot(qc[i], kc[j])), -j))
        counts[best] += 1
    assert np.allclose(uinf, counts, rtol=0, atol=1e-9)


def test_esa_votes_default_temperature_is_inverse_sqrt_width():
    qc, kc = _votes_case(43, 3, 20, d_c=16)
    a, _ = oesa.importance(qc, kc, np.inf, correction="votes")
    b, _ = oesa.importance(qc, kc, np.inf, correction="votes", tau=0.25)
    assert np.allclose(a, b, rtol=1e-14, atol=0)


def test_esa_votes_decode_keeps_raw_ranking():
    """One query: the votes are a monotone map of the raw scores, so the
    selection (radius 0) is the raw-score top-k."""
    r = rng(44)
    T, H, d, d_c = 300, 2, 4, 6
    q = r.standard_normal((1, H, d))
    Wq = r.standard_normal((d_c, H * d))
    kc = round_to_bf16(r.standard_normal((T, d_c)))
    c0 = T - 1
    sel, _, _, _ = oesa.select(q, Wq, None, kc, c0, 5, 20, 12, radius=0, clip=1.0, correction="votes")
    _, M, _ = oesa.partition(c0, 5, 20)
    raw = kc[M] @ (q.reshape(1, -1) @ Wq.T)[0]
    assert np.array_equal(sel, np.sort(M[np.argsort(-raw, kind="stable")[:12]]))


def test_esa_votes_differ_from_clamp_in_prefill():
    """Several queries: the two readings rank differently in general (a query
    with one dominant token gives it a vote near 1 under votes, but only its
    own clamp range under the clamp)."""
    r = rng(45)
    m, H, d, d_c, T = 16, 2, 8, 8, 400
    q = r.standard_normal((m, H, d))
    Wq = r.standard_normal((d_c, H * d)) / 4
    kc = round_to_bf16(r.standard_normal((T, d_c)))
    c0 = T - m
    a, _, _, _ = oesa.select(q, Wq, None, kc, c0, 4, 32, 40, radius=0, clip=5.0)
    b, _, _, _ = oesa.select(q, Wq, None, kc, c0, 4, 32, 40, radius=0, clip=5.0, correction="votes")
    assert not np.array_equal(a, b)


def test_esa_radius_lifts_neighbours_of_a_peak():
    u = np.zeros(20)
    u[7] = 5.0
    up = oesa.neighbour(u, 2)
    assert np.array_equal(np.nonzero(up == 5.0)[0], np.arange(5, 10))
    # top-5 then picks the whole segment around the peak
    assert np.array_equal(oesa.top_k(up, 5), np.arange(5, 10))


@pytest.mark.parametrize("c0,m", [(40, 8), (5, 6), (0, 4)])
def test_esa_full_selection_equals_dense_causal(c0, m):
    r = rng(19)
    H, d, d_c = 2, 8, 4
    T = c0 + m
    q_all = r.standard_normal((T, H, d))
    k = r.standard_normal((T, H, d))
    v = r.standard_normal((T, H, d))
    Wq = r.standard_normal((d_c, H * d))
    kc = round_to_bf16(r.standard_normal((T, d_c)))
    n_init, W = 3, 5
    q = q_all[c0:]
    sel, _, _, _ = oesa.select(q, Wq, None, kc, c0, n_init, W, topk=10 ** 6, radius=1, clip=3.0)
    _, M, _ = oesa.partition(c0, n_init, W)
    assert np.array_equal(sel, M)
    o, _ = oesa.attend(q, k, v, sel, c0, n_init, W, 0.3)
    ref = sdpa_causal(q_all, k, v, 0.3)[c0:]
    np.testing.assert_allclose(o, ref, atol=1e-12)


def test_esa_parts_are_one_joint_softmax():
    """Attention over I u S u L u chunk equals the merge of the global part
    (I u S) and the window part (L u chunk)."""
    r = rng(20)
    T, H, d = 60, 2, 4
    k, v = r.standard_normal((T, H, d)), r.standard_normal((T, H, d))
    c0, n_init, W = 50, 4, 8
    q = r.standard_normal((10, H, d))
    sel = np.array([6, 9, 20, 33])
    o, lse = oesa.attend(q, k, v, sel, c0, n_init, W, 0.4)
    I, _, L = oesa.partition(c0, n_init, W)
    for i in range(10):
        g = np.concatenate([I, sel])
        w = np.concatenate([L, np.arange(c0, c0 + i + 1)])
        for h in range(H):
            pg = oatt.attend(q[i, h], k[g, h], v[g, h], 0.4)
            pw = oatt.attend(q[i, h], k[w, h], v[w, h], 0.4)
            oo, ll = oatt.merge([pg, pw])
            np.testing.assert_allclose(oo, o[i, h], atol=1e-12)
            np.testing.assert_allclose(ll, lse[i, h], atol=1e-12)


def test_esa_needles_are_selected_in_decode():
    """Planted needles (keys equal to the decode query in every head) win
    the compressed scoring under the unit-variance random compression; each
    lifts its +-r neighbours onto the same plateau."""
    T, H, d, d_c = 4096, 8, 32, 64
    seed = 4
    q, k, v, info = synth.esa_inputs(seed, 1, T, 1, H, d, torch.float32, needles=6,
                                     needle_lo=64, needle_hi=T - 1 - 512, needle_gap=5,
                                     needle_scale=1.0)
    Wq = synth.compression_weights(seed, d_c, H * d, dtype=torch.float32).double().numpy()
    kc = oesa.key_cache(k[0].double().numpy(), Wq)
    sel, _, _, _ = oesa.select(q[0].double().numpy(), Wq, None, kc, T - 1, 64, 512, 128, 2, 48.0)
    for p in info["needles"][0]:
        assert set(range(p - 2, p + 3)) <= set(sel.tolist())


def test_esa_step_ratio_matches_page():
    g = json.load(open(GOLDEN))
    e = g["esa_step_ratio_long_sequence"]
    s = e["shape"]
    ratio = oracle.cost.esa_step_ratio(s["T"], s["D"], s["d_c"], s["n_init"], s["k_sel"], s["window"])
    assert abs(ratio - e["value"]) <= e["abs_tol"]
    c = g["esa_compression_ratio"]
    assert abs(c["shape"]["d_c"] / c["shape"]["D"] - c["value"]) <= c["abs_tol"]
    # the ratio falls with T towards d_c / (2 D)
    assert oracle.cost.esa_step_ratio(2 ** 17) > oracle.cost.esa_step_ratio(2 ** 20) > 128 / 8192
