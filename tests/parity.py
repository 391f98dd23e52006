"""Comparison rules shared by the GPU parity tests.

Selections: the index sets must be equal, except that an index in the
symmetric difference is allowed when its oracle score lies within
1e-5 * max(|s_k|, 1e-30) of the oracle's k-th largest score s_k (a near-tie
that float32 scoring may order either way). Outputs: elementwise
|gpu - ref| <= atol + rtol * |ref|, with the reference computed by the oracle
on the GPU's own selection so that legitimate near-tie swaps do not fail it.
"""
import numpy as np
import torch

SEL_BAND = 1e-5
BF16_TOL = 2e-2
F32_TOL = 1e-4


def selection_ok(got, want, scores, k, band=SEL_BAND):
    """got/want: iterables of candidate indices; scores: oracle scores indexed
    by candidate index. Returns (ok, n_band_swaps)."""
    got, want = set(int(x) for x in got), set(int(x) for x in want)
    if len(got) != len(want):
        return False, 0
    diff = got ^ want
    if not diff:
        return True, 0
    sc = np.asarray(scores, np.float64)
    finite = sc[np.isfinite(sc)]
    s_k = np.sort(finite)[::-1][min(k, finite.size) - 1]
    tol = band * max(abs(s_k), 1e-30)
    for i in diff:
        if not abs(sc[i] - s_k) <= tol:
            return False, len(diff)
    return True, len(diff)


def moba_rows_ok(blk_gpu, blk_ref, scores_ref, rows, block, topk):
    """blk_* [len(rows), Hq, topk]; scores_ref [len(rows), Hq, nb]."""
    bad, swaps = [], 0
    for r, t in enumerate(rows):
        cur = t // block
        for h in range(blk_gpu.shape[1]):
            g = [int(b) for b in blk_gpu[r, h]]
            w = [int(b) for b in blk_ref[r, h]]
            # structure: ascending valid entries, current block last, -1 pad
            valid = [b for b in g if b >= 0]
            if valid != sorted(valid) or not valid or valid[-1] != cur or g[len(valid):] != [-1] * (topk - len(valid)):
                bad.append((t, h, g, w))
                continue
            ok, n = selection_ok(valid[:-1], [b for b in w if 0 <= b < cur], scores_ref[r, h], topk - 1)
            swaps += n
            if not ok:
                bad.append((t, h, g, w))
    return bad, swaps


def assert_close(got, ref, tol, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    lim = tol + tol * np.abs(ref)
    worst = np.max(err - lim) if err.size else -1
    if worst > 0:
        i = np.unravel_index(np.argmax(err - lim), err.shape)
        raise AssertionError(f"{what}: |gpu-ref| exceeds {tol}+{tol}|ref| at {i}: gpu={got[i]} ref={ref[i]} "
                             f"(max abs err {err.max():.3e})")


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()
