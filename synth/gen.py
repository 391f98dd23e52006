"""Counter-based normal generator and the workload recipes.

Generator (one definition, two implementations that must agree bit for bit):

* splitmix64 finaliser (Steele, Lea and Flood, "Fast splittable pseudorandom
  number generators", OOPSLA 2014; the 64-bit constants are the published
  ones) applied to ``base + (c + 1) * GOLDEN`` where ``c`` is a counter and
  ``base`` mixes the seed and a tensor id;
* two 53-bit uniforms per element (counters ``2i`` and ``2i + 1``),
  ``u = (x >> 11) * 2**-53 + 2**-54`` so that ``u`` lies in (0, 1);
* Box-Muller, cosine branch only: ``z = sqrt(-2 ln u1) * cos(2 pi u2)``,
  evaluated in float64 and rounded once to the target dtype (round to
  nearest even, as torch's casts do).

``normal_np`` is the numpy/uint64 reference of the integer part; ``normal``
runs the same steps in torch int64 (with masked logical shifts) on any
device, chunked so that tensors of many GB can be generated in place on the
GPU. A CPU test checks that both agree.
"""
from __future__ import annotations

import math

import numpy as np
import torch

GOLDEN = 0x9E3779B97F4A7C15
M1 = 0xBF58476D1CE4E5B9
M2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1

# tensor ids
TID_Q, TID_K, TID_V, TID_W, TID_STRUCT, TID_WK = 1, 2, 3, 4, 5, 6


def _signed(x: int) -> int:
    x &= MASK64
    return x - (1 << 64) if x >= (1 << 63) else x


def _mix_py(z: int) -> int:
    z &= MASK64
    z = ((z ^ (z >> 30)) * M1) & MASK64
    z = ((z ^ (z >> 27)) * M2) & MASK64
    return z ^ (z >> 31)


def stream_base(seed: int, tensor_id: int) -> int:
    """64-bit stream key for (seed, tensor id)."""
    return _mix_py((seed & 0xFFFFFFFF) << 32 ^ (tensor_id & 0xFFFF) << 8 ^ 0x5EED)


# ---------------------------------------------------------------- numpy path
def splitmix64_np(base: int, counters: np.ndarray) -> np.ndarray:
    c = counters.astype(np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(base) + (c + np.uint64(1)) * np.uint64(GOLDEN)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(M1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(M2)
        z = z ^ (z >> np.uint64(31))
    return z


def normal_np(seed: int, tensor_id: int, n: int, start: int = 0) -> np.ndarray:
    """float64 N(0,1) draws for flat indices [start, start + n)."""
    base = stream_base(seed, tensor_id)
    idx = np.arange(start, start + n, dtype=np.uint64)
    x1 = splitmix64_np(base, idx * np.uint64(2))
    x2 = splitmix64_np(base, idx * np.uint64(2) + np.uint64(1))
    u1 = (x1 >> np.uint64(11)).astype(np.float64) * 2.0 ** -53 + 2.0 ** -54
    u2 = (x2 >> np.uint64(11)).astype(np.float64) * 2.0 ** -53 + 2.0 ** -54
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)


# ---------------------------------------------------------------- torch path
def _lsr(x: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of int64 bit patterns."""
    return (x >> s) & ((1 << (64 - s)) - 1)


def _mix_t(z: torch.Tensor) -> torch.Tensor:
    z = (z ^ _lsr(z, 30)) * _signed(M1)
    z = (z ^ _lsr(z, 27)) * _signed(M2)
    return z ^ _lsr(z, 31)


def _normal_chunk(base: int, start: int, n: int, device) -> torch.Tensor:
    idx = torch.arange(start, start + n, dtype=torch.int64, device=device)
    c1 = idx * 2
    z1 = _mix_t(_signed(base) + (c1 + 1) * _signed(GOLDEN))
    z2 = _mix_t(_signed(base) + (c1 + 2) * _signed(GOLDEN))
    del idx, c1
    u1 = _lsr(z1, 11).to(torch.float64) * 2.0 ** -53 + 2.0 ** -54
    del z1
    u2 = _lsr(z2, 11).to(torch.float64) * 2.0 ** -53 + 2.0 ** -54
    del z2
    return torch.sqrt(-2.0 * torch.log(u1)) * torch.cos((2.0 * math.pi) * u2)


def normal(seed: int, tensor_id: int, shape, dtype=torch.bfloat16,
           device="cpu", start: int = 0, scale: float = 1.0,
           chunk: int = 1 << 25) -> torch.Tensor:
    """N(0,1)*scale draws laid out row-major in ``shape``; flat index i of the
    result uses counter ``start + i``. Rounded once from float64."""
    numel = int(np.prod(shape)) if len(shape) else 1
    out = torch.empty(numel, dtype=dtype, device=device)
    for s in range(0, numel, chunk):
        n = min(chunk, numel - s)
        z = _normal_chunk(stream_base(seed, tensor_id), start + s, n, device)
        if scale != 1.0:
            z = z * scale
        out[s:s + n] = z.to(dtype)
        del z
    return out.view(*shape)


# ---------------------------------------------------------------- structure
def _uniform_ints(seed: int, tensor_id: int, count: int, hi: int) -> list[int]:
    base = stream_base(seed, tensor_id)
    x = splitmix64_np(base, np.arange(count, dtype=np.uint64))
    return [int(v % np.uint64(hi)) for v in x]


def planted_block_ids(seed: int, n_planted: int, n_choices: int) -> list[int]:
    """Distinct block ids drawn from [0, n_choices), in draw order."""
    out: list[int] = []
    c = 0
    base = stream_base(seed, TID_STRUCT)
    while len(out) < n_planted:
        v = int(splitmix64_np(base, np.array([c], dtype=np.uint64))[0] % np.uint64(n_choices))
        c += 1
        if v not in out:
            out.append(v)
    return out


def needle_positions(seed: int, batch_index: int, n_needles: int, lo: int,
                     hi: int, min_gap: int) -> list[int]:
    """Sorted positions in [lo, hi) with pairwise distance > min_gap."""
    out: list[int] = []
    c = 0
    base = stream_base(seed * 1000 + batch_index, TID_STRUCT)
    while len(out) < n_needles:
        v = lo + int(splitmix64_np(base, np.array([c], dtype=np.uint64))[0] % np.uint64(hi - lo))
        c += 1
        if all(abs(v - p) > min_gap for p in out):
            out.append(v)
    return sorted(out)


# ---------------------------------------------------------------- workloads
def moba_inputs(seed: int, batch: int, n: int, hq: int, hkv: int, d: int,
                dtype=torch.bfloat16, device="cpu", planted: int = 0,
                block: int = 0, plant_noise: float = 0.25):
    """q [batch,n,hq,d], k,v [batch,n,hkv,d] i.i.d. N(0,1).

    With ``planted`` > 0, that many distinct key blocks (ids drawn from
    [0, n/block - 1), so never the last block) are overwritten, for every KV
    head g, by c_{b,g} + plant_noise * z, where c_{b,g} ~ N(0, I) is one
    vector per (block, head): the block mean is then close to c_{b,g}, whose
    norm is about sqrt(d), so those blocks win the block scoring whenever
    <q, c> > 0.
    """
    q = normal(seed, TID_Q, (batch, n, hq, d), dtype, device)
    k = normal(seed, TID_K, (batch, n, hkv, d), dtype, device)
    v = normal(seed, TID_V, (batch, n, hkv, d), dtype, device)
    info = {}
    if planted:
        nb = n // block
        ids = planted_block_ids(seed, planted, nb - 1)
        info["planted_blocks"] = ids
        for r, b in enumerate(ids):
            centre = normal(seed, TID_STRUCT, (batch, 1, hkv, d), torch.float64,
                            device, start=(r + 1) << 32)
            sl = slice(b * block, (b + 1) * block)
            z = k[:, sl].to(torch.float64)
            k[:, sl] = (centre + plant_noise * z).to(dtype)
    return q, k, v, info


def moba_decode_inputs(seed: int, batch: int, n: int, q_len: int, hq: int, hkv: int, d: int,
                       dtype=torch.bfloat16, device="cpu", planted: int = 0, block: int = 0):
    """Decode-step inputs: the KV cache k, v [batch, n, hkv, d] as in
    moba_inputs (same draws and planting for the same seed) and the queries of
    the last q_len positions only, q [batch, q_len, hq, d], drawn from their
    own stream (tensor id TID_Q, counters from 1 << 40 on)."""
    k = normal(seed, TID_K, (batch, n, hkv, d), dtype, device)
    v = normal(seed, TID_V, (batch, n, hkv, d), dtype, device)
    info = {}
    if planted:
        nb = n // block
        ids = planted_block_ids(seed, planted, nb - 1)
        info["planted_blocks"] = ids
        for r, b in enumerate(ids):
            centre = normal(seed, TID_STRUCT, (batch, 1, hkv, d), torch.float64,
                            device, start=(r + 1) << 32)
            sl = slice(b * block, (b + 1) * block)
            z = k[:, sl].to(torch.float64)
            k[:, sl] = (centre + 0.25 * z).to(dtype)
    q = normal(seed, TID_Q, (batch, q_len, hq, d), dtype, device, start=1 << 40)
    return q, k, v, info


def compression_weights(seed: int, d_c: int, d_model: int, tensor_id: int = TID_W,
                        dtype=torch.bfloat16, device="cpu") -> torch.Tensor:
    """W = G / sqrt(d_model) with G ~ N(0,1) rounded to bf16 first; for a
    power-of-four d_model the scaling is exact in bf16. A random
    Johnson-Lindenstrauss map stands in for the trained compression layer."""
    g = normal(seed, tensor_id, (d_c, d_model), dtype, device)
    return (g.to(torch.float64) / math.sqrt(d_model)).to(dtype)


def esa_inputs(seed: int, batch: int, ctx: int, m: int, h: int, d: int,
               dtype=torch.bfloat16, device="cpu", needles: int = 0,
               needle_lo: int = 0, needle_hi: int = 0, needle_gap: int = 0,
               needle_scale: float = 0.375):
    """q [batch,m,h,d] for the chunk's queries; K,V caches [batch,ctx,h,d].

    With ``needles`` > 0 (decode, m == 1), that many keys per sequence at
    seeded positions in [needle_lo, needle_hi) are set to needle_scale * q of
    the same sequence, for every head.
    """
    q = normal(seed, TID_Q, (batch, m, h, d), dtype, device)
    k = normal(seed, TID_K, (batch, ctx, h, d), dtype, device)
    v = normal(seed, TID_V, (batch, ctx, h, d), dtype, device)
    info = {}
    if needles:
        pos = []
        for bi in range(batch):
            p = needle_positions(seed, bi, needles, needle_lo, needle_hi, needle_gap)
            pos.append(p)
            val = (q[bi, 0].to(torch.float64) * needle_scale).to(dtype)
            for t in p:
                k[bi, t] = val
        info["needles"] = pos
    return q, k, v, info
