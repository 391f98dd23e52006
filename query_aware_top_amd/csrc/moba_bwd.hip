// MoBA attention gradients with the gating held fixed (the gated sets are a
// discrete choice; the gate has no parameters of its own): for every
// processed row (t, h) with key set I = gated earlier blocks + [cur*B, t],
//   p_j = exp(scale q.k_j - lse),  dp_j = dO.v_j,  D = sum_j p_j dp_j,
//   ds_j = p_j (dp_j - D),  dq = scale sum_j ds_j k_j,
//   dv_j += p_j dO,  dk_j += scale ds_j q   (GQA: the query heads of a KV
//   head add into it).
// MoBA write-up, sections 2-3 (the attention over the gated set); the
// gradient is that of softmax attention restricted to the set.
//
// Kernels:
//   dq      bfloat16: on the matrix cores (gated blocks per dispatch tile
//           into float32 partials, own block + partials per row, below);
//           float32: one
//           wave per row, four 16-lane groups taking every fourth key of the
//           row's set, p straight from the forward lse (no running max) and
//           D accumulated in the same pass through
//           dq = scale (sum p dp k - D sum p k);
//   own     a workgroup per (sequence, KV head, 64 keys of a block): the
//           block's own rows (positions in the block, every query head of
//           the group, causal); writes dk, dv of its keys (every key of the
//           sequence is written by exactly one workgroup);
//   gated   the rows that gated the block, as bucketed by the forward
//           dispatch: bfloat16, a workgroup per (run of up to 8 dispatch
//           tiles of one bucket, 128 keys) writing its sums to its own slot,
//           then one pass adding each bucket's slots in run order (no
//           atomics, deterministic); float32, a workgroup per (run of
//           dispatch tiles, 64 keys) adding into dk, dv with float atomics
//           once per bucket the run touches.
// The key kernels run in vector float32 arithmetic: lane (key i, quarter c) of a wave holds dims
// [c D/4, (c+1) D/4) of key i's K, V, dK and dV; rows pass through LDS 16 at
// a time as float32 (quarters padded against bank conflicts).
#include <algorithm>
#include <type_traits>

#include "attn_bwd.h"
#include "attn_core.h"
#include "common.h"
#include "launch.h"

namespace qat {

constexpr int kBwdKeys = 64;   // keys per workgroup of the key kernels (16 per wave)
constexpr int kBwdRows = 16;   // rows staged per LDS round
constexpr int kBwdTilesPerWg = 8;
constexpr int kRowsPerTileBwd = 256;   // rows per forward dispatch tile

template <typename T, int N>
__device__ __forceinline__ void load_f32(const T* p, float (&x)[N]) {
#pragma unroll
  for (int e = 0; e < N; ++e) x[e] = to_f32(p[e]);
}

// ---------------------------------------------------------------------------
// dq and D, one wave per row; row = ((bi * q_len) + r) * hq + h; q holds the
// whole sequence ([batch, seq_len, hq, D]), dO and dq the processed rows.
template <typename T, int D>
__global__ __launch_bounds__(256) void moba_bwd_dq_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const int32_t* __restrict__ blk,
    const T* __restrict__ dout, const float* __restrict__ lse, float* __restrict__ dq, float* __restrict__ delta,
    int64_t rows, int64_t seq_len, int64_t hq, int64_t hkv, int64_t q_start, int64_t q_len, int block, int topk,
    float scale) {
  constexpr int E = D / 16;
  constexpr int NK = 2;   // keys per group and step
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63, grp = lane >> 4, sub = lane & 15;
  const int64_t h = row % hq;
  const int64_t r = (row / hq) % q_len;
  const int64_t bi = row / (hq * q_len);
  const int64_t g = h / (hq / hkv);
  const int64_t t = q_start + r;
  const int64_t cur = t / block;
  float qf[E], df[E];
  load_f32<T, E>(q + ((bi * seq_len + t) * hq + h) * D + sub * E, qf);
  load_f32<T, E>(dout + row * D + sub * E, df);
  const float sl2 = scale * kLog2e, lse2 = lse[row] * kLog2e;
  float A[E], Bv[E], Ds = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) { A[e] = 0.f; Bv[e] = 0.f; }
  const int64_t base = (bi * seq_len * hkv + g) * D + sub * E, stride = hkv * D;
  auto span = [&](int64_t a, int64_t b) {   // keys a .. b-1
    for (int64_t j0 = a; j0 < b; j0 += 4 * NK) {
      float kx[NK][E], vx[NK][E];
      bool ok[NK];
#pragma unroll
      for (int u = 0; u < NK; ++u) {
        const int64_t j = j0 + 4 * u + grp;
        ok[u] = j < b;
        const int64_t f = base + (ok[u] ? j : a) * stride;
        load_f32<T, E>(k + f, kx[u]);
        load_f32<T, E>(v + f, vx[u]);
      }
#pragma unroll
      for (int u = 0; u < NK; ++u) {
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          s = fmaf(qf[e], kx[u][e], s);
          dp = fmaf(df[e], vx[u][e], dp);
        }
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) {   // within the 16-lane group
          s += __shfl_xor(s, off, 64);
          dp += __shfl_xor(dp, off, 64);
        }
        const float p = ok[u] ? __builtin_amdgcn_exp2f(s * sl2 - lse2) : 0.f;
        const float pd = p * dp;
        Ds += pd;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          A[e] = fmaf(pd, kx[u][e], A[e]);
          Bv[e] = fmaf(p, kx[u][e], Bv[e]);
        }
      }
    }
  };
  const int32_t* br = blk + row * topk;
  for (int s = 0; s < topk - 1; ++s) {   // gated earlier blocks sit in the first topk - 1 slots
    const int32_t b = br[s];
    if (b < 0 || b >= cur) continue;
    span((int64_t)b * block, (int64_t)(b + 1) * block);
  }
  span(cur * block, t + 1);
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) {   // the four groups
    Ds += __shfl_xor(Ds, off, 64);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      A[e] += __shfl_xor(A[e], off, 64);
      Bv[e] += __shfl_xor(Bv[e], off, 64);
    }
  }
  if (grp == 0) {
#pragma unroll
    for (int e = 0; e < E; ++e) dq[row * D + sub * E + e] = scale * (A[e] - Ds * Bv[e]);
  }
  if (lane == 0) delta[row] = Ds;
}

// ---------------------------------------------------------------------------
// Key-side state of one lane and the rows staged in LDS.
template <int D>
struct BwdRows {
  static constexpr int Q4 = D / 4;
  static constexpr int RS = 4 * (Q4 + 4);   // a row: four padded quarters
  float q[kBwdRows * RS];
  float d[kBwdRows * RS];
  float lse2[kBwdRows];
  float di[kBwdRows];
  int32_t t[kBwdRows];
};

template <typename T, int D>
struct KeyGrad {
  static constexpr int Q4 = D / 4;
  float kf[Q4], vf[Q4], dk[Q4], dv[Q4];
  __device__ void load(const T* __restrict__ K, const T* __restrict__ V, int64_t off) {
    load_f32<T, Q4>(K + off, kf);
    load_f32<T, Q4>(V + off, vf);
#pragma unroll
    for (int i = 0; i < Q4; ++i) { dk[i] = 0.f; dv[i] = 0.f; }
  }
  // one staged row; qr / dr point at this lane's quarter; `on`: key in the row's set
  __device__ void row(const float* qr, const float* dr, float lse2, float di, float sl2, bool on) {
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int i = 0; i < Q4; i += 4) {
      const float4 a = *reinterpret_cast<const float4*>(qr + i);
      const float4 b = *reinterpret_cast<const float4*>(dr + i);
      s = fmaf(a.x, kf[i], fmaf(a.y, kf[i + 1], fmaf(a.z, kf[i + 2], fmaf(a.w, kf[i + 3], s))));
      dp = fmaf(b.x, vf[i], fmaf(b.y, vf[i + 1], fmaf(b.z, vf[i + 2], fmaf(b.w, vf[i + 3], dp))));
    }
    s += __shfl_xor(s, 1, 64);   // the key's four quarters
    s += __shfl_xor(s, 2, 64);
    dp += __shfl_xor(dp, 1, 64);
    dp += __shfl_xor(dp, 2, 64);
    const float p = on ? __builtin_amdgcn_exp2f(s * sl2 - lse2) : 0.f;
    const float ds = p * (dp - di);
#pragma unroll
    for (int i = 0; i < Q4; i += 4) {
      const float4 a = *reinterpret_cast<const float4*>(qr + i);
      const float4 b = *reinterpret_cast<const float4*>(dr + i);
      dv[i] = fmaf(p, b.x, dv[i]);
      dv[i + 1] = fmaf(p, b.y, dv[i + 1]);
      dv[i + 2] = fmaf(p, b.z, dv[i + 2]);
      dv[i + 3] = fmaf(p, b.w, dv[i + 3]);
      dk[i] = fmaf(ds, a.x, dk[i]);
      dk[i + 1] = fmaf(ds, a.y, dk[i + 1]);
      dk[i + 2] = fmaf(ds, a.z, dk[i + 2]);
      dk[i + 3] = fmaf(ds, a.w, dk[i + 3]);
    }
  }
};

// Stage row i (< kBwdRows) of the round: q row qrow of q, dO row `row`.
template <typename T, int D>
__device__ __forceinline__ void bwd_stage(BwdRows<D>& L, int i, const T* __restrict__ q, int64_t qrow,
                                          const T* __restrict__ dout, int64_t row, int part) {
  // part p of 16 covers dims [p D/16, (p+1) D/16) of both rows
  constexpr int E = D / 16, Q4 = D / 4;
  const int d0 = part * E;
  const int dst = i * BwdRows<D>::RS + (d0 / Q4) * (Q4 + 4) + d0 % Q4;
  float x[E];
  load_f32<T, E>(q + qrow * D + d0, x);
#pragma unroll
  for (int e = 0; e < E; ++e) L.q[dst + e] = x[e];
  load_f32<T, E>(dout + row * D + d0, x);
#pragma unroll
  for (int e = 0; e < E; ++e) L.d[dst + e] = x[e];
}

// ---------------------------------------------------------------------------
// Own-block rows. grid (blocks * chunks per block, hkv, batch).
template <typename T, int D>
__global__ __launch_bounds__(256) void moba_bwd_own_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta, float* __restrict__ dk, float* __restrict__ dv,
    int64_t seq_len, int64_t hq, int64_t hkv, int64_t q_start, int64_t q_len, int block, int cpb, float scale) {
  constexpr int Q4 = D / 4;
  __shared__ __align__(16) BwdRows<D> L;
  const int64_t b = blockIdx.x / cpb, c = blockIdx.x % cpb, g = blockIdx.y, bi = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qd = lane & 3;
  const int64_t blk0 = b * block, blk1 = min(blk0 + block, seq_len);
  const int64_t c0 = blk0 + c * kBwdKeys;
  if (c0 >= blk1) return;   // uniform: chunk past a partial last block
  const int64_t c1 = min(c0 + kBwdKeys, blk1);
  const int64_t key = c0 + wave * 16 + (lane >> 2);
  const bool kvalid = key < c1;
  const int64_t off = ((bi * seq_len + (kvalid ? key : c0)) * hkv + g) * D + qd * Q4;
  KeyGrad<T, D> kg;
  kg.load(k, v, off);
  const float sl2 = scale * kLog2e;
  // rows: positions [max(c0, q_start), min(blk1, q_start + q_len)) x the group's heads
  const int64_t G = hq / hkv;
  const int64_t t0 = max(c0, q_start), t1 = min(blk1, q_start + q_len);
  const int64_t nrows = t1 > t0 ? (t1 - t0) * G : 0;
  for (int64_t r0 = 0; r0 < nrows; r0 += kBwdRows) {
    const int nr = (int)min((int64_t)kBwdRows, nrows - r0);
    __syncthreads();   // the previous round's rows are consumed
    {
      const int i = tid >> 4, part = tid & 15;
      if (i < nr) {
        const int64_t ri = r0 + i, tt = t0 + ri / G, h = g * G + ri % G;
        const int64_t row = (bi * q_len + (tt - q_start)) * hq + h;
        bwd_stage<T, D>(L, i, q, (bi * seq_len + tt) * hq + h, dout, row, part);
        if (part == 0) {
          L.lse2[i] = lse[row] * kLog2e;
          L.di[i] = delta[row];
          L.t[i] = (int32_t)tt;
        }
      }
    }
    __syncthreads();
    for (int i = 0; i < nr; ++i) {
      const float* qr = L.q + i * BwdRows<D>::RS + qd * (Q4 + 4);
      const float* dr = L.d + i * BwdRows<D>::RS + qd * (Q4 + 4);
      kg.row(qr, dr, L.lse2[i], L.di[i], sl2, kvalid && key <= L.t[i]);
    }
  }
  if (kvalid) {
#pragma unroll
    for (int i = 0; i < Q4; ++i) {
      dk[off + i] = scale * kg.dk[i];
      dv[off + i] = kg.dv[i];
    }
  }
}

// ---------------------------------------------------------------------------
// Gated rows, over the forward dispatch's tiles (a tile: rows of one bucket
// (sequence, KV head, block); tiles of a bucket are adjacent). grid (runs of
// kBwdTilesPerWg tiles, chunks per block).
template <typename T, int D>
__global__ __launch_bounds__(256) void moba_bwd_gated_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta, const int4* __restrict__ tiles,
    const int32_t* __restrict__ ntiles, const int2* __restrict__ entries, float* __restrict__ dk,
    float* __restrict__ dv, int64_t hkv, int block, float scale) {
  constexpr int Q4 = D / 4;
  __shared__ __align__(16) BwdRows<D> L;
  const int nt = ntiles[0];
  const int tb = blockIdx.x * kBwdTilesPerWg;
  if (tb >= nt) return;   // uniform
  const int te = min(nt, tb + kBwdTilesPerWg);
  const int c = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qd = lane & 3;
  const int kl = c * kBwdKeys + wave * 16 + (lane >> 2);   // key within the block
  if (c * kBwdKeys >= block) return;                         // uniform
  const bool kvalid = kl < block;
  const int64_t koff = (int64_t)(kvalid ? kl : 0) * hkv * D + qd * Q4;
  const float sl2 = scale * kLog2e;
  KeyGrad<T, D> kg;
  int64_t cur_kv = -1;
  auto flush = [&]() {
    if (cur_kv < 0 || !kvalid) return;
#pragma unroll
    for (int i = 0; i < Q4; ++i) {
      unsafeAtomicAdd(dk + cur_kv + koff + i, scale * kg.dk[i]);
      unsafeAtomicAdd(dv + cur_kv + koff + i, kg.dv[i]);
    }
  };
  for (int ti = tb; ti < te; ++ti) {
    const int4 tile = tiles[ti];
    const int64_t kv = (int64_t)(uint32_t)tile.x | ((int64_t)tile.y << 32);
    if (kv != cur_kv) {
      flush();
      cur_kv = kv;
      kg.load(k + kv, v + kv, koff);
    }
    const int e0 = tile.z, n = tile.w;
    for (int r0 = 0; r0 < n; r0 += kBwdRows) {
      const int nr = min(kBwdRows, n - r0);
      __syncthreads();
      {
        const int i = tid >> 4, part = tid & 15;
        if (i < nr) {
          const int2 en = entries[e0 + r0 + i];
          const int64_t row = en.x >> 4;
          bwd_stage<T, D>(L, i, q, (int64_t)en.y, dout, row, part);
          if (part == 0) {
            L.lse2[i] = lse[row] * kLog2e;
            L.di[i] = delta[row];
          }
        }
      }
      __syncthreads();
      for (int i = 0; i < nr; ++i) {
        const float* qr = L.q + i * BwdRows<D>::RS + qd * (Q4 + 4);
        const float* dr = L.d + i * BwdRows<D>::RS + qd * (Q4 + 4);
        kg.row(qr, dr, L.lse2[i], L.di[i], sl2, kvalid);
      }
    }
  }
  flush();
}

constexpr int kBwdCurRows = 32 * kBwdNW;

template <int D>
constexpr int bwd_part_stride() { return 2 * D + 4; }   // A, B, D (+ padding) per (row, slot)

// dq of gated blocks: two workgroups per dispatch tile (128 rows each) leave
// float32 partials (A, B, D) per (row, slot); the own-block kernel adds its
// causal part and the row's partials, writes dq and D (which the key
// kernels read).
// Gated blocks: two workgroups per dispatch tile (rows [128 half, 128 half +
// 128)); part[(row * (topk-1) + slot) * PS + ...] = A, B (accumulator layout
// d = 32 t + 8 (i/4) + 4 (lane/32) + i%4), D.
template <int D>
__global__ __launch_bounds__(64 * kBwdNW, 1) void moba_bwd_dq_past_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const float* __restrict__ lse, const int4* __restrict__ tiles,
    const int32_t* __restrict__ ntiles, const int2* __restrict__ entries, float* __restrict__ part, int64_t hkv,
    int block, int topk, float scale) {
  constexpr int PS = bwd_part_stride<D>();
  QAT_FA_SMEM(D, sm);
  const int64_t id = xcd_logical_id(blockIdx.x, gridDim.x);
  const int64_t tile = id >> 1;
  if (tile >= ntiles[0]) return;
  const int4 td = tiles[tile];
  const int64_t kv_off = (int64_t)(uint32_t)td.x | ((int64_t)td.y << 32);
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int row0 = (int)(id & 1) * kBwdCurRows + wave * 32;   // the wave's first row of the tile
  if ((int)(id & 1) * kBwdCurRows >= td.w) return;   // uniform: no rows in this half
  DqState<D> st;
  {
    const int myrow = row0 + (lane & 31);
    const bool valid = myrow < td.w;
    const int2 e2 = valid ? entries[td.z + myrow] : make_int2(0, 0);
    const int64_t row = e2.x >> 4;
    dq_init<D>(st, q + (int64_t)e2.y * D, dout + row * D, valid ? lse[row] : 0.f, valid);
  }
  const int kv_stride = (int)(hkv * D);
  dq_segment<D, kBwdNW>(st, sm, k + kv_off, v + kv_off, block, scale * kLog2e,
                        [=](int j) { return j * kv_stride; }, [](int) { return true; });
  const float dsum = xor32_sum(st.dsum);
  // the row and slot again from the dispatch entry (not held across the loop:
  // this kernel is at the register limit)
  const int myrow = row0 + (fa_fresh_lane() & 31);
  if (myrow >= td.w) return;
  const int2 e2 = entries[td.z + myrow];
  const int64_t row = e2.x >> 4;
  const int slot = e2.x & 15;
  float* dst = part + (row * (topk - 1) + slot) * PS;
  const int h = lane >> 5;
#pragma unroll
  for (int tq = 0; tq < D / 32; ++tq)
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      f32x4 wa, wb;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        wa[e] = st.fa.o[tq][4 * gi + e];
        wb[e] = st.b[tq][4 * gi + e];
      }
      *(f32x4*)(dst + 32 * tq + 8 * gi + 4 * h) = wa;
      *(f32x4*)(dst + D + 32 * tq + 8 * gi + 4 * h) = wb;
    }
  if (h == 0) dst[2 * D] = dsum;
}

// Own block (causal) plus the row's gated partials -> dq and D. Row mapping
// as the forward's current-block kernel: a workgroup holds 32*NW rows =
// 32*NW/P consecutive positions x P query heads of one KV group.
template <int D>
__global__ __launch_bounds__(64 * kBwdNW, 1) void moba_bwd_dq_cur_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const float* __restrict__ lse, const int32_t* __restrict__ blk,
    const float* __restrict__ part, float* __restrict__ dq, float* __restrict__ delta, int64_t seq_len, int64_t hq,
    int64_t hkv, int64_t q_start, int64_t q_len, int block, int topk, float scale, int pack, int tiles_per_block,
    int64_t nblocks) {
  constexpr int NW = kBwdNW;
  constexpr int PS = bwd_part_stride<D>();
  QAT_FA_SMEM(D, sm);
  int64_t id = xcd_logical_id(blockIdx.x, gridDim.x);
  const int tt = (int)(id % tiles_per_block);
  id /= tiles_per_block;
  const int64_t cb = id % nblocks;
  id /= nblocks;
  const int64_t gs = hq / hkv;
  const int64_t npk = gs / pack;
  const int64_t hp = id % npk;
  id /= npk;
  const int64_t g = id % hkv;
  const int64_t bi = id / hkv;
  const int64_t c = q_start / block + cb;
  const int64_t lo = max(c * block, q_start);
  const int64_t hi = min((c + 1) * block, q_start + q_len);
  const int tok_per_tile = kBwdCurRows / pack;
  const int64_t t0 = lo + (int64_t)tt * tok_per_tile;
  if (t0 >= hi) return;   // uniform
  const int64_t t_last = min(hi, t0 + tok_per_tile) - 1;
  const int64_t h0 = g * gs + hp * pack;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int myrow = wave * 32 + (lane & 31);
  const int64_t t = t0 + myrow / pack;
  const int64_t h = h0 + myrow % pack;
  const bool valid = t <= t_last;
  const int64_t tv = valid ? t : t0;
  const int64_t row = (bi * q_len + (tv - q_start)) * hq + h;
  DqState<D> st;
  dq_init<D>(st, q + ((bi * seq_len + tv) * hq + h) * D, dout + row * D, lse[row], valid);
  const int64_t kpos0 = c * block;
  const int kv_stride = (int)(hkv * D);
  const int lim = valid ? (int)(t - kpos0) : -1;
  dq_segment<D, NW>(st, sm, k + ((bi * seq_len + kpos0) * hkv + g) * D, v + ((bi * seq_len + kpos0) * hkv + g) * D,
                    (int)(t_last - kpos0 + 1), scale * kLog2e, [=](int j) { return j * kv_stride; },
                    [=](int j) { return j <= lim; });
  float dsum = xor32_sum(st.dsum);
  if (!valid) return;
  const int hl = lane >> 5;
  const int km = topk - 1;
  const int64_t cur = t / block;
  for (int s = 0; s < km; ++s) {   // gated blocks sit in the first topk - 1 slots
    const int32_t b = blk[row * topk + s];
    if (b < 0 || b >= cur) continue;
    const float* src = part + (row * km + s) * PS;
#pragma unroll
    for (int tq = 0; tq < D / 32; ++tq)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const f32x4 wa = *(const f32x4*)(src + 32 * tq + 8 * gi + 4 * hl);
        const f32x4 wb = *(const f32x4*)(src + D + 32 * tq + 8 * gi + 4 * hl);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          st.fa.o[tq][4 * gi + e] += wa[e];
          st.b[tq][4 * gi + e] += wb[e];
        }
      }
    dsum += src[2 * D];
  }
  float* dst = dq + row * D;
#pragma unroll
  for (int tq = 0; tq < D / 32; ++tq)
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      f32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = scale * (st.fa.o[tq][4 * gi + e] - dsum * st.b[tq][4 * gi + e]);
      *(f32x4*)(dst + 32 * tq + 8 * gi + 4 * hl) = w;
    }
  if (hl == 0) delta[row] = dsum;
}

int64_t moba_bwd_max_runs(int64_t max_tiles, int64_t nbuckets);
constexpr int kKvRun = 8;              // dispatch tiles per gated workgroup
constexpr int kKvDynBytes = 6 * 64 * 4 + kKvRun * kRowsPerTileBwd * 8;

// Own-block rows. grid (blocks * key chunks, hkv, batch); rows = positions
// [max(chunk start, q_start), min(block end, q_start + q_len)) x the group's
// heads, row r = position t0 + r / G, head g G + r % G.
template <int D>
__global__ __launch_bounds__(64 * kBwdNW, 1) void moba_bwd_kv_own_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    float* __restrict__ dk, float* __restrict__ dv, int64_t seq_len, int64_t hq, int64_t hkv, int64_t q_start,
    int64_t q_len, int block, int cpb, float scale) {
  QAT_FA_SMEM(D, sm);
  extern __shared__ __align__(16) char kv_dyn[];
  float* s_lse = reinterpret_cast<float*>(kv_dyn);          // [2][64]
  float* s_di = s_lse + 128;                                 // [2][64]
  const int64_t b = blockIdx.x / cpb, c = blockIdx.x % cpb, g = blockIdx.y, bi = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t blk0 = b * block, blk1 = min(blk0 + block, seq_len);
  const int64_t c0 = blk0 + c * kKvKeys;
  if (c0 >= blk1) return;   // uniform
  const int64_t c1 = min(c0 + kKvKeys, blk1);
  const int64_t key = c0 + wave * 32 + (lane & 31);
  const bool kvalid = key < c1;
  const int64_t krow = ((bi * seq_len + (kvalid ? key : c0)) * hkv + g) * D;
  KvState<D> st;
  const int64_t G = hq / hkv;
  const int64_t t0 = max(c0, q_start), t1 = min(blk1, q_start + q_len);
  const int nrows = t1 > t0 ? (int)((t1 - t0) * G) : 0;
  const int nt = (nrows + 63) / 64;
  const bf16* qbase = q + bi * seq_len * hq * D;
  const bf16* dbase = dout + bi * q_len * hq * D;
  const float sl2 = scale * kLog2e;
  // row r: position t0 + r / G, head g G + r % G; offsets in 32 bits (one
  // sequence's q rows hold fewer than 2^31 elements)
  const int Gi = (int)G, hqi = (int)hq;
  const int q0 = (int)(t0 * hq + g * G), d0 = (int)((t0 - q_start) * hq + g * G);
  auto issue = [&](bf16* qdst, bf16* ddst, int buf, int rt) {
    const int r0 = rt * 64, n = min(64, nrows - r0);
    // lane terms recomputed at each issue (the kernel is at the register limit)
    auto qofs = [=](int j) {
      const int r = r0 + j, ti = r / Gi;
      return (q0 + ti * hqi + (r - ti * Gi)) * D;
    };
    auto dofs = [=](int j) {
      const int r = r0 + j, ti = r / Gi;
      return (d0 + ti * hqi + (r - ti * Gi)) * D;
    };
    fa_issue_one<D, kBwdNW, decltype(qofs), true, true>(qdst, qbase, 0, n, qofs);
    fa_issue_one<D, kBwdNW, decltype(dofs), true, true>(ddst, dbase, 0, n, dofs);
    if (wave == 0) {
      // rows past the tile's end repeat its last row (masked)
      const int r = r0 + min(lane, n - 1), ti = r / Gi;
      const int64_t tt = t0 + ti;
      const int64_t row = (bi * q_len + (tt - q_start)) * hq + g * G + (r - ti * Gi);
      __builtin_amdgcn_global_load_lds((const global_void*)(lse + row), (lds_void*)(s_lse + buf * 64), 4, 0, 0);
      __builtin_amdgcn_global_load_lds((const global_void*)(delta + row), (lds_void*)(s_di + buf * 64), 4, 0, 0);
    }
  };
  // causal mask: row m of tile rt (position t0 + (64 rt + m) / G) sees this
  // lane's key iff m >= (key - t0) G - 64 rt
  // (the lane's key is re-derived per tile from fa_fresh_lane(), and its row
  // after the loop: nothing per lane is held across the loop)
  auto row_ok = [=](int rt) {
    const int64_t kf = c0 + wave * 32 + (fa_fresh_lane() & 31);
    const int kfirst = (int)(kf - t0) * Gi;
    const int n = min(64, nrows - rt * 64), m0 = kfirst - rt * 64;
    return [=](int m) { return m < n && m >= m0; };
  };
  if (nt > 0) issue(sm.k0, sm.v0, 0, 0);
  kv_load<D>(st, k + krow, v + krow);   // after the first tile's loads, which then overlap it
  for (int rt = 0; rt < nt; rt += 2) {
    fa_wait_loads();
    fa_lds_barrier();
    if (rt + 1 < nt) issue(sm.k1, sm.v1, 1, rt + 1);
    kv_tile<D>(st, sm.k0, sm.v0, s_lse, s_di, sl2, row_ok(rt));
    if (rt + 1 >= nt) break;
    fa_wait_loads();
    fa_lds_barrier();
    if (rt + 2 < nt) issue(sm.k0, sm.v0, 0, rt + 2);
    kv_tile<D>(st, sm.k1, sm.v1, s_lse + 64, s_di + 64, sl2, row_ok(rt + 1));
  }
  if (kvalid) {
    const int64_t kend = c0 + wave * 32 + (fa_fresh_lane() & 31);
    const int64_t krow_end = ((bi * seq_len + kend) * hkv + g) * D;
    kv_write<D, false>(st, dk + krow_end, dv + krow_end, scale);
  }
}

// Runs of the gated key kernel: bucket b's dispatch tiles [tile_off[b],
// tile_off[b + 1]) cut into runs of kKvRun; run_off[b] = runs before bucket b,
// run_off[nb] = all runs. One workgroup, 1024 buckets per pass (inclusive
// Hillis-Steele scan in LDS).
__global__ __launch_bounds__(1024) void moba_bwd_runs_kernel(const int32_t* __restrict__ tile_off, int32_t nb,
                                                             int32_t* __restrict__ run_off) {
  __shared__ int32_t s[1024];
  __shared__ int32_t carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int32_t base = 0; base < nb; base += 1024) {
    const int32_t i = base + threadIdx.x;
    const int32_t c = i < nb ? (tile_off[i + 1] - tile_off[i] + kKvRun - 1) / kKvRun : 0;
    s[threadIdx.x] = c;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int32_t a = threadIdx.x >= off ? s[threadIdx.x - off] : 0;
      __syncthreads();
      s[threadIdx.x] += a;
      __syncthreads();
    }
    if (i < nb) run_off[i] = carry + s[threadIdx.x] - c;
    __syncthreads();
    if (threadIdx.x == 1023) carry += s[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) run_off[nb] = carry;
}

// Gated rows: grid (runs, key chunks of the block); a run is up to kKvRun
// dispatch tiles of one bucket (sequence, KV head, block). The run's entries
// are staged in LDS; its sums (dK already scaled) go to its own slot of
// `part` ([run][chunk][dK, dV][kKvKeys][D]) with plain stores, and
// moba_bwd_kv_reduce_kernel adds the slots of each bucket in run order.
template <int D>
__global__ __launch_bounds__(64 * kBwdNW, 1) void moba_bwd_kv_gated_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    const int4* __restrict__ tiles, const int32_t* __restrict__ tile_off, const int32_t* __restrict__ run_off,
    int32_t nb, const int2* __restrict__ entries, float* __restrict__ part, int64_t seq_len, int64_t hq,
    int64_t hkv, int64_t q_len, int block, float scale) {
  QAT_FA_SMEM(D, sm);
  extern __shared__ __align__(16) char kv_dyn[];
  float* s_lse = reinterpret_cast<float*>(kv_dyn);   // [2][64]
  float* s_di = s_lse + 128;                          // [2][64]
  int2* s_ent = reinterpret_cast<int2*>(s_di + 256);  // the run's entries (after [2][64] unused ints)
  const int32_t w = blockIdx.x;
  if (w >= run_off[nb]) return;   // uniform
  const int c = blockIdx.y;
  if (c * kKvKeys >= block) return;   // uniform
  // the run's bucket: the last one whose first run is not after w
  int32_t lo = 0, hi = nb - 1;
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if (run_off[mid] <= w) lo = mid;
    else hi = mid - 1;
  }
  const int tb = tile_off[lo] + (w - run_off[lo]) * kKvRun;
  const int te = min(tb + kKvRun, tile_off[lo + 1]);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kl = c * kKvKeys + wave * 32 + (lane & 31);   // key within the block
  const bool kvalid = kl < block;
  const int e_first = tiles[tb].z;
  {
    const int4 tl = tiles[te - 1];
    const int nent = tl.z + tl.w - e_first;
    for (int i = threadIdx.x; i < nent; i += 64 * kBwdNW) s_ent[i] = entries[e_first + i];
  }
  __syncthreads();
  const int4 t0d = tiles[tb];
  const int64_t kv = (int64_t)(uint32_t)t0d.x | ((int64_t)t0d.y << 32);
  const int64_t bi = kv / (seq_len * hkv * D);
  const int64_t qo = bi * seq_len * hq, dof = bi * q_len * hq;
  const bf16* qbase = q + qo * D;
  const bf16* dbase = dout + dof * D;
  const float sl2 = scale * kLog2e;
  auto issue = [&](bf16* qdst, bf16* ddst, int buf, int ti, int r0) {
    const int4 tl = tiles[ti];
    const int n = min(64, tl.w - r0);
    const int e0 = tl.z - e_first + r0;
    fa_issue_one<D, kBwdNW>(qdst, qbase, 0, n, [=](int j) { return (int)((s_ent[e0 + j].y - qo) * D); });
    fa_issue_one<D, kBwdNW>(ddst, dbase, 0, n,
                            [=](int j) { return (int)(((int64_t)(s_ent[e0 + j].x >> 4) - dof) * D); });
    if (wave == 0) {
      const int64_t row = s_ent[e0 + min(lane, n - 1)].x >> 4;
      __builtin_amdgcn_global_load_lds((const global_void*)(lse + row), (lds_void*)(s_lse + buf * 64), 4, 0, 0);
      __builtin_amdgcn_global_load_lds((const global_void*)(delta + row), (lds_void*)(s_di + buf * 64), 4, 0, 0);
    }
  };
  auto advance = [&](int& ti, int& r0) {
    r0 += 64;
    if (r0 >= tiles[ti].w) { ++ti; r0 = 0; }
  };
  auto rows_of = [&](int ti, int r0) { return min(64, tiles[ti].w - r0); };
  int ti = tb, r0 = 0;
  issue(sm.k0, sm.v0, 0, ti, r0);
  KvState<D> st;
  const int64_t koff = (int64_t)(kvalid ? kl : 0) * hkv * D;
  kv_load<D>(st, k + kv + koff, v + kv + koff);   // after the first tile's loads, which then overlap it
  for (;;) {
    fa_wait_loads();
    fa_lds_barrier();
    int tn = ti, rn = r0;
    advance(tn, rn);
    if (tn < te) issue(sm.k1, sm.v1, 1, tn, rn);
    {
      const int n = rows_of(ti, r0);
      kv_tile<D>(st, sm.k0, sm.v0, s_lse, s_di, sl2, [=](int m) { return m < n; });
    }
    ti = tn;
    r0 = rn;
    if (ti >= te) break;
    fa_wait_loads();
    fa_lds_barrier();
    advance(tn, rn);
    if (tn < te) issue(sm.k0, sm.v0, 0, tn, rn);
    {
      const int n = rows_of(ti, r0);
      kv_tile<D>(st, sm.k1, sm.v1, s_lse + 64, s_di + 64, sl2, [=](int m) { return m < n; });
    }
    ti = tn;
    r0 = rn;
    if (ti >= te) break;
  }
  fa_wait_loads();
  if (kvalid) {
    float* slot = part + ((int64_t)w * gridDim.y + c) * 2 * kKvKeys * D + (wave * 32 + (lane & 31)) * D;
    kv_write<D, false>(st, slot, slot + kKvKeys * D, scale);
  }
}

// dK, dV of bucket b's keys += the sums of its runs, in run order: grid
// (buckets, key chunks, kRedSlices); a thread adds float4 pieces, the
// slices split a chunk's pieces so that a bucket with many runs (a block
// many rows gated) is spread over several workgroups.
constexpr int kRedSlices = 8;
template <int D>
__global__ __launch_bounds__(256) void moba_bwd_kv_reduce_kernel(const float* __restrict__ part,
                                                                 const int32_t* __restrict__ run_off,
                                                                 const int32_t* __restrict__ tile_off,
                                                                 const int4* __restrict__ tiles,
                                                                 float* __restrict__ dk, float* __restrict__ dv,
                                                                 int64_t hkv, int block) {
  const int32_t b = blockIdx.x;
  const int32_t r0 = run_off[b], r1 = run_off[b + 1];
  if (r0 == r1) return;   // no gated rows in this bucket
  const int c = blockIdx.y;
  const int nk = min(kKvKeys, block - c * kKvKeys);
  if (nk <= 0) return;
  const int4 td = tiles[tile_off[b]];
  const int64_t kv = (int64_t)(uint32_t)td.x | ((int64_t)td.y << 32);
  constexpr int D4 = D / 4;
  const int ncpk = gridDim.y;
  const int64_t rstride = (int64_t)ncpk * 2 * kKvKeys * D;   // floats between consecutive runs' slots
#pragma unroll 2
  for (int e = threadIdx.x + blockIdx.z * 256; e < 2 * nk * D4; e += 256 * kRedSlices) {
    const int tsr = e / (nk * D4), rem = e % (nk * D4), j = rem / D4, d4 = rem % D4;
    const float* src = part + (((int64_t)r0 * ncpk + c) * 2 + tsr) * kKvKeys * D + j * D + 4 * d4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    int32_t w = r0;
    for (; w + 4 <= r1; w += 4, src += 4 * rstride) {   // four runs' loads in flight, added in run order
      const f32x4 x0 = *(const f32x4*)src, x1 = *(const f32x4*)(src + rstride);
      const f32x4 x2 = *(const f32x4*)(src + 2 * rstride), x3 = *(const f32x4*)(src + 3 * rstride);
      acc += x0;
      acc += x1;
      acc += x2;
      acc += x3;
    }
    for (; w < r1; ++w, src += rstride) acc += *(const f32x4*)src;
    float* dst = (tsr == 0 ? dk : dv) + kv + (int64_t)(c * kKvKeys + j) * hkv * D + 4 * d4;
    f32x4 y = *(const f32x4*)dst;
    *(f32x4*)dst = y + acc;
  }
}

// ---------------------------------------------------------------------------
int moba_bwd_chunks(int block) { return (int)cdiv(block, kBwdKeys); }

template <typename T, int D>
static hipError_t launch_moba_bwd_d(const T* q, const T* k, const T* v, const int32_t* blk,
                                    const T* dout, const float* lse, const int4* tiles, const int32_t* ntiles,
                                    const int2* entries, int64_t max_tiles, const int32_t* tile_off,
                                    int64_t nbuckets, int32_t* run_off, float* kv_part, float* dq_part, float* dq,
                                    float* delta,
                                    float* dk, float* dv, int64_t batch, int64_t seq_len, int64_t hq, int64_t hkv,
                                    int64_t q_start, int64_t q_len, int block, int topk, float scale,
                                    hipStream_t s) {
  constexpr bool kMfma = std::is_same<T, bf16>::value;
  const int64_t rows = batch * q_len * hq;
  const int cpb = moba_bwd_chunks(block);
  const int64_t nb_all = cdiv(seq_len, block);
  const bool gated = topk > 1 && max_tiles > 0;
  hipError_t e;
  if constexpr (kMfma) {
    if (gated) {
      KTimer tm("moba_bwd_dq_past", s);
      launch_timed("moba_bwd_dq_past", moba_bwd_dq_past_kernel<D>, dim3((unsigned)(2 * max_tiles)),
                   dim3(64 * kBwdNW), 0, s, q, k, v, dout, lse, tiles, ntiles, entries, dq_part, hkv, block, topk,
                   scale);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const int64_t gs = hq / hkv;
    const int pack = (kBwdCurRows % gs == 0) ? (int)gs : 1;
    const int tiles_per_block = (int)cdiv(block, kBwdCurRows / pack);
    const int64_t nblocks = (q_start + q_len - 1) / block - q_start / block + 1;
    const int64_t nwg = (int64_t)tiles_per_block * nblocks * batch * hkv * (gs / pack);
    {
      KTimer tm("moba_bwd_dq", s);
      launch_timed("moba_bwd_dq", moba_bwd_dq_cur_kernel<D>, dim3((unsigned)nwg), dim3(64 * kBwdNW), 0, s, q, k, v,
                   dout, lse, blk, (const float*)dq_part, dq, delta, seq_len, hq, hkv, q_start, q_len, block, topk,
                   scale, pack, tiles_per_block, nblocks);
    }
  } else {
    KTimer tm("moba_bwd_dq", s);
    launch_timed("moba_bwd_dq", moba_bwd_dq_kernel<T, D>, dim3((unsigned)cdiv(rows, 4)), dim3(256), 0, s, q, k, v,
                 blk, dout, lse, dq, delta, rows, seq_len, hq, hkv, q_start, q_len, block, topk, scale);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if constexpr (kMfma) {
    // the matrix-core key kernels address one sequence's q / dO rows with
    // 32-bit offsets from the sequence's base
    if (seq_len * hq * D < (1ll << 31) && moba_rows_per_tile() == kRowsPerTileBwd) {
      static const bool lds_ok = [] {
        bool ok = hipFuncSetAttribute((const void*)moba_bwd_kv_own_kernel<D>,
                                      hipFuncAttributeMaxDynamicSharedMemorySize, kKvDynBytes) == hipSuccess;
        ok &= hipFuncSetAttribute((const void*)moba_bwd_kv_gated_kernel<D>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, kKvDynBytes) == hipSuccess;
        return ok;
      }();
      if (!lds_ok) return hipErrorInvalidConfiguration;
      const int cpk = (int)cdiv(block, kKvKeys);
      {
        KTimer tm("moba_bwd_own", s);
        launch_timed("moba_bwd_own", moba_bwd_kv_own_kernel<D>,
                     dim3((unsigned)(nb_all * cpk), (unsigned)hkv, (unsigned)batch), dim3(64 * kBwdNW), 1536, s, q,
                     k, v, dout, lse, (const float*)delta, dk, dv, seq_len, hq, hkv, q_start, q_len, block, cpk,
                     scale);
      }
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if (gated) {
        KTimer tm("moba_bwd_gated", s);
        hipLaunchKernelGGL(moba_bwd_runs_kernel, dim3(1), dim3(1024), 0, s, tile_off, (int32_t)nbuckets, run_off);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        launch_timed("moba_bwd_gated", moba_bwd_kv_gated_kernel<D>,
                     dim3((unsigned)moba_bwd_max_runs(max_tiles, nbuckets), (unsigned)cpk), dim3(64 * kBwdNW),
                     kKvDynBytes, s, q, k, v, dout, lse, (const float*)delta, tiles, (const int32_t*)tile_off,
                     (const int32_t*)run_off, (int32_t)nbuckets, entries, kv_part, seq_len, hq, hkv, q_len, block,
                     scale);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(moba_bwd_kv_reduce_kernel<D>, dim3((unsigned)nbuckets, (unsigned)cpk, kRedSlices), dim3(256),
                           0, s,
                           (const float*)kv_part, (const int32_t*)run_off, (const int32_t*)tile_off, tiles, dk, dv,
                           hkv, block);
      }
      return hipGetLastError();
    }
  }
  {
    KTimer tm("moba_bwd_own", s);
    launch_timed("moba_bwd_own", moba_bwd_own_kernel<T, D>, dim3((unsigned)(nb_all * cpb), (unsigned)hkv,
                 (unsigned)batch), dim3(256), 0, s, q, k, v, dout, lse, (const float*)delta, dk, dv, seq_len, hq,
                 hkv, q_start, q_len, block, cpb, scale);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (gated) {
    KTimer tm("moba_bwd_gated", s);
    launch_timed("moba_bwd_gated", moba_bwd_gated_kernel<T, D>,
                 dim3((unsigned)std::max<int64_t>(1, cdiv(max_tiles, kBwdTilesPerWg)), (unsigned)cpb), dim3(256), 0,
                 s, q, k, v, dout, lse, (const float*)delta, tiles, ntiles, entries, dk, dv, hkv, block, scale);
  }
  return hipGetLastError();
}

int64_t moba_bwd_part_floats(int64_t rows, int topk, int64_t d) { return rows * (topk - 1) * (2 * d + 4); }
int64_t moba_bwd_max_runs(int64_t max_tiles, int64_t nbuckets) { return cdiv(max_tiles, kKvRun) + nbuckets; }
int64_t moba_bwd_kv_part_floats(int64_t max_tiles, int64_t nbuckets, int block, int64_t d) {
  return moba_bwd_max_runs(max_tiles, nbuckets) * cdiv(block, kKvKeys) * 2 * kKvKeys * d;
}

hipError_t launch_moba_bwd(const void* q, const void* k, const void* v, const int32_t* blk,
                           const void* dout, const float* lse, const int4* tiles, const int32_t* ntiles,
                           const int2* entries, int64_t max_tiles, const int32_t* tile_off, int64_t nbuckets,
                           int32_t* run_off, float* kv_part, float* dq_part, float* dq, float* delta, float* dk,
                           float* dv, bool bf, int64_t batch, int64_t seq_len, int64_t hq, int64_t hkv, int64_t d,
                           int64_t q_start, int64_t q_len, int block, int topk, float scale, hipStream_t s) {
  if (batch * q_len * hq == 0) return hipSuccess;
#define QAT_BWD(T_, D_)                                                                                     \
  return launch_moba_bwd_d<T_, D_>((const T_*)q, (const T_*)k, (const T_*)v, blk,                          \
                                   (const T_*)dout, lse, tiles, ntiles, entries, max_tiles, tile_off, nbuckets, \
                                   run_off, kv_part, dq_part, dq, delta,                                        \
                                   dk, dv, batch, seq_len, hq, hkv, q_start, q_len, block, topk, scale, s)
  if (bf) {
    if (d == 64) QAT_BWD(bf16, 64);
    QAT_BWD(bf16, 128);
  }
  if (d == 64) QAT_BWD(float, 64);
  QAT_BWD(float, 128);
#undef QAT_BWD
}

}  // namespace qat
