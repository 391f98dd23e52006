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
// Three kernels, vector float32 arithmetic:
//   dq      one wave per row, four 16-lane groups taking every fourth key of
//           the row's set; p comes straight from the forward lse (no running
//           max), and D is accumulated in the same pass through
//           dq = scale (sum p dp k - D sum p k);
//   own     a workgroup per (sequence, KV head, 64 keys of a block): the
//           block's own rows (positions in the block, every query head of
//           the group, causal); writes dk, dv of its keys (every key of the
//           sequence is written by exactly one workgroup);
//   gated   a workgroup per (run of dispatch tiles, 64 keys of the block):
//           the rows that gated the block, as bucketed by the forward
//           dispatch; adds into dk, dv with float atomics, once per bucket
//           the run touches.
// In the two key kernels, lane (key i, quarter c) of a wave holds dims
// [c D/4, (c+1) D/4) of key i's K, V, dK and dV; rows pass through LDS 16 at
// a time as float32 (quarters padded against bank conflicts).
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace qat {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kBwdKeys = 64;   // keys per workgroup of the key kernels (16 per wave)
constexpr int kBwdRows = 16;   // rows staged per LDS round
constexpr int kBwdTilesPerWg = 8;

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

// ---------------------------------------------------------------------------
int moba_bwd_chunks(int block) { return (int)cdiv(block, kBwdKeys); }

hipError_t launch_moba_bwd(const void* q, const void* k, const void* v, const int32_t* blk, const void* dout,
                           const float* lse, const int4* tiles, const int32_t* ntiles, const int2* entries,
                           int64_t max_tiles, float* dq, float* delta, float* dk, float* dv, bool bf,
                           int64_t batch, int64_t seq_len, int64_t hq, int64_t hkv, int64_t d, int64_t q_start,
                           int64_t q_len, int block, int topk, float scale, hipStream_t s) {
  const int64_t rows = batch * q_len * hq;
  const int cpb = moba_bwd_chunks(block);
  const int64_t nb_all = cdiv(seq_len, block);
  dim3 g_dq((unsigned)cdiv(rows, 4));
  dim3 g_own((unsigned)(nb_all * cpb), (unsigned)hkv, (unsigned)batch);
  dim3 g_gt((unsigned)std::max<int64_t>(1, cdiv(max_tiles, kBwdTilesPerWg)), (unsigned)cpb);
#define QAT_BWD(T_, D_)                                                                                      \
  do {                                                                                                       \
    {                                                                                                        \
      KTimer tm_("moba_bwd_dq", s);                                                                          \
      launch_timed("moba_bwd_dq", moba_bwd_dq_kernel<T_, D_>, g_dq, dim3(256), 0, s, (const T_*)q,           \
                   (const T_*)k, (const T_*)v, blk, (const T_*)dout, lse, dq, delta, rows, seq_len, hq, hkv,  \
                   q_start, q_len, block, topk, scale);                                                      \
    }                                                                                                        \
    if ((e = hipGetLastError()) != hipSuccess) return e;                                                     \
    {                                                                                                        \
      KTimer tm_("moba_bwd_own", s);                                                                         \
      launch_timed("moba_bwd_own", moba_bwd_own_kernel<T_, D_>, g_own, dim3(256), 0, s, (const T_*)q,        \
                   (const T_*)k, (const T_*)v, (const T_*)dout, lse, (const float*)delta, dk, dv, seq_len,  \
                   hq, hkv, q_start, q_len, block, cpb, scale);                                              \
    }                                                                                                        \
    if ((e = hipGetLastError()) != hipSuccess) return e;                                                     \
    if (topk > 1 && max_tiles > 0) {                                                                         \
      KTimer tm_("moba_bwd_gated", s);                                                                       \
      launch_timed("moba_bwd_gated", moba_bwd_gated_kernel<T_, D_>, g_gt, dim3(256), 0, s, (const T_*)q,     \
                   (const T_*)k, (const T_*)v, (const T_*)dout, lse, (const float*)delta, tiles, ntiles,     \
                   entries, dk, dv, hkv, block, scale);                                                      \
    }                                                                                                        \
  } while (0)
  hipError_t e = hipSuccess;
  if (rows == 0) return e;
  if (bf) {
    if (d == 64) QAT_BWD(bf16, 64);
    else QAT_BWD(bf16, 128);
  } else {
    if (d == 64) QAT_BWD(float, 64);
    else QAT_BWD(float, 128);
  }
#undef QAT_BWD
  return hipGetLastError();
}

}  // namespace qat
