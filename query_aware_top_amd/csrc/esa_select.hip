// ESA token selection: compressed scoring, score correction, importance
// summed over the chunk's queries, neighbour influence and exact top-k.
//
// ESA write-up (hlszyjy.com/post/6872.html): importance of a middle token is
// the product of query and key, taking every query of the current chunk into
// account (decode: the one query), with all heads merged into one score and
// q/k compressed to a low dimension; scores are corrected so that relative
// size is kept and no single token dominates; a token's score is also shaped
// by its neighbours; the top-k tokens are kept so the attended key count is
// fixed. The two dropped formulas are read as
//   correction  s^_ij = max(s_ij - max_j' s_ij', -clip)
//   neighbours  u'_j  = max{u_t : t in M, |t - j| <= r}
// and the importance as u_j = sum_i s^_ij. The alternative reading of the
// correction (per-query softmax votes, s^_ij = exp(tau s_ij) / sum_j'
// exp(tau s_ij')) is the VOTE instantiation: pass 1 also keeps each query's
// running sum of exp2(tau2 (s - running max)) (tau2 = tau log2 e), the final
// pass turns (max, sum) into the log2 normaliser c_i = tau2 max + log2 sum,
// and pass 2 adds exp2(tau2 s_ij - c_i).
//
// Prefill scoring runs on the bf16 matrix cores with q~ (float32) split into
// two bf16 terms (hi + lo): the products with the bf16 compressed keys are
// exact and the float32 sums carry ~2^-17 relative error, far inside the
// selection tolerance. Decode scoring is a float32 matrix-vector stream
// (HBM-bound). Top-k is an exact radix select on order-preserving uint32
// keys with the lowest index winning ties.
//
// Per-head selection (the other arm of the write-up's ablation on head
// merging): each (sequence, head) is its own selection, scored with the
// head's uncompressed bf16 q and k rows (one bf16 term, products exact), so
// the same kernels run over "selections" v = b H + h with the operands'
// addresses given by ScGeom.
#include <algorithm>

#include "attn_core.h"
#include "common.h"
#include "launch.h"

namespace qat {

// ---------------------------------------------------------------------------
// Prefill scoring. Both passes stream 64-row tiles of one operand through LDS
// (direct global->LDS loads, double-buffered, one barrier per tile, the next
// tile's loads in flight during the current tile's matrix ops) and hold the
// other operand in registers; rows are stored with the attention engine's
// chunk swizzle so the A-operand reads are bank-conflict free.
// Clears the top-k histograms of the selections (n ints at h; h may be
// NULL): the scoring kernels do it as a side job, since the top-k passes
// that count into them run after the scoring in stream order.
__device__ __forceinline__ void clear_topk_hist(int32_t* __restrict__ h, int64_t n) {
  if (!h) return;
  const int64_t nthr = (int64_t)gridDim.x * gridDim.y * gridDim.z * blockDim.x;
  const int64_t wg = ((int64_t)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
  for (int64_t i = wg * blockDim.x + threadIdx.x; i < n; i += nthr) h[i] = 0;
}

constexpr int kScWaves = 4;

constexpr int kScRows = 32 * kScWaves;   // register-held rows per workgroup

// A operand (32 rows x 16 k) of sub-tile sb, k-step c, from a swizzled tile
template <int DC>
__device__ __forceinline__ bf16x8 sc_a(const bf16* tile, int sb, int c) {
  const int lane = threadIdx.x & 63;
  const int r = sb * 32 + (lane & 31);
  const int ch = (2 * c + (lane >> 5)) ^ fa_swz<DC>(r);
  return *(const bf16x8*)(tile + r * DC + ch * 8);
}

// Pass 1: partial row maxima. grid (query tiles of 128, key splits, batch);
// S^T = K~ Q~^T with Q~ = hi + lo in registers, so each lane holds one query
// and 16 key scores per 32-key sub-tile.
// Online (max, sum of exp2(tau2 (x - max))) pairs: merge of two.
__device__ __forceinline__ void vote_merge(float& m, float& l, float om, float ol, float tau2) {
  const float mm = fmaxf(m, om);
  if (mm == -__builtin_inff()) return;
  l = l * __builtin_amdgcn_exp2f(tau2 * (m - mm)) + ol * __builtin_amdgcn_exp2f(tau2 * (om - mm));
  m = mm;
}

template <int DC, bool VOTE, bool HILO>
__global__ __launch_bounds__(64 * kScWaves) void esa_rowmax_kernel(
    const bf16* __restrict__ q_hi, const bf16* __restrict__ q_lo, const bf16* __restrict__ kc, ScGeom g,
    int64_t m, int64_t mid0, int64_t n_mid, int64_t keys_per_split, int nsplit,
    float tau2, float* __restrict__ rowmax_part, float* __restrict__ rowsum_part) {
  __shared__ __align__(16) bf16 kt0[kKT * DC];
  __shared__ __align__(16) bf16 kt1[kKT * DC];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, r32 = lane & 31;
  const int64_t bi = blockIdx.z;
  const int64_t qi = (int64_t)blockIdx.x * kScRows + wave * 32 + r32;
  const bool qvalid = qi < m;
  const int64_t qofs = g.qoff(bi) + (qvalid ? qi : 0) * g.q_row;
  bf16x8 qh[DC / 16], ql[DC / 16];
#pragma unroll
  for (int c = 0; c < DC / 16; ++c) {
    qh[c] = *(const bf16x8*)(q_hi + qofs + 16 * c + 8 * h);
    if constexpr (HILO) ql[c] = *(const bf16x8*)(q_lo + qofs + 16 * c + 8 * h);
  }
  const int64_t k0 = (int64_t)blockIdx.y * keys_per_split;
  const int n = (int)(min(n_mid, k0 + keys_per_split) - k0);
  const bf16* kbase = kc + g.koff(bi) + (mid0 + k0) * g.k_row;
  const int krow = (int)g.k_row;
  auto row_ofs = [krow](int j) { return j * krow; };
  const int nt = (n + kKT - 1) / kKT;
  float mx = -__builtin_inff(), lsum = 0.f;
  // one tile's scores folded into the running max (and vote sum); the loop
  // below runs tiles in pairs so that each call reads a fixed LDS buffer
  auto tile_max = [&](const bf16* tile, int t) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      f32x16 acc = {};
#pragma unroll
      for (int c = 0; c < DC / 16; ++c) {
        const bf16x8 a = sc_a<DC>(tile, sb, c);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qh[c], acc, 0, 0, 0);
        if constexpr (HILO) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, ql[c], acc, 0, 0, 0);
      }
      const int base = t * kKT + sb * 32;
      if constexpr (VOTE) {
        auto vote = [&](auto masked_c) {   // keys past the split's end only in its last tile
          constexpr bool MK = decltype(masked_c)::value;
          float tm = -__builtin_inff();
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (!MK || base + (i >> 2) * 8 + h * 4 + (i & 3) < n) tm = fmaxf(tm, acc[i]);
          const float mn = fmaxf(mx, tm);
          if (mn != -__builtin_inff()) {
            float add = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i)
              if (!MK || base + (i >> 2) * 8 + h * 4 + (i & 3) < n) add += __builtin_amdgcn_exp2f(tau2 * (acc[i] - mn));
            lsum = lsum * __builtin_amdgcn_exp2f(tau2 * (mx - mn)) + add;
            mx = mn;
          }
        };
        if (base + 32 <= n) vote(std::false_type{});
        else vote(std::true_type{});
      } else if (base + 32 <= n) {
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, acc[i]);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (base + (i >> 2) * 8 + h * 4 + (i & 3) < n) mx = fmaxf(mx, acc[i]);
      }
    }
  };
  fa_issue_one<DC, kScWaves>(kt0, kbase, 0, n, row_ofs);
  for (int t = 0; t < nt; t += 2) {
    fa_wait_loads();
    __syncthreads();
    if (t + 1 < nt) fa_issue_one<DC, kScWaves>(kt1, kbase, (t + 1) * kKT, n, row_ofs);
    tile_max(kt0, t);
    if (t + 1 >= nt) break;
    fa_wait_loads();
    __syncthreads();
    if (t + 2 < nt) fa_issue_one<DC, kScWaves>(kt0, kbase, (t + 2) * kKT, n, row_ofs);
    tile_max(kt1, t + 1);
  }
  if constexpr (VOTE) {
    vote_merge(mx, lsum, __shfl_xor(mx, 32, 64), __shfl_xor(lsum, 32, 64), tau2);
    if (qvalid && h == 0) rowsum_part[(bi * m + qi) * nsplit + blockIdx.y] = lsum;
  } else {
    mx = xor32_max(mx);
  }
  if (qvalid && h == 0) rowmax_part[(bi * m + qi) * nsplit + blockIdx.y] = mx;
}

// One wave per query row: the row's partial maxima are read contiguously
// and reduced across the wave. VOTE: the (max, sum) pairs are merged and the
// row's log2 normaliser tau2 max + log2 sum is stored instead of the max.
template <bool VOTE>
__global__ __launch_bounds__(256) void esa_rowmax_final_kernel(const float* __restrict__ part,
                                                               const float* __restrict__ sum_part, int nsplit,
                                                               int64_t rows, float tau2, float* __restrict__ rowmax) {
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= rows) return;
  float mx = -__builtin_inff(), l = 0.f;
  for (int s = lane; s < nsplit; s += 64) {
    if constexpr (VOTE) vote_merge(mx, l, part[i * nsplit + s], sum_part[i * nsplit + s], tau2);
    else mx = fmaxf(mx, part[i * nsplit + s]);
  }
  for (int off = 32; off >= 1; off >>= 1) {
    if constexpr (VOTE) vote_merge(mx, l, __shfl_xor(mx, off, 64), __shfl_xor(l, off, 64), tau2);
    else mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  }
  if (lane == 0) rowmax[i] = VOTE ? tau2 * mx + __builtin_log2f(l) : mx;
}

// Pass 2: partial importance. grid (key tiles of 128, query splits, batch);
// S = Q~ K~^T with the keys in registers, so each lane holds one key and 16
// query rows per 32-query sub-tile; the corrected scores are summed in
// float32 per sub-tile and in float64 across sub-tiles (fixed order).
template <int DC, bool VOTE, bool HILO>
__global__ __launch_bounds__(64 * kScWaves) void esa_colsum_kernel(
    const bf16* __restrict__ q_hi, const bf16* __restrict__ q_lo, const float* __restrict__ rowmax,
    const bf16* __restrict__ kc, ScGeom g, int64_t m, int64_t mid0, int64_t n_mid,
    int64_t rows_per_split, int nqsplit, float clip, float tau2, float* __restrict__ upart,
    int32_t* __restrict__ hist0, int64_t nhist) {
  __shared__ __align__(16) bf16 qh0[kKT * DC];
  __shared__ __align__(16) bf16 qh1[kKT * DC];
  __shared__ __align__(16) bf16 ql0[HILO ? kKT * DC : 8];
  __shared__ __align__(16) bf16 ql1[HILO ? kKT * DC : 8];
  __shared__ __align__(16) float rm0[kKT];
  __shared__ __align__(16) float rm1[kKT];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, r32 = lane & 31;
  const int64_t bi = blockIdx.z;
  const int64_t key = (int64_t)blockIdx.x * kScRows + wave * 32 + r32;
  const bool kvalid = key < n_mid;
  const bf16* kr = kc + g.koff(bi) + (mid0 + (kvalid ? key : 0)) * g.k_row;
  bf16x8 kf[DC / 16];
#pragma unroll
  for (int c = 0; c < DC / 16; ++c) kf[c] = *(const bf16x8*)(kr + 16 * c + 8 * h);
  const int64_t i0 = (int64_t)blockIdx.y * rows_per_split;
  const int n = (int)(min(m, i0 + rows_per_split) - i0);
  const bf16* hb = q_hi + g.qoff(bi) + i0 * g.q_row;
  const bf16* lb = HILO ? q_lo + g.qoff(bi) + i0 * g.q_row : nullptr;
  const float* rb = rowmax + bi * m + i0;
  const int qrow = (int)g.q_row;
  auto row_ofs = [qrow](int j) { return j * qrow; };
  auto issue = [&](int t) {
    const int j0 = t * kKT;
    fa_issue_one<DC, kScWaves>((t & 1) ? qh1 : qh0, hb, j0, n, row_ofs);
    if constexpr (HILO) fa_issue_one<DC, kScWaves>((t & 1) ? ql1 : ql0, lb, j0, n, row_ofs);
    if (wave == 0) {
      const int j = min(j0 + lane, n - 1);
      __builtin_amdgcn_global_load_lds((const global_void*)(rb + j), (lds_void*)((t & 1) ? rm1 : rm0), 4, 0, 0);
    }
  };
  const int nt = (n + kKT - 1) / kKT;
  double total = 0.0;
  // One tile's scores and their clamped sum; buffers fixed per call site (the
  // loop below runs tiles in pairs), and only a tile that reaches past the
  // chunk's last row masks its rows.
  auto tile_sum = [&](const bf16* th, const bf16* tl, const float* trm, int t, auto masked_c) {
    constexpr bool MASKED = decltype(masked_c)::value;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      f32x16 acc = {};
#pragma unroll
      for (int c = 0; c < DC / 16; ++c) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sc_a<DC>(th, sb, c), kf[c], acc, 0, 0, 0);
        if constexpr (HILO) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sc_a<DC>(tl, sb, c), kf[c], acc, 0, 0, 0);
      }
      const int base = t * kKT + sb * 32;
      float part = 0.f;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 r4 = *(const f32x4*)(trm + sb * 32 + g * 8 + h * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = VOTE ? __builtin_amdgcn_exp2f(tau2 * acc[4 * g + e] - r4[e])
                               : fmaxf(acc[4 * g + e] - r4[e], -clip);
          if constexpr (MASKED) part += (base + g * 8 + h * 4 + e < n) ? v : 0.f;
          else part += v;
        }
      }
      total += (double)part;
    }
  };
  auto tile = [&](const bf16* th, const bf16* tl, const float* trm, int t) {
    if ((t + 1) * kKT <= n) tile_sum(th, tl, trm, t, std::false_type{});
    else tile_sum(th, tl, trm, t, std::true_type{});
  };
  issue(0);
  if constexpr (DC <= 128) {
    for (int t = 0; t < nt; t += 2) {
      fa_wait_loads();
      __syncthreads();
      if (t + 1 < nt) issue(t + 1);
      tile(qh0, ql0, rm0, t);
      if (t + 1 >= nt) break;
      fa_wait_loads();
      __syncthreads();
      if (t + 2 < nt) issue(t + 2);
      tile(qh1, ql1, rm1, t + 1);
    }
  } else {   // d_c 256: one copy of the tile code (four would not fit the registers)
    for (int t = 0; t < nt; ++t) {
      fa_wait_loads();
      __syncthreads();
      if (t + 1 < nt) issue(t + 1);
      tile_sum((t & 1) ? qh1 : qh0, (t & 1) ? ql1 : ql0, (t & 1) ? rm1 : rm0, t, std::true_type{});
    }
  }
  total += __shfl_xor(total, 32, 64);
  if (kvalid && h == 0) upart[(bi * nqsplit + blockIdx.y) * n_mid + key] = (float)total;
  clear_topk_hist(hist0, nhist);
}

constexpr int kScanUnroll = 8;

// ---------------------------------------------------------------------------
// Decode scoring: s_j = <q~, k~_j> (float32) for every middle token, plus the
// workgroup maxima. DC/8 lanes per key, 8 elements (16 B) per lane.
// VOTE: also the workgroup's sum of exp2(tau2 (s - workgroup max)), counted
// once per key (by the key's first lane).
template <int DC, bool VOTE, typename QT>
__global__ __launch_bounds__(256) void esa_decode_scan_kernel(
    const QT* __restrict__ qc, const bf16* __restrict__ kc, ScGeom g, int64_t mid0, int64_t n_mid,
    int64_t keys_per_wg, float tau2, float* __restrict__ s_out, float* __restrict__ smax_part,
    float* __restrict__ ssum_part, int32_t* __restrict__ hist0, int64_t nhist) {
  constexpr int LPK = DC / 8;          // lanes per key
  constexpr int KPW = 256 / LPK;       // keys per workgroup pass
  __shared__ float wmax[4], wsum[4];
  const int64_t bi = blockIdx.y;
  const int tid = threadIdx.x;
  const int sub = tid % LPK;
  float qv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) qv[j] = (float)qc[g.qoff(bi) + sub * 8 + j];
  const int64_t k0 = (int64_t)blockIdx.x * keys_per_wg;
  const int64_t k1 = min(n_mid, k0 + keys_per_wg);
  const bf16* kbase = kc + g.koff(bi) + mid0 * g.k_row;
  float mx = -__builtin_inff(), lsum = 0.f;
  // kScanUnroll keys per lane group in flight at once
  constexpr int U = kScanUnroll;
  for (int64_t kb = k0; kb < k1; kb += (int64_t)KPW * U) {
    bf16x8 kv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t key = min(kb + (int64_t)u * KPW + tid / LPK, k1 - 1);
      kv[u] = *(const bf16x8*)(kbase + key * g.k_row + sub * 8);
    }
    float acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      acc[u] = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[u] = fmaf(qv[j], (float)kv[u][j], acc[u]);
    }
#pragma unroll
    for (int off = 1; off < LPK; off <<= 1)
#pragma unroll
      for (int u = 0; u < U; ++u) acc[u] += __shfl_xor(acc[u], off, 64);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t key = kb + (int64_t)u * KPW + tid / LPK;
      if (key < k1) {
        if (sub == 0) s_out[bi * n_mid + key] = acc[u];
        if (VOTE && sub == 0) vote_merge(mx, lsum, acc[u], 1.f, tau2);
        else mx = fmaxf(mx, acc[u]);
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    if constexpr (VOTE) vote_merge(mx, lsum, __shfl_xor(mx, off, 64), __shfl_xor(lsum, off, 64), tau2);
    else mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  }
  if ((tid & 63) == 0) { wmax[tid >> 6] = mx; wsum[tid >> 6] = lsum; }
  __syncthreads();
  if (tid == 0) {
    float m2 = wmax[0], l2 = wsum[0];
    for (int w = 1; w < 4; ++w) {
      if constexpr (VOTE) vote_merge(m2, l2, wmax[w], wsum[w], tau2);
      else m2 = fmaxf(m2, wmax[w]);
    }
    smax_part[bi * gridDim.x + blockIdx.x] = m2;
    if (VOTE) ssum_part[bi * gridDim.x + blockIdx.x] = l2;
  }
  clear_topk_hist(hist0, nhist);
}

// ---------------------------------------------------------------------------
// Top-k over the middle part, several workgroups per sequence, each owning a
// slice of 256 PER consecutive candidates (PER per thread, contiguous):
//   prep   u_j (mode 0, prefill: the query-split partial sums added in
//          float64 in split order; mode 1, decode: max(s_j - max s, -clip);
//          mode 2, decode with votes: exp2(tau2 (s_j - max s)) / sum),
//          u'_j = max of u over |t - j| <= r within M (halo recomputed from
//          the inputs), order-preserving uint32 keys, histogram of the top
//          11 key bits;
//   hist   (twice) the next 11 / 10 bits of the keys that match the digits
//          fixed so far;
//   count  keys above / equal to the k-th largest key T, per slice;
//   emit   stable compaction: every key above T, and the lowest-index keys
//          equal to T up to k, in ascending position order.
// Each kernel re-derives the digits fixed so far from the global
// histograms (2048 bins, cheap), so no state passes between them. prep,
// hist and count visit the slice with stride 256 (element e of thread t is
// candidate e*256 + t: every load and store is coalesced); emit stages the
// slice's keys in LDS with the same coalesced loads and then gives each
// thread PER consecutive candidates, as the stable compaction needs.
constexpr int kTkThreads = 256;
constexpr int kTkPerMin = 2;   // candidates per thread: 2 to 32, so that a pass has >= 256 workgroups where it can
constexpr int kTkMaxRadius = 1024;
constexpr int kTkWin = 4;      // radii up to this use an unrolled neighbour window
constexpr int kTkBins = 2048;
__host__ __device__ constexpr int tk_shift(int pass) { return pass == 0 ? 21 : pass == 1 ? 10 : 0; }
__host__ __device__ constexpr int tk_bits(int pass) { return pass == 2 ? 10 : 11; }

// exclusive prefix sum over the workgroup's 256 threads; *total = the sum
__device__ __forceinline__ int32_t tk_scan(int32_t v, int32_t* s_w, int32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_w[wave] = x;
  __syncthreads();
  int32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kTkThreads / 64; ++w) {
    before += w < wave ? s_w[w] : 0;
    all += s_w[w];
  }
  __syncthreads();
  if (total) *total = all;
  return before + x - v;
}

// Digits of the k-th largest key fixed by histogram passes [0, npass):
// prefix/mask of the fixed bits and how many keys with that prefix are
// still to be taken (1 <= need). Uniform over the workgroup.
struct TkCut {
  uint32_t prefix, mask;
  int32_t need;
};

__device__ TkCut tk_cut(const int32_t* __restrict__ hist, int npass, int32_t k, int32_t* s_w, TkCut* s_cut) {
  TkCut cut{0u, 0u, k};
  // the bins of all three passes are read at once (one memory round trip;
  // the histogram array always holds three passes)
  int32_t cc[3][8];
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int nb = 1 << tk_bits(pass);
    const int per = nb / kTkThreads;   // 8 or 4 bins per thread, descending
#pragma unroll
    for (int p = 0; p < 8; ++p) cc[pass][p] = p < per ? hist[pass * kTkBins + nb - 1 - (threadIdx.x * per + p)] : 0;
  }
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    if (pass >= npass) break;
    const int nb = 1 << tk_bits(pass);
    const int per = nb / kTkThreads;
    const int32_t* c = cc[pass];
    int32_t local = 0;
#pragma unroll
    for (int p = 0; p < 8; ++p) local += c[p];
    int32_t acc = tk_scan(local, s_w, nullptr);
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      if (p < per && acc < cut.need && acc + c[p] >= cut.need) {
        const int bin = nb - 1 - (threadIdx.x * per + p);
        s_cut->prefix = cut.prefix | ((uint32_t)bin << tk_shift(pass));
        s_cut->mask = cut.mask | ((uint32_t)(nb - 1) << tk_shift(pass));
        s_cut->need = cut.need - acc;
      }
      acc += c[p];
    }
    __syncthreads();
    cut = *s_cut;
    __syncthreads();
  }
  return cut;
}

template <int PER>
__global__ __launch_bounds__(kTkThreads) void esa_topk_prep_kernel(
    int mode, const float* __restrict__ upart, int nqsplit, const float* __restrict__ s_in,
    const float* __restrict__ smax_part, const float* __restrict__ ssum_part, int nsmax, float clip, float tau2,
    int64_t n_mid, int radius, uint32_t* __restrict__ keys, float* __restrict__ scores_out,
    int32_t* __restrict__ hist) {
  __shared__ float s_u[kTkThreads * PER + 2 * kTkMaxRadius];
  __shared__ int32_t s_h[kTkBins];
  __shared__ float s_red[kTkThreads / 64], s_rsum[kTkThreads / 64];
  const int tid = threadIdx.x;
  const int64_t bi = blockIdx.y;
  const int64_t j0 = (int64_t)blockIdx.x * (kTkThreads * PER);
  float mx = 0.f, inv_l = 1.f;
  if (mode == 1) {   // max of the raw scores over M, from the scan's per-workgroup maxima
    float m = -__builtin_inff();
    for (int sp = tid; sp < nsmax; sp += kTkThreads) m = fmaxf(m, smax_part[bi * nsmax + sp]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    if ((tid & 63) == 0) s_red[tid >> 6] = m;
    __syncthreads();
    mx = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  } else if (mode == 2) {   // max and softmax denominator over M, from the scan's per-workgroup pairs
    float m = -__builtin_inff(), l = 0.f;
    for (int sp = tid; sp < nsmax; sp += kTkThreads)
      vote_merge(m, l, smax_part[bi * nsmax + sp], ssum_part[bi * nsmax + sp], tau2);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) vote_merge(m, l, __shfl_xor(m, off, 64), __shfl_xor(l, off, 64), tau2);
    if ((tid & 63) == 0) { s_red[tid >> 6] = m; s_rsum[tid >> 6] = l; }
    __syncthreads();
    m = s_red[0];
    l = s_rsum[0];
    for (int w = 1; w < kTkThreads / 64; ++w) vote_merge(m, l, s_red[w], s_rsum[w], tau2);
    mx = m;
    inv_l = 1.f / l;
  }
  for (int i = tid; i < kTkBins; i += kTkThreads) s_h[i] = 0;
  // element jl of the slice (jl in [-lo_ok, nl + hi_ok): the slice and its
  // halo of up to r elements on each side, clipped to M) goes to
  // s_u[jl + radius]
  const int nl = (int)min((int64_t)(kTkThreads * PER), n_mid - j0);
  const int lo_ok = (int)min((int64_t)radius, j0);
  const int hi_ok = (int)min((int64_t)radius, n_mid - j0 - nl);
  const int nh = lo_ok + hi_ok;
  if (nh <= kTkThreads) {
    // one round: PER slice elements per thread plus, for the first nh
    // threads, one halo element, all loads in flight together (clamped
    // positions, results masked)
    const int hh = min(tid, max(nh - 1, 0));
    const int hl = hh < lo_ok ? hh - lo_ok : nl + (hh - lo_ok);   // slice-local index of the halo element
    int64_t jg[PER + 1];
#pragma unroll
    for (int e = 0; e < PER; ++e) jg[e] = j0 + min(e * kTkThreads + tid, nl - 1);
    jg[PER] = j0 + min(max(hl, -lo_ok), nl - 1 + hi_ok);
    float uv[PER + 1];
    if (mode == 0) {   // the query-split partial sums, added in float64 in split order
      double acc[PER + 1];
#pragma unroll
      for (int e = 0; e <= PER; ++e) acc[e] = 0.0;
      for (int sp = 0; sp < nqsplit; ++sp) {
        float t[PER + 1];
#pragma unroll
        for (int e = 0; e <= PER; ++e) t[e] = upart[(bi * nqsplit + sp) * n_mid + jg[e]];
#pragma unroll
        for (int e = 0; e <= PER; ++e) acc[e] += (double)t[e];
      }
#pragma unroll
      for (int e = 0; e <= PER; ++e) uv[e] = (float)acc[e];
    } else {
      float t[PER + 1];
#pragma unroll
      for (int e = 0; e <= PER; ++e) t[e] = s_in[bi * n_mid + jg[e]];
#pragma unroll
      for (int e = 0; e <= PER; ++e)
        uv[e] = mode == 2 ? __builtin_amdgcn_exp2f(tau2 * (t[e] - mx)) * inv_l : fmaxf(t[e] - mx, -clip);
    }
#pragma unroll
    for (int e = 0; e < PER; ++e)
      if (e * kTkThreads + tid < nl) s_u[e * kTkThreads + tid + radius] = uv[e];
    if (tid < nh) s_u[hl + radius] = uv[PER];
  } else {
    // u over [j0 - r, j0 + slice + r) clipped to M, PER values per thread and
    // round with all their loads in flight (clamped indices, results masked)
    const int64_t lo = max((int64_t)0, j0 - radius);
    const int64_t hi = min(n_mid, j0 + (kTkThreads * PER) + radius);
    for (int64_t jb = lo; jb < hi; jb += (int64_t)kTkThreads * PER) {
      float uv[PER];
      if (mode == 0) {   // the query-split partial sums, added in float64 in split order
        double acc[PER];
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = 0.0;
        for (int sp = 0; sp < nqsplit; ++sp) {
          float t[PER];
#pragma unroll
          for (int e = 0; e < PER; ++e) t[e] = upart[(bi * nqsplit + sp) * n_mid + min(jb + e * kTkThreads + tid, hi - 1)];
#pragma unroll
          for (int e = 0; e < PER; ++e) acc[e] += (double)t[e];
        }
#pragma unroll
        for (int e = 0; e < PER; ++e) uv[e] = (float)acc[e];
      } else {
        float t[PER];
#pragma unroll
        for (int e = 0; e < PER; ++e) t[e] = s_in[bi * n_mid + min(jb + e * kTkThreads + tid, hi - 1)];
#pragma unroll
        for (int e = 0; e < PER; ++e)
          uv[e] = mode == 2 ? __builtin_amdgcn_exp2f(tau2 * (t[e] - mx)) * inv_l : fmaxf(t[e] - mx, -clip);
      }
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const int64_t j = jb + e * kTkThreads + tid;
        if (j < hi) s_u[j - j0 + radius] = uv[e];
      }
    }
  }
  __syncthreads();
  // neighbour max in slice-local 32-bit indices: the window [jl - r, jl + r]
  // of element jl, clipped to the middle part
  auto emit_key = [&](int jl, float v) {
    const int64_t j = j0 + jl;
    const uint32_t key = float_key(v);
    keys[bi * n_mid + j] = key;
    if (scores_out) scores_out[bi * n_mid + j] = v;
    atomicAdd(&s_h[key >> tk_shift(0)], 1);
  };
  if (radius <= kTkWin) {
    // a fixed window of 2 kTkWin + 1 reads per element, masked to the
    // radius: every read of the thread's elements is issued at once (a
    // loop of runtime length would wait for each read in turn)
    float vv[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int jl = min(e * kTkThreads + tid, nl - 1);
      float v = s_u[jl + radius];
#pragma unroll
      for (int d = -kTkWin; d <= kTkWin; ++d) {
        const int t = min(max(jl + d, -lo_ok), nl - 1 + hi_ok);
        const float w = s_u[t + radius];
        v = (d >= -radius && d <= radius) ? fmaxf(v, w) : v;
      }
      vv[e] = v;
    }
#pragma unroll
    for (int e = 0; e < PER; ++e)
      if (e * kTkThreads + tid < nl) emit_key(e * kTkThreads + tid, vv[e]);
  } else {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int jl = e * kTkThreads + tid;
      if (jl >= nl) break;
      float v = s_u[jl + radius];
      const int a = max(jl - radius, -lo_ok), b = min(jl + radius, nl - 1 + hi_ok);
      for (int t = a; t <= b; ++t) v = fmaxf(v, s_u[t + radius]);
      emit_key(jl, v);
    }
  }
  __syncthreads();
  int32_t* gh = hist + bi * 3 * kTkBins;
  for (int i = tid; i < kTkBins; i += kTkThreads)
    if (s_h[i]) atomicAdd(&gh[i], s_h[i]);
}

template <int PER>
__global__ __launch_bounds__(kTkThreads) void esa_topk_hist_kernel(int pass, const uint32_t* __restrict__ keys,
                                                                   int64_t n_mid, int topk,
                                                                   int32_t* __restrict__ hist) {
  __shared__ int32_t s_h[kTkBins];
  __shared__ int32_t s_w[kTkThreads / 64];
  __shared__ TkCut s_cut;
  const int64_t bi = blockIdx.y;
  int32_t* gh = hist + bi * 3 * kTkBins;
  const TkCut cut = tk_cut(gh, pass, topk, s_w, &s_cut);
  const int nb = 1 << tk_bits(pass);
  for (int i = threadIdx.x; i < nb; i += kTkThreads) s_h[i] = 0;
  __syncthreads();
  const int64_t j0 = (int64_t)blockIdx.x * (kTkThreads * PER) + threadIdx.x;
  uint32_t kv[PER];   // all loads in flight at once (clamped indices, masked below)
#pragma unroll
  for (int e = 0; e < PER; ++e) kv[e] = keys[bi * n_mid + min(j0 + e * kTkThreads, n_mid - 1)];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const uint32_t key = kv[e];
    if (j0 + e * kTkThreads < n_mid && (key & cut.mask) == cut.prefix)
      atomicAdd(&s_h[(key >> tk_shift(pass)) & (nb - 1)], 1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nb; i += kTkThreads)
    if (s_h[i]) atomicAdd(&gh[pass * kTkBins + i], s_h[i]);
}

// per slice: (#keys > T, #keys == T)
template <int PER>
__global__ __launch_bounds__(kTkThreads) void esa_topk_count_kernel(const uint32_t* __restrict__ keys,
                                                                    int64_t n_mid, int topk,
                                                                    const int32_t* __restrict__ hist,
                                                                    int2* __restrict__ wgcnt) {
  __shared__ int32_t s_w[kTkThreads / 64];
  __shared__ TkCut s_cut;
  const int64_t bi = blockIdx.y;
  const TkCut cut = tk_cut(hist + bi * 3 * kTkBins, 3, topk, s_w, &s_cut);
  const uint32_t T = cut.prefix;
  const int64_t j0 = (int64_t)blockIdx.x * (kTkThreads * PER) + threadIdx.x;
  int32_t gt = 0, eq = 0;
  uint32_t kv[PER];   // all loads in flight at once (clamped indices, masked below)
#pragma unroll
  for (int e = 0; e < PER; ++e) kv[e] = keys[bi * n_mid + min(j0 + e * kTkThreads, n_mid - 1)];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const bool in = j0 + e * kTkThreads < n_mid;
    gt += in && kv[e] > T;
    eq += in && kv[e] == T;
  }
  int32_t tgt, teq;
  tk_scan(gt, s_w, &tgt);
  tk_scan(eq, s_w, &teq);
  if (threadIdx.x == 0) wgcnt[bi * gridDim.x + blockIdx.x] = make_int2(tgt, teq);
}

template <int PER>
__global__ __launch_bounds__(kTkThreads) void esa_topk_emit_kernel(const uint32_t* __restrict__ keys,
                                                                   int64_t n_mid, int topk, int64_t mid0,
                                                                   const int32_t* __restrict__ hist,
                                                                   const int2* __restrict__ wgcnt,
                                                                   int32_t* __restrict__ sel,
                                                                   int32_t* __restrict__ n_sel) {
  __shared__ int32_t s_w[kTkThreads / 64];
  __shared__ TkCut s_cut;
  __shared__ uint32_t s_k[kTkThreads * (PER + 1)];   // one pad word per PER: conflict-free reads
  const int64_t bi = blockIdx.y;
  const int nwg = gridDim.x;
  int32_t* osel = sel + bi * topk;
  const int64_t nsel = min((int64_t)topk, n_mid);
  if (blockIdx.x == 0) {
    if (threadIdx.x == 0) n_sel[bi] = (int32_t)nsel;
    for (int64_t j = nsel + threadIdx.x; j < topk; j += kTkThreads) osel[j] = -1;
  }
  const int64_t j0 = (int64_t)blockIdx.x * (kTkThreads * PER) + threadIdx.x * PER;
  if (n_mid <= topk) {   // every candidate is selected
#pragma unroll
    for (int e = 0; e < PER; ++e)
      if (j0 + e < n_mid) osel[j0 + e] = (int32_t)(mid0 + j0 + e);
    return;
  }
  const TkCut cut = tk_cut(hist + bi * 3 * kTkBins, 3, topk, s_w, &s_cut);
  const uint32_t T = cut.prefix;
  const int32_t take_eq = cut.need;   // keys equal to T to take, lowest positions first
  // slices before this one: keys taken and keys equal to T seen
  int32_t out_before = 0, eq_before = 0;
  for (int w = threadIdx.x; w < (int)blockIdx.x; w += kTkThreads) {
    const int2 c = wgcnt[bi * nwg + w];
    eq_before += c.y;
    out_before += c.x;
  }
  int32_t eq_sum, gt_sum;
  tk_scan(eq_before, s_w, &eq_sum);
  tk_scan(out_before, s_w, &gt_sum);
  // equal keys taken before this slice = min(eq_sum, take_eq)
  const int32_t base = gt_sum + min(eq_sum, take_eq);
  int32_t gt = 0, eq = 0;
  uint32_t kv[PER];
  {   // the slice's keys through LDS: coalesced loads, then PER consecutive per thread
    const int64_t s0 = (int64_t)blockIdx.x * (kTkThreads * PER);
    uint32_t t[PER];   // all loads in flight at once (clamped indices, masked below)
#pragma unroll
    for (int e = 0; e < PER; ++e) t[e] = keys[bi * n_mid + min(s0 + e * kTkThreads + threadIdx.x, n_mid - 1)];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int64_t j = s0 + e * kTkThreads + threadIdx.x;
      const int jl = e * kTkThreads + threadIdx.x;
      s_k[jl + jl / PER] = j < n_mid ? t[e] : 0u;
    }
    __syncthreads();
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int64_t j = j0 + e;
    kv[e] = s_k[threadIdx.x * (PER + 1) + e];
    if (j < n_mid) {
      gt += kv[e] > T;
      eq += kv[e] == T;
    }
  }
  const int32_t eq_local = tk_scan(eq, s_w, nullptr);
  const int32_t eq_avail = max(0, take_eq - eq_sum - eq_local);   // equal keys this thread may still take
  const int32_t my_eq = min(eq, eq_avail);
  int32_t pos = base + tk_scan(gt + my_eq, s_w, nullptr);
  int32_t used = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int64_t j = j0 + e;
    if (j >= n_mid) break;
    bool take = kv[e] > T;
    if (kv[e] == T && used < my_eq) {
      take = true;
      ++used;
    }
    if (take) osel[pos++] = (int32_t)(mid0 + j);
  }
}

// ---------------------------------------------------------------------------
// about 1024 workgroups per pass; splits hold whole 64-row tiles
int esa_key_splits(int64_t n_mid, int64_t m) {
  const int64_t qt = cdiv(m, kScRows);
  int64_t ks = cdiv(1024, qt);
  const int64_t max_ks = cdiv(n_mid, 4 * kKT);
  if (ks > max_ks) ks = max_ks;
  return (int)(ks < 1 ? 1 : ks);
}
int esa_query_splits(int64_t n_mid, int64_t m) {
  const int64_t kt = cdiv(n_mid, kScRows);
  int64_t qs = cdiv(1024, kt);
  const int64_t max_qs = cdiv(m, 4 * kKT);
  if (qs > max_qs) qs = max_qs;
  return (int)(qs < 1 ? 1 : qs);
}
int esa_scan_wgs(int64_t n_mid) {
  const int64_t w = cdiv(n_mid, 2048);
  return (int)(w < 1 ? 1 : w);
}

template <int DC, bool VOTE, bool HILO>
static void launch_scores_dc(const bf16* q_hi, const bf16* q_lo, const bf16* kc, const ScGeom& g, dim3 g1, dim3 g2,
                             int64_t m, int64_t mid0, int64_t n_mid, int64_t kps, int ks_eff, int64_t rps, int qs_eff,
                             int64_t rows, float clip, float tau2, float* rowmax_part, float* rowsum_part,
                             float* rowmax, float* upart, int32_t* hist0, int64_t nhist, hipStream_t s) {
  launch_timed("esa_rowmax", esa_rowmax_kernel<DC, VOTE, HILO>, g1, dim3(64 * kScWaves), 0, s, q_hi, q_lo, kc, g, m,
               mid0, n_mid, kps, ks_eff, tau2, rowmax_part, rowsum_part);
  hipLaunchKernelGGL(esa_rowmax_final_kernel<VOTE>, dim3((unsigned)cdiv(rows, 4)), dim3(256), 0, s, rowmax_part,
                     rowsum_part, ks_eff, rows, tau2, rowmax);
  launch_timed("esa_colsum", esa_colsum_kernel<DC, VOTE, HILO>, g2, dim3(64 * kScWaves), 0, s, q_hi, q_lo, rowmax, kc,
               g, m, mid0, n_mid, rps, qs_eff, clip, tau2, upart, hist0, nhist);
}

hipError_t launch_esa_prefill_scores(const bf16* q_hi, const bf16* q_lo, const bf16* kc, const ScGeom& g,
                                     int64_t nsel, int64_t m, int64_t mid0, int64_t n_mid, int64_t dc, float clip,
                                     float tau2, float* rowmax_part, float* rowsum_part, float* rowmax,
                                     float* upart, int32_t* hist0, int64_t nhist, hipStream_t s) {
  if (n_mid <= 0) return hipSuccess;
  const bool vote = tau2 > 0.f;
  const int ks = esa_key_splits(n_mid, m);
  const int64_t kps = cdiv(cdiv(n_mid, ks), kKT) * kKT;
  const int ks_eff = (int)cdiv(n_mid, kps);
  const dim3 g1((unsigned)cdiv(m, kScRows), (unsigned)ks_eff, (unsigned)nsel);
  const int qs = esa_query_splits(n_mid, m);
  const int64_t rps = cdiv(cdiv(m, qs), kKT) * kKT;
  const int qs_eff = (int)cdiv(m, rps);
  const dim3 g2((unsigned)cdiv(n_mid, kScRows), (unsigned)qs_eff, (unsigned)nsel);
#define QAT_SC(DC_, HL_)                                                                                       \
  do {                                                                                                         \
    if (vote)                                                                                                  \
      launch_scores_dc<DC_, true, HL_>(q_hi, q_lo, kc, g, g1, g2, m, mid0, n_mid, kps, ks_eff, rps, qs_eff,    \
                                       nsel * m, clip, tau2, rowmax_part, rowsum_part, rowmax, upart, hist0, nhist, s);      \
    else                                                                                                       \
      launch_scores_dc<DC_, false, HL_>(q_hi, q_lo, kc, g, g1, g2, m, mid0, n_mid, kps, ks_eff, rps, qs_eff,   \
                                        nsel * m, clip, tau2, rowmax_part, rowsum_part, rowmax, upart, hist0, nhist, s);     \
  } while (0)
  if (q_lo) {
    switch (dc) {
      case 32: QAT_SC(32, true); break;
      case 64: QAT_SC(64, true); break;
      case 128: QAT_SC(128, true); break;
      default: QAT_SC(256, true); break;
    }
  } else if (dc == 64) {
    QAT_SC(64, false);
  } else {
    QAT_SC(128, false);
  }
#undef QAT_SC
  return hipGetLastError();
}

int esa_prefill_qsplits_eff(int64_t n_mid, int64_t m) {
  const int qs = esa_query_splits(n_mid, m);
  const int64_t rps = cdiv(cdiv(m, qs), kKT) * kKT;
  return (int)cdiv(m, rps);
}

template <int DC, typename QT>
static void launch_scan_dc(const QT* q, const bf16* kc, const ScGeom& g, dim3 grid, int64_t mid0, int64_t n_mid,
                           int64_t kpw, float tau2, float* s_out, float* smax_part, float* ssum_part,
                           int32_t* hist0, int64_t nhist, hipStream_t s) {
  if (tau2 > 0.f)
    launch_timed("esa_decode_scan", esa_decode_scan_kernel<DC, true, QT>, grid, dim3(256), 0, s, q, kc, g, mid0,
                 n_mid, kpw, tau2, s_out, smax_part, ssum_part, hist0, nhist);
  else
    launch_timed("esa_decode_scan", esa_decode_scan_kernel<DC, false, QT>, grid, dim3(256), 0, s, q, kc, g, mid0,
                 n_mid, kpw, tau2, s_out, smax_part, ssum_part, hist0, nhist);
}

hipError_t launch_esa_decode_scan(const void* q, bool q_bf16, const bf16* kc, const ScGeom& g, int64_t nsel,
                                  int64_t mid0, int64_t n_mid, int64_t dc, float tau2, float* s_out,
                                  float* smax_part, float* ssum_part, int32_t* hist0, int64_t nhist,
                                  hipStream_t s) {
  if (n_mid <= 0) return hipSuccess;
  const int nw = esa_scan_wgs(n_mid);
  const int64_t kpw = cdiv(n_mid, nw);
  const dim3 grid((unsigned)nw, (unsigned)nsel);
  const float* qf = (const float*)q;
  const bf16* qb = (const bf16*)q;
  if (q_bf16) {
    if (dc == 64) launch_scan_dc<64>(qb, kc, g, grid, mid0, n_mid, kpw, tau2, s_out, smax_part, ssum_part, hist0, nhist, s);
    else launch_scan_dc<128>(qb, kc, g, grid, mid0, n_mid, kpw, tau2, s_out, smax_part, ssum_part, hist0, nhist, s);
  } else {
    switch (dc) {
      case 32: launch_scan_dc<32>(qf, kc, g, grid, mid0, n_mid, kpw, tau2, s_out, smax_part, ssum_part, hist0, nhist, s); break;
      case 64: launch_scan_dc<64>(qf, kc, g, grid, mid0, n_mid, kpw, tau2, s_out, smax_part, ssum_part, hist0, nhist, s); break;
      case 128: launch_scan_dc<128>(qf, kc, g, grid, mid0, n_mid, kpw, tau2, s_out, smax_part, ssum_part, hist0, nhist, s); break;
      default: launch_scan_dc<256>(qf, kc, g, grid, mid0, n_mid, kpw, tau2, s_out, smax_part, ssum_part, hist0, nhist, s); break;
    }
  }
  return hipGetLastError();
}

// workgroups per sequence at the finest split (the workspace holds that many per-slice counts)
int esa_topk_slices(int64_t n_mid) { return (int)std::max<int64_t>(1, cdiv(n_mid, kTkThreads * kTkPerMin)); }
int esa_topk_max_radius() { return kTkMaxRadius; }

template <int PER>
static hipError_t launch_esa_topk_per(int mode, const float* upart, int nqsplit, const float* s_in,
                                      const float* smax_part, const float* ssum_part, int nsmax, float clip,
                                      float tau2, int64_t batch, int64_t n_mid,
                                      int radius, int topk, int64_t mid0, int32_t* hist, int2* wgcnt,
                                      uint32_t* keys, float* scores_out, int32_t* sel, int32_t* n_sel,
                                      bool hist_clear, hipStream_t s) {
  const int64_t nwg = std::max<int64_t>(1, cdiv(n_mid, kTkThreads * PER));
  const dim3 grid((unsigned)nwg, (unsigned)batch);
  hipError_t e;
  if (n_mid > 0) {
    if (!hist_clear && (e = launch_fill_i32(hist, batch * 3 * kTkBins, 0, s)) != hipSuccess) return e;
    hipLaunchKernelGGL(esa_topk_prep_kernel<PER>, grid, dim3(kTkThreads), 0, s, mode, upart, nqsplit, s_in,
                       smax_part, ssum_part, nsmax, clip, tau2, n_mid, radius, keys, scores_out, hist);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (n_mid > topk) {
      for (int pass = 1; pass < 3; ++pass) {
        hipLaunchKernelGGL(esa_topk_hist_kernel<PER>, grid, dim3(kTkThreads), 0, s, pass, keys, n_mid, topk, hist);
        if ((e = hipGetLastError()) != hipSuccess) return e;
      }
      hipLaunchKernelGGL(esa_topk_count_kernel<PER>, grid, dim3(kTkThreads), 0, s, keys, n_mid, topk, hist, wgcnt);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  hipLaunchKernelGGL(esa_topk_emit_kernel<PER>, grid, dim3(kTkThreads), 0, s, keys, n_mid, topk, mid0, hist, wgcnt,
                     sel, n_sel);
  return hipGetLastError();
}

hipError_t launch_esa_topk(int mode, const float* upart, int nqsplit, const float* s_in, const float* smax_part,
                           const float* ssum_part, int nsmax, float clip, float tau2, int64_t batch, int64_t n_mid,
                           int radius, int topk, int64_t mid0,
                           int32_t* hist, int2* wgcnt, uint32_t* keys, float* scores_out, int32_t* sel,
                           int32_t* n_sel, bool hist_clear, hipStream_t s) {
  // the widest split that still gives every pass 256 workgroups (the
  // passes are latency-bound: fewer candidates per thread when there are
  // few sequences); wgcnt holds esa_topk_slices(n_mid) >= slices entries
  // per sequence
  const int64_t s8 = batch * cdiv(n_mid, kTkThreads * 8), s4 = batch * cdiv(n_mid, kTkThreads * 4);
  // many selections (one per head): 32 per thread halves the passes'
  // per-workgroup cost (reading the histograms, clearing the bins)
  if (batch * cdiv(n_mid, kTkThreads * 32) >= 1024)
    return launch_esa_topk_per<32>(mode, upart, nqsplit, s_in, smax_part, ssum_part, nsmax, clip, tau2, batch, n_mid, radius, topk,
                                   mid0, hist, wgcnt, keys, scores_out, sel, n_sel, hist_clear, s);
  if (batch * cdiv(n_mid, kTkThreads * 16) >= 256)
    return launch_esa_topk_per<16>(mode, upart, nqsplit, s_in, smax_part, ssum_part, nsmax, clip, tau2, batch, n_mid, radius, topk,
                                   mid0, hist, wgcnt, keys, scores_out, sel, n_sel, hist_clear, s);
  if (s8 >= 256)
    return launch_esa_topk_per<8>(mode, upart, nqsplit, s_in, smax_part, ssum_part, nsmax, clip, tau2, batch, n_mid, radius, topk,
                                  mid0, hist, wgcnt, keys, scores_out, sel, n_sel, hist_clear, s);
  if (s4 >= 256)
    return launch_esa_topk_per<4>(mode, upart, nqsplit, s_in, smax_part, ssum_part, nsmax, clip, tau2, batch, n_mid, radius, topk,
                                  mid0, hist, wgcnt, keys, scores_out, sel, n_sel, hist_clear, s);
  return launch_esa_topk_per<kTkPerMin>(mode, upart, nqsplit, s_in, smax_part, ssum_part, nsmax, clip, tau2, batch, n_mid, radius,
                                        topk, mid0, hist, wgcnt, keys, scores_out, sel, n_sel, hist_clear, s);
}

}  // namespace qat
