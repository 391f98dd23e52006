// CCA-style core-token attention (CCA-Attention write-up: global-aware
// pooling, locality-preserving module, global-local fusion; the page drops
// the formulas, the library reads them as follows):
//   groups     non-overlapping groups of g tokens, group i = [i g, (i+1) g);
//   core token the group's last query scores the group's keys,
//              a_j = softmax_j(scale <q_last, k_j>), and the core key / value
//              are the a-weighted sums of the group's keys / values (the two
//              modules share their linear maps, so pooling then projecting
//              is pooling the projected keys and values);
//   window     query t sees the raw tokens [ls(t), t], ls(t) = max(0,
//              floor(t/g) g - ceil(w/g) g): group-aligned, >= w tokens;
//   global     the core tokens of the groups before ls(t);
//   fusion     one softmax over core tokens + window.
//
// Two kernels: cca_pool_kernel (one wave per (sequence, group, query head),
// an online softmax over the group's keys accumulating both the key and
// the value sums; a memory-bound pass over K and V), and cca_attn_kernel
// (the matrix-core tile engine over two segments, the core tokens then the
// window, in one online softmax).
#include <algorithm>

#include "attn_core.h"
#include "common.h"
#include "launch.h"

namespace qat {

constexpr int kCcaNW = 8;
constexpr int kCcaThreads = 64 * kCcaNW;
constexpr int kCcaRows = 32 * kCcaNW;

__host__ __device__ __forceinline__ int64_t cca_window_start(int64_t t, int64_t g, int64_t wg) {
  const int64_t s = (t / g) * g - wg;
  return s > 0 ? s : 0;
}

// ---------------------------------------------------------------------------
// Pooling: wave per (bi, i, h) with row = (bi * ngroups + i) * hq + h; lanes
// as the per-row attention kernels (four groups of 16 lanes, every fourth
// key, E = D / 16 dims per lane).
template <int D>
__global__ __launch_bounds__(256) void cca_pool_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                       const bf16* __restrict__ v, bf16* __restrict__ kc,
                                                       bf16* __restrict__ vc, int64_t rows, int64_t seq_len,
                                                       int64_t hq, int64_t hkv, int64_t ngroups, int group,
                                                       float scale_log2) {
  constexpr int E = D / 16;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63, grp = lane >> 4, sub = lane & 15;
  const int64_t h = row % hq;
  const int64_t i = (row / hq) % ngroups;
  const int64_t bi = row / (hq * ngroups);
  const int64_t g = h / (hq / hkv);
  float qf[E], ak[E], av[E];
  const bf16* qp = q + ((bi * seq_len + (i + 1) * group - 1) * hq + h) * D + sub * E;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    qf[e] = (float)qp[e];
    ak[e] = 0.f;
    av[e] = 0.f;
  }
  float m = -__builtin_inff(), l = 0.f;
  const int64_t base = ((bi * seq_len + i * group) * hkv + g) * D + sub * E, stride = hkv * D;
  for (int j = grp; j < group; j += 4) {
    float kx[E], vx[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      kx[e] = (float)k[base + j * stride + e];
      vx[e] = (float)v[base + j * stride + e];
    }
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) s = fmaf(qf[e], kx[e], s);
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
    s *= scale_log2;
    const float m_new = fmaxf(m, s);
    const float a = __builtin_amdgcn_exp2f(m - m_new), p = __builtin_amdgcn_exp2f(s - m_new);
    l = fmaf(l, a, p);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      ak[e] = fmaf(ak[e], a, p * kx[e]);
      av[e] = fmaf(av[e], a, p * vx[e]);
    }
    m = m_new;
  }
  // merge the four groups (a group with no key has m = -inf, l = 0)
  float mg = fmaxf(m, __shfl_xor(m, 16, 64));
  mg = fmaxf(mg, __shfl_xor(mg, 32, 64));
  const float w = m == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m - mg);
  float lt = l * w;
  lt += __shfl_xor(lt, 16, 64);
  lt += __shfl_xor(lt, 32, 64);
  const float inv = 1.f / lt;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    float x = ak[e] * w, y = av[e] * w;
    x += __shfl_xor(x, 16, 64);
    x += __shfl_xor(x, 32, 64);
    y += __shfl_xor(y, 16, 64);
    y += __shfl_xor(y, 32, 64);
    if (grp == 0) {
      kc[row * D + sub * E + e] = (bf16)(x * inv);
      vc[row * D + sub * E + e] = (bf16)(y * inv);
    }
  }
}

// ---------------------------------------------------------------------------
// Attention: grid (256-row tiles of the processed positions, query head,
// sequence); segment 1 the core tokens [0, nc(t)), segment 2 the raw window
// [ls(t), t]; one online softmax over both.
template <int D>
__global__ __launch_bounds__(kCcaThreads, 1) void cca_attn_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ kc, const bf16* __restrict__ vc, bf16* __restrict__ out, float* __restrict__ lse_out,
    int64_t seq_len, int64_t hq, int64_t hkv, int64_t q_start, int64_t q_len, int64_t ngroups, int group,
    int window, float scale_log2) {
  QAT_FA_SMEM(D, sm);
  int64_t id = xcd_logical_id(blockIdx.x, gridDim.x);
  const int64_t ntile = cdiv(q_len, kCcaRows);
  // later row tiles attend more core tokens: they are dispatched first, so
  // the launch ends on short tiles
  const int64_t rt = ntile - 1 - id % ntile;
  id /= ntile;
  const int64_t h = id % hq, bi = id / hq;
  const int64_t g = h / (hq / hkv);
  const int64_t t0 = q_start + rt * kCcaRows;
  const int64_t t1 = min(q_start + q_len, t0 + kCcaRows) - 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = t0 + wave * 32 + (lane & 31);
  const bool valid = t <= t1;
  const int64_t tv = valid ? t : t0;
  FaState<D> st;
  fa_init<D>(st, q + ((bi * seq_len + tv) * hq + h) * D, valid);
  const int64_t gg = group;
  const int64_t wg = cdiv(window, gg) * gg;
  const int64_t ls = cca_window_start(tv, gg, wg);
  // wave-uniform bounds: the wave's first and last valid rows
  const int64_t tw0 = t0 + wave * 32, tw1 = min(t1, tw0 + 31);
  // core tokens: this lane sees c < nc(t); every lane of the wave sees c < nc(tw0)
  const int nc_lane = valid ? (int)(ls / gg) : 0;
  const int nc_wave = tw0 <= t1 ? (int)(cca_window_start(tw0, gg, wg) / gg) : 0;
  const int nc_max = (int)(cca_window_start(t1, gg, wg) / gg);
  const int hd = (int)(hq * D);
  fa_segment<D, kCcaNW, true, false>(st, sm, kc + (bi * ngroups * hq + h) * D, vc + (bi * ngroups * hq + h) * D, nc_max,
                              scale_log2, [=](int c) { return c * hd; }, [=](int c) { return c < nc_lane; },
                              [=](int c0) { return c0 + kKT <= nc_wave; });
  // raw window: keys [lmin, t1] of the tile; this lane sees [ls(t), t]
  const int64_t lmin = cca_window_start(t0, gg, wg);
  const int n_raw = (int)(t1 - lmin + 1);
  const int lo = valid ? (int)(ls - lmin) : 1, hi = valid ? (int)(t - lmin) : 0;
  const int lo_w = tw0 <= t1 ? (int)(cca_window_start(tw1, gg, wg) - lmin) : 1 << 30;
  const int hi_w = (int)(tw0 - lmin);
  const int kvs = (int)(hkv * D);
  const int64_t rbase = ((bi * seq_len + lmin) * hkv + g) * D;
  fa_segment<D, kCcaNW, true, false>(st, sm, k + rbase, v + rbase, n_raw, scale_log2, [=](int j) { return j * kvs; },
                              [=](int j) { return j >= lo && j <= hi; },
                              [=](int j0) { return j0 >= lo_w && j0 + kKT - 1 <= hi_w; });
  float inv_l, lse;
  fa_finish<D>(st, inv_l, lse);
  const int64_t orow0 = (bi * q_len + (t0 - q_start)) * hq + h;   // row of position t0
  if (lse_out && valid && (lane >> 5) == 0) lse_out[orow0 + (t - t0) * hq] = lse;
  constexpr int TPR = D / 8;
  constexpr int RPP = kCcaThreads / TPR;
  const int sub = threadIdx.x % TPR;
  const int nrows = (int)(t1 - t0 + 1);
  for (int half = 0; half < kCcaNW / 4; ++half) {
    fa_rows_to_lds<D>(st, sm, inv_l, half);
    __syncthreads();
    for (int rr = threadIdx.x / TPR; rr < 128; rr += RPP) {
      const int tr = half * 128 + rr;
      if (tr >= nrows) continue;
      const f32x4 a = fa_row_chunk<D>(sm, rr, 2 * sub), cc = fa_row_chunk<D>(sm, rr, 2 * sub + 1);
      u32x4 w;
      w[0] = pack_bf16x2(a[0], a[1]);
      w[1] = pack_bf16x2(a[2], a[3]);
      w[2] = pack_bf16x2(cc[0], cc[1]);
      w[3] = pack_bf16x2(cc[2], cc[3]);
      *(u32x4*)(out + (orow0 + (int64_t)tr * hq) * D + sub * 8) = w;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
int64_t cca_groups_needed(int64_t seq_len, int64_t q_start, int64_t q_len, int group, int window) {
  const int64_t wg = cdiv(window, group) * group;
  const int64_t need = cca_window_start(q_start + q_len - 1, group, wg) / group;
  return std::min<int64_t>(need, seq_len / group);
}

hipError_t launch_cca_pool(const void* q, const void* k, const void* v, void* kc, void* vc, int64_t batch,
                           int64_t seq_len, int64_t hq, int64_t hkv, int64_t d, int64_t ngroups, int64_t npool,
                           int group, float scale, hipStream_t s) {
  // pools groups [0, npool) of each sequence into kc, vc laid out with ngroups groups per sequence
  if (npool <= 0) return hipSuccess;
  const float sl2 = scale * kLog2e;
  for (int64_t bi = 0; bi < batch; ++bi) {
    const int64_t rows = npool * hq;
    const size_t qo = (size_t)bi * seq_len * hq * d, ko = (size_t)bi * seq_len * hkv * d;
    const size_t co = (size_t)bi * ngroups * hq * d;
    dim3 grid((unsigned)cdiv(rows, 4));
    if (d == 64)
      launch_timed("cca_pool", cca_pool_kernel<64>, grid, dim3(256), 0, s, (const bf16*)q + qo,
                   (const bf16*)k + ko, (const bf16*)v + ko, (bf16*)kc + co, (bf16*)vc + co, rows, seq_len, hq, hkv,
                   npool, group, sl2);
    else
      launch_timed("cca_pool", cca_pool_kernel<128>, grid, dim3(256), 0, s, (const bf16*)q + qo,
                   (const bf16*)k + ko, (const bf16*)v + ko, (bf16*)kc + co, (bf16*)vc + co, rows, seq_len, hq, hkv,
                   npool, group, sl2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_cca_attn(const void* q, const void* k, const void* v, const void* kc, const void* vc, void* out,
                           float* lse, int64_t batch, int64_t seq_len, int64_t hq, int64_t hkv, int64_t d,
                           int64_t q_start, int64_t q_len, int64_t ngroups, int group, int window, float scale,
                           hipStream_t s) {
  dim3 grid((unsigned)(cdiv(q_len, kCcaRows) * hq * batch));
  const float sl2 = scale * kLog2e;
  if (d == 64)
    launch_timed("cca_attn", cca_attn_kernel<64>, grid, dim3(kCcaThreads), 0, s, (const bf16*)q, (const bf16*)k,
                 (const bf16*)v, (const bf16*)kc, (const bf16*)vc, (bf16*)out, lse, seq_len, hq, hkv, q_start,
                 q_len, ngroups, group, window, sl2);
  else
    launch_timed("cca_attn", cca_attn_kernel<128>, grid, dim3(kCcaThreads), 0, s, (const bf16*)q, (const bf16*)k,
                 (const bf16*)v, (const bf16*)kc, (const bf16*)vc, (bf16*)out, lse, seq_len, hq, hkv, q_start,
                 q_len, ngroups, group, window, sl2);
  return hipGetLastError();
}

}  // namespace qat
