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
// and the importance as u_j = sum_i s^_ij.
//
// Prefill scoring runs on the bf16 matrix cores with q~ (float32) split into
// two bf16 terms (hi + lo): the products with the bf16 compressed keys are
// exact and the float32 sums carry ~2^-17 relative error, far inside the
// selection tolerance. Decode scoring is a float32 matrix-vector stream
// (HBM-bound). Top-k is an exact radix select on order-preserving uint32
// keys with the lowest index winning ties.
#include "common.h"
#include "launch.h"

namespace qat {

// ---------------------------------------------------------------------------
// Prefill pass 1: partial row maxima. grid (query tiles of 128, key splits,
// batch); a wave owns 32 queries and computes S^T = K~ Q~^T so each lane
// holds one query and 16 key scores per 32-key subtile.
template <int DC>
__global__ __launch_bounds__(256) void esa_rowmax_kernel(
    const bf16* __restrict__ q_hi, const bf16* __restrict__ q_lo, const bf16* __restrict__ kc,
    int64_t m, int64_t ctx_len, int64_t mid0, int64_t n_mid, int64_t keys_per_split, int nsplit,
    float* __restrict__ rowmax_part) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, r32 = lane & 31;
  const int64_t bi = blockIdx.z;
  const int64_t qi = (int64_t)blockIdx.x * 128 + wave * 32 + r32;
  const bool qvalid = qi < m;
  const int64_t qrow = bi * m + (qvalid ? qi : 0);
  bf16x8 qh[DC / 16], ql[DC / 16];
#pragma unroll
  for (int c = 0; c < DC / 16; ++c) {
    qh[c] = *(const bf16x8*)(q_hi + qrow * DC + 16 * c + 8 * h);
    ql[c] = *(const bf16x8*)(q_lo + qrow * DC + 16 * c + 8 * h);
  }
  const int64_t k0 = (int64_t)blockIdx.y * keys_per_split;
  const int64_t k1 = min(n_mid, k0 + keys_per_split);
  const bf16* kbase = kc + (bi * ctx_len + mid0) * DC;
  float mx = -__builtin_inff();
  for (int64_t kb = k0; kb < k1; kb += 32) {
    const int64_t key = kb + r32;
    const bf16* kr = kbase + (key < k1 ? key : k0) * DC;
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
    for (int c = 0; c < DC / 16; ++c) {
      const bf16x8 a = *(const bf16x8*)(kr + 16 * c + 8 * h);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qh[c], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, ql[c], acc, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t kk = kb + (i >> 2) * 8 + h * 4 + (i & 3);
      if (kk < k1) mx = fmaxf(mx, acc[i]);
    }
  }
  mx = fmaxf(mx, shfl_xor_f(mx, 32));
  if (qvalid && h == 0) rowmax_part[(bi * m + qi) * nsplit + blockIdx.y] = mx;
}

__global__ void esa_rowmax_final_kernel(const float* __restrict__ part, int nsplit, int64_t rows,
                                        float* __restrict__ rowmax) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows) return;
  float mx = -__builtin_inff();
  for (int s = 0; s < nsplit; ++s) mx = fmaxf(mx, part[i * nsplit + s]);
  rowmax[i] = mx;
}

// Prefill pass 2: partial importance. grid (key tiles of 128, query splits,
// batch); a wave owns 32 keys and computes S = Q~ K~^T so each lane holds one
// key and 16 query rows per 32-query subtile; corrected scores are summed in
// float32 per subtile and in float64 across subtiles (fixed order).
template <int DC>
__global__ __launch_bounds__(256) void esa_colsum_kernel(
    const bf16* __restrict__ q_hi, const bf16* __restrict__ q_lo, const float* __restrict__ rowmax,
    const bf16* __restrict__ kc, int64_t m, int64_t ctx_len, int64_t mid0, int64_t n_mid,
    int64_t rows_per_split, int nqsplit, float clip, float* __restrict__ upart) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, r32 = lane & 31;
  const int64_t bi = blockIdx.z;
  const int64_t key = (int64_t)blockIdx.x * 128 + wave * 32 + r32;
  const bool kvalid = key < n_mid;
  const bf16* kr = kc + (bi * ctx_len + mid0 + (kvalid ? key : 0)) * DC;
  bf16x8 kf[DC / 16];
#pragma unroll
  for (int c = 0; c < DC / 16; ++c) kf[c] = *(const bf16x8*)(kr + 16 * c + 8 * h);
  const int64_t i0 = (int64_t)blockIdx.y * rows_per_split;
  const int64_t i1 = min(m, i0 + rows_per_split);
  const float* rm = rowmax + bi * m;
  double total = 0.0;
  for (int64_t ib = i0; ib < i1; ib += 32) {
    const int64_t qi = ib + r32;
    const int64_t qrow = bi * m + (qi < i1 ? qi : i0);
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
    for (int c = 0; c < DC / 16; ++c) {
      const bf16x8 ah = *(const bf16x8*)(q_hi + qrow * DC + 16 * c + 8 * h);
      const bf16x8 al = *(const bf16x8*)(q_lo + qrow * DC + 16 * c + 8 * h);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, kf[c], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, kf[c], acc, 0, 0, 0);
    }
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t qq = ib + (i >> 2) * 8 + h * 4 + (i & 3);
      if (qq < i1) part += fmaxf(acc[i] - rm[qq], -clip);
    }
    total += (double)part;
  }
  total += __shfl_xor(total, 32, 64);
  if (kvalid && h == 0) upart[(bi * nqsplit + blockIdx.y) * n_mid + key] = (float)total;
}

// ---------------------------------------------------------------------------
// Decode scoring: s_j = <q~, k~_j> (float32) for every middle token, plus the
// workgroup maxima. DC/8 lanes per key, 8 elements (16 B) per lane.
template <int DC>
__global__ __launch_bounds__(256) void esa_decode_scan_kernel(
    const float* __restrict__ qc, const bf16* __restrict__ kc, int64_t ctx_len, int64_t mid0, int64_t n_mid,
    int64_t keys_per_wg, float* __restrict__ s_out, float* __restrict__ smax_part) {
  constexpr int LPK = DC / 8;          // lanes per key
  constexpr int KPW = 256 / LPK;       // keys per workgroup pass
  __shared__ float wmax[4];
  const int64_t bi = blockIdx.y;
  const int tid = threadIdx.x;
  const int sub = tid % LPK;
  float qv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) qv[j] = qc[bi * DC + sub * 8 + j];
  const int64_t k0 = (int64_t)blockIdx.x * keys_per_wg;
  const int64_t k1 = min(n_mid, k0 + keys_per_wg);
  const bf16* kbase = kc + (bi * ctx_len + mid0) * DC;
  float mx = -__builtin_inff();
  for (int64_t kb = k0; kb < k1; kb += KPW) {
    const int64_t key = kb + tid / LPK;
    float acc = 0.f;
    if (key < k1) {
      const bf16x8 kv = *(const bf16x8*)(kbase + key * DC + sub * 8);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc = fmaf(qv[j], (float)kv[j], acc);
    }
#pragma unroll
    for (int off = 1; off < LPK; off <<= 1) acc += __shfl_xor(acc, off, 64);
    if (key < k1) {
      if (sub == 0) s_out[bi * n_mid + key] = acc;
      mx = fmaxf(mx, acc);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if ((tid & 63) == 0) wmax[tid >> 6] = mx;
  __syncthreads();
  if (tid == 0)
    smax_part[bi * gridDim.x + blockIdx.x] = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
}

// ---------------------------------------------------------------------------
// Top-k: one workgroup of 1024 threads per sequence.
// mode 0 (prefill): u_j = sum of the query-split partials (float64, in order).
// mode 1 (decode):  u_j = max(s_j - max_j' s_j', -clip).
// Then u'_j = max over |t - j| <= r; keys = order-preserving uint32 of u';
// radix select of the k-th largest key (11 + 11 + 10 bits), then a stable
// compaction in index order taking the lowest-index ties.
constexpr int kTopkThreads = 1024;

__device__ int32_t block_exclusive_scan(int32_t v, int32_t* s_tmp, int32_t* total) {
  const int tid = threadIdx.x;
  s_tmp[tid] = v;
  __syncthreads();
  for (int off = 1; off < kTopkThreads; off <<= 1) {
    const int32_t a = tid >= off ? s_tmp[tid - off] : 0;
    __syncthreads();
    s_tmp[tid] += a;
    __syncthreads();
  }
  const int32_t incl = s_tmp[tid];
  if (total) *total = s_tmp[kTopkThreads - 1];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(kTopkThreads) void esa_topk_kernel(
    int mode, const float* __restrict__ upart, int nqsplit, const float* __restrict__ s_in,
    const float* __restrict__ smax_part, int nsmax, float clip, int64_t n_mid, int radius, int topk,
    int64_t mid0, float* __restrict__ u_tmp, uint32_t* __restrict__ keys, float* __restrict__ scores_out,
    int32_t* __restrict__ sel, int32_t* __restrict__ n_sel) {
  __shared__ int32_t hist[2048];
  __shared__ int32_t s_tmp[kTopkThreads];
  __shared__ float s_red[kTopkThreads / 64];
  __shared__ uint32_t s_prefix, s_mask;
  __shared__ int32_t s_kk, s_total;
  const int tid = threadIdx.x;
  const int64_t bi = blockIdx.x;
  int32_t* osel = sel + bi * topk;
  const int64_t nsel = min((int64_t)topk, n_mid);
  if (tid == 0) n_sel[bi] = (int32_t)nsel;
  for (int64_t j = nsel + tid; j < topk; j += kTopkThreads) osel[j] = -1;
  if (n_mid == 0) return;

  // pass 0a: importance u
  float* u = u_tmp + bi * n_mid;
  if (mode == 0) {
    for (int64_t j = tid; j < n_mid; j += kTopkThreads) {
      double acc = 0.0;
      for (int s = 0; s < nqsplit; ++s) acc += (double)upart[(bi * nqsplit + s) * n_mid + j];
      u[j] = (float)acc;
    }
  } else {
    float mx = -__builtin_inff();
    for (int s = tid; s < nsmax; s += kTopkThreads) mx = fmaxf(mx, smax_part[bi * nsmax + s]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    if ((tid & 63) == 0) s_red[tid >> 6] = mx;
    __syncthreads();
    mx = s_red[0];
    for (int w = 1; w < kTopkThreads / 64; ++w) mx = fmaxf(mx, s_red[w]);
    for (int64_t j = tid; j < n_mid; j += kTopkThreads) u[j] = fmaxf(s_in[bi * n_mid + j] - mx, -clip);
  }
  __threadfence_block();
  __syncthreads();
  // pass 0b: neighbour max-pool, keys
  uint32_t* kk_arr = keys + bi * n_mid;
  for (int64_t j = tid; j < n_mid; j += kTopkThreads) {
    float v = u[j];
    const int64_t lo = max((int64_t)0, j - radius), hi = min(n_mid - 1, j + (int64_t)radius);
    for (int64_t t = lo; t <= hi; ++t) v = fmaxf(v, u[t]);
    kk_arr[j] = float_key(v);
    if (scores_out) scores_out[bi * n_mid + j] = v;
  }
  __threadfence_block();
  __syncthreads();

  if (n_mid <= topk) {   // everything is selected
    for (int64_t j = tid; j < n_mid; j += kTopkThreads) osel[j] = (int32_t)(mid0 + j);
    return;
  }
  // radix select of the topk-th largest key
  if (tid == 0) { s_prefix = 0; s_mask = 0; s_kk = topk; }
  __syncthreads();
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = shifts[pass], nbins = 1 << widths[pass];
    for (int i = tid; i < nbins; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
    const uint32_t prefix = s_prefix, mask = s_mask;
    for (int64_t j = tid; j < n_mid; j += kTopkThreads) {
      const uint32_t key = kk_arr[j];
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & (nbins - 1)], 1);
    }
    __syncthreads();
    // suffix sums over bins (descending order): thread t owns bins
    // nbins-1-2t and nbins-2-2t (two per thread for 2048 bins).
    const int per = nbins / kTopkThreads;   // 2 or 1
    int32_t local = 0;
    for (int p = 0; p < per; ++p) local += hist[nbins - 1 - (tid * per + p)];
    int32_t total;
    const int32_t before = block_exclusive_scan(local, s_tmp, &total);
    const int32_t need = s_kk;
    int32_t acc = before;
    for (int p = 0; p < per; ++p) {
      const int bin = nbins - 1 - (tid * per + p);
      const int32_t c = hist[bin];
      if (acc < need && acc + c >= need) {
        s_prefix = prefix | ((uint32_t)bin << shift);
        s_mask = mask | ((uint32_t)(nbins - 1) << shift);
        s_total = need - acc;   // still to take from this bin
      }
      acc += c;
    }
    __syncthreads();
    if (tid == 0) s_kk = s_total;
    __syncthreads();
  }
  const uint32_t T = s_prefix;
  const int32_t take_eq = s_kk;
  // stable compaction: each thread owns a contiguous index range
  const int64_t per = cdiv(n_mid, kTopkThreads);
  const int64_t j0 = min(n_mid, (int64_t)tid * per), j1 = min(n_mid, j0 + per);
  int32_t gt = 0, eq = 0;
  for (int64_t j = j0; j < j1; ++j) {
    const uint32_t key = kk_arr[j];
    gt += key > T;
    eq += key == T;
  }
  const int32_t eq_before = block_exclusive_scan(eq, s_tmp, nullptr);
  const int32_t my_eq = max(0, min(eq, take_eq - eq_before));
  const int32_t out_before = block_exclusive_scan(gt + my_eq, s_tmp, nullptr);
  int32_t pos = out_before, eq_used = 0;
  for (int64_t j = j0; j < j1; ++j) {
    const uint32_t key = kk_arr[j];
    bool take = key > T;
    if (key == T && eq_used < my_eq) { take = true; ++eq_used; }
    if (take) osel[pos++] = (int32_t)(mid0 + j);
  }
}

// ---------------------------------------------------------------------------
int esa_key_splits(int64_t n_mid, int64_t m) {
  const int64_t qt = cdiv(m, 128);
  int64_t ks = cdiv(1024, qt);
  const int64_t max_ks = cdiv(n_mid, 256);
  if (ks > max_ks) ks = max_ks;
  return (int)(ks < 1 ? 1 : ks);
}
int esa_query_splits(int64_t n_mid, int64_t m) {
  const int64_t kt = cdiv(n_mid, 128);
  int64_t qs = cdiv(1024, kt);
  const int64_t max_qs = cdiv(m, 256);
  if (qs > max_qs) qs = max_qs;
  return (int)(qs < 1 ? 1 : qs);
}
int esa_scan_wgs(int64_t n_mid) {
  const int64_t w = cdiv(n_mid, 2048);
  return (int)(w < 1 ? 1 : w);
}

hipError_t launch_esa_prefill_scores(const bf16* q_hi, const bf16* q_lo, const bf16* kc, int64_t batch, int64_t m,
                                     int64_t ctx_len, int64_t mid0, int64_t n_mid, int64_t d_c, float clip,
                                     float* rowmax_part, float* rowmax, float* upart, hipStream_t s) {
  if (n_mid <= 0) return hipSuccess;
  const int ks = esa_key_splits(n_mid, m);
  const int64_t kps = cdiv(cdiv(n_mid, ks), 32) * 32;
  const int ks_eff = (int)cdiv(n_mid, kps);
  dim3 g1((unsigned)cdiv(m, 128), (unsigned)ks_eff, (unsigned)batch);
#define QAT_RM(DC_)                                                                                  \
  hipLaunchKernelGGL(esa_rowmax_kernel<DC_>, g1, dim3(256), 0, s, q_hi, q_lo, kc, m, ctx_len, mid0, \
                     n_mid, kps, ks_eff, rowmax_part)
  switch (d_c) {
    case 32: QAT_RM(32); break;
    case 64: QAT_RM(64); break;
    case 96: QAT_RM(96); break;
    case 128: QAT_RM(128); break;
    case 160: QAT_RM(160); break;
    case 192: QAT_RM(192); break;
    case 224: QAT_RM(224); break;
    default: QAT_RM(256); break;
  }
#undef QAT_RM
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(esa_rowmax_final_kernel, dim3((unsigned)cdiv(batch * m, 256)), dim3(256), 0, s,
                     rowmax_part, ks_eff, batch * m, rowmax);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int qs = esa_query_splits(n_mid, m);
  const int64_t rps = cdiv(cdiv(m, qs), 32) * 32;
  const int qs_eff = (int)cdiv(m, rps);
  dim3 g2((unsigned)cdiv(n_mid, 128), (unsigned)qs_eff, (unsigned)batch);
#define QAT_CS(DC_)                                                                                       \
  hipLaunchKernelGGL(esa_colsum_kernel<DC_>, g2, dim3(256), 0, s, q_hi, q_lo, rowmax, kc, m, ctx_len, mid0, \
                     n_mid, rps, qs_eff, clip, upart)
  switch (d_c) {
    case 32: QAT_CS(32); break;
    case 64: QAT_CS(64); break;
    case 96: QAT_CS(96); break;
    case 128: QAT_CS(128); break;
    case 160: QAT_CS(160); break;
    case 192: QAT_CS(192); break;
    case 224: QAT_CS(224); break;
    default: QAT_CS(256); break;
  }
#undef QAT_CS
  return hipGetLastError();
}

int esa_prefill_qsplits_eff(int64_t n_mid, int64_t m) {
  const int qs = esa_query_splits(n_mid, m);
  const int64_t rps = cdiv(cdiv(m, qs), 32) * 32;
  return (int)cdiv(m, rps);
}

hipError_t launch_esa_decode_scan(const float* qc, const bf16* kc, int64_t batch, int64_t ctx_len, int64_t mid0,
                                  int64_t n_mid, int64_t d_c, float* s_out, float* smax_part, hipStream_t s) {
  if (n_mid <= 0) return hipSuccess;
  const int nw = esa_scan_wgs(n_mid);
  const int64_t kpw = cdiv(n_mid, nw);
  dim3 grid((unsigned)nw, (unsigned)batch);
#define QAT_DS(DC_)                                                                                       \
  hipLaunchKernelGGL(esa_decode_scan_kernel<DC_>, grid, dim3(256), 0, s, qc, kc, ctx_len, mid0, n_mid, kpw, \
                     s_out, smax_part)
  switch (d_c) {
    case 32: QAT_DS(32); break;
    case 64: QAT_DS(64); break;
    case 128: QAT_DS(128); break;
    default: QAT_DS(256); break;
  }
#undef QAT_DS
  return hipGetLastError();
}

hipError_t launch_esa_topk(int mode, const float* upart, int nqsplit, const float* s_in, const float* smax_part,
                           int nsmax, float clip, int64_t batch, int64_t n_mid, int radius, int topk, int64_t mid0,
                           float* u_tmp, uint32_t* keys, float* scores_out, int32_t* sel, int32_t* n_sel,
                           hipStream_t s) {
  hipLaunchKernelGGL(esa_topk_kernel, dim3((unsigned)batch), dim3(kTopkThreads), 0, s, mode, upart, nqsplit, s_in,
                     smax_part, nsmax, clip, n_mid, radius, topk, mid0, u_tmp, keys, scores_out, sel, n_sel);
  return hipGetLastError();
}

}  // namespace qat
