// MoBA block gating: block mean-pool of the keys, block affinity scores and
// top-(k-1) selection plus the forced current block.
//
// MoBA write-up (dtcms.com/wzjs/567377.html), section 3 "block partition and
// selection": blocks of B keys; affinity s_i = <q, mean_pool(K[I_i])>; top-k
// gate; causality (no future blocks); the query's own block is always
// attended. k counts that forced block, so k - 1 earlier blocks are chosen;
// the current block never competes.
#include "common.h"
#include "launch.h"

namespace qat {

// ---------------------------------------------------------------------------
// Mean pool, pass 1: each workgroup sums a slice of one block's tokens for all
// Hkv*d columns in float64 (HBM-bound stream of K, coalesced rows).
template <typename T>
__global__ __launch_bounds__(256) void meanpool_partial_kernel(
    const T* __restrict__ k, int64_t seq_len, int64_t cols, int block, int tokens_per_split,
    int nsplit, int64_t nbc, double* __restrict__ partial) {
  const int split = blockIdx.x;
  const int64_t b = blockIdx.y;
  const int64_t bi = blockIdx.z;
  const int64_t t0 = b * block + (int64_t)split * tokens_per_split;
  const int64_t t1 = min(b * block + (int64_t)block, t0 + tokens_per_split);
  const T* base = k + bi * seq_len * cols;
  double* dst = partial + ((bi * nbc + b) * nsplit + split) * cols;
  for (int64_t cg = threadIdx.x; cg < cols / 4; cg += blockDim.x) {
    double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
    for (int64_t t = t0; t < t1; ++t) {
      const T* p = base + t * cols + cg * 4;
      a0 += (double)to_f32(p[0]);
      a1 += (double)to_f32(p[1]);
      a2 += (double)to_f32(p[2]);
      a3 += (double)to_f32(p[3]);
    }
    dst[cg * 4 + 0] = a0;
    dst[cg * 4 + 1] = a1;
    dst[cg * 4 + 2] = a2;
    dst[cg * 4 + 3] = a3;
  }
}

// Mean pool, pass 2: sum the slices in order and divide by B.
__global__ void meanpool_finalize_kernel(const double* __restrict__ partial, int nsplit, int64_t nrows,
                                         int64_t cols, int block, float* __restrict__ kbar) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= nrows * cols) return;
  const int64_t r = idx / cols, c = idx % cols;
  double s = 0.0;
  for (int i = 0; i < nsplit; ++i) s += partial[(r * nsplit + i) * cols + c];
  kbar[idx] = (float)(s / (double)block);
}

// ---------------------------------------------------------------------------
// Scoring and selection: one thread per query row (t, h); a workgroup covers
// 256 consecutive positions of one query head, so all its threads read the
// same KV head's block means (staged in LDS, broadcast reads).
// The running top list holds KMAX entries ordered by (score desc, block
// asc); a candidate bubbles in with that order, so equal scores keep the
// smaller block first (blocks arrive in ascending order).
constexpr int kSelChunk = 64;   // block means staged per LDS round

template <typename T, int D, int KMAX>
__global__ __launch_bounds__(256) void moba_score_select_kernel(
    const T* __restrict__ q, const float* __restrict__ kbar, int32_t* __restrict__ blk,
    int64_t seq_len, int64_t hq, int64_t hkv, int64_t nbc, int64_t q_start, int64_t q_len, int block,
    int topk) {
  __shared__ float kb_s[kSelChunk * D];
  const int64_t bi = blockIdx.z;
  const int64_t h = blockIdx.y;
  const int64_t g = h / (hq / hkv);
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // row within [0, q_len)
  const bool valid = r < q_len;
  const int64_t t = q_start + (valid ? r : 0);
  const int64_t cur = t / block;
  const int km = topk - 1;

  float qf[D];
  {
    const T* qp = q + ((bi * seq_len + t) * hq + h) * D;
#pragma unroll
    for (int i = 0; i < D; ++i) qf[i] = to_f32(qp[i]);
  }
  float tv[KMAX];
  int ti[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) { tv[i] = -__builtin_inff(); ti[i] = 0x7fffffff; }

  // Candidate blocks of this workgroup: [0, max cur over its rows).
  const int64_t t_last = q_start + min(q_len, (int64_t)(blockIdx.x + 1) * blockDim.x) - 1;
  const int64_t nb_wg = km > 0 ? min(nbc, t_last / block) : 0;
  const float* kb_g = kbar + (bi * nbc) * hkv * D + g * D;   // block b at kb_g + b*hkv*D
  for (int64_t c0 = 0; c0 < nb_wg; c0 += kSelChunk) {
    const int64_t nc = min((int64_t)kSelChunk, nb_wg - c0);
    __syncthreads();
    for (int64_t i = threadIdx.x; i < nc * D; i += blockDim.x) {
      const int64_t bb = i / D, dd = i % D;
      kb_s[i] = kb_g[(c0 + bb) * hkv * D + dd];
    }
    __syncthreads();
    const int64_t nmine = valid ? min(nc, cur - c0) : 0;
    for (int64_t bb = 0; bb < nmine; ++bb) {
      const float* kr = kb_s + bb * D;
      float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
      for (int i = 0; i < D; i += 4) {
        a0 = fmaf(qf[i + 0], kr[i + 0], a0);
        a1 = fmaf(qf[i + 1], kr[i + 1], a1);
        a2 = fmaf(qf[i + 2], kr[i + 2], a2);
        a3 = fmaf(qf[i + 3], kr[i + 3], a3);
      }
      float cs = (a0 + a1) + (a2 + a3);
      int cb = (int)(c0 + bb);
#pragma unroll
      for (int i = 0; i < KMAX; ++i) {
        const bool better = (cs > tv[i]) || (cs == tv[i] && cb < ti[i]);
        const float sv = tv[i];
        const int sb = ti[i];
        tv[i] = better ? cs : sv;
        ti[i] = better ? cb : sb;
        cs = better ? sv : cs;
        cb = better ? sb : cb;
      }
    }
  }
  if (!valid) return;
  // Keep the first min(km, cur) picks, sort them ascending, append cur.
  const int npick = (int)min((int64_t)km, cur);
#pragma unroll
  for (int i = 0; i < KMAX; ++i)
    if (i >= npick) ti[i] = 0x7fffffff;
#pragma unroll
  for (int a = 0; a < KMAX; ++a)
#pragma unroll
    for (int b2 = 0; b2 + 1 < KMAX - a; ++b2) {
      const int lo = min(ti[b2], ti[b2 + 1]);
      const int hi = max(ti[b2], ti[b2 + 1]);
      ti[b2] = lo;
      ti[b2 + 1] = hi;
    }
  int32_t* out = blk + ((bi * q_len + r) * hq + h) * topk;
#pragma unroll
  for (int i = 0; i < KMAX; ++i)
    if (i < npick) out[i] = ti[i];
  out[npick] = (int32_t)cur;
  for (int i = npick + 1; i < topk; ++i) out[i] = -1;
}

// ---------------------------------------------------------------------------
int meanpool_splits(int block) { return (int)cdiv(block, 256); }

hipError_t launch_moba_meanpool(const void* k, bool bf, int64_t batch, int64_t seq_len, int64_t hkv,
                                int64_t d, int block, int64_t nbc, double* partial, float* kbar,
                                hipStream_t s) {
  if (nbc <= 0) return hipSuccess;
  const int nsplit = meanpool_splits(block);
  const int tps = (int)cdiv(block, nsplit);
  const int64_t cols = hkv * d;
  dim3 grid((unsigned)nsplit, (unsigned)nbc, (unsigned)batch);
  if (bf)
    hipLaunchKernelGGL(meanpool_partial_kernel<bf16>, grid, dim3(256), 0, s, (const bf16*)k, seq_len,
                       cols, block, tps, nsplit, nbc, partial);
  else
    hipLaunchKernelGGL(meanpool_partial_kernel<float>, grid, dim3(256), 0, s, (const float*)k, seq_len,
                       cols, block, tps, nsplit, nbc, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t total = batch * nbc * cols;
  hipLaunchKernelGGL(meanpool_finalize_kernel, dim3((unsigned)cdiv(total, 256)), dim3(256), 0, s,
                     partial, nsplit, batch * nbc, cols, block, kbar);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_select_d(const T* q, const float* kbar, int32_t* blk, int64_t batch,
                                  int64_t seq_len, int64_t hq, int64_t hkv, int64_t nbc, int64_t q_start,
                                  int64_t q_len, int block, int topk, hipStream_t s) {
  dim3 grid((unsigned)cdiv(q_len, 256), (unsigned)hq, (unsigned)batch);
  const int km = topk - 1;
#define QAT_SEL(KM_)                                                                                    \
  hipLaunchKernelGGL((moba_score_select_kernel<T, D, KM_>), grid, dim3(256), 0, s, q, kbar, blk, seq_len, \
                     hq, hkv, nbc, q_start, q_len, block, topk)
  if (km <= 1) QAT_SEL(1);
  else if (km <= 3) QAT_SEL(3);
  else if (km <= 7) QAT_SEL(7);
  else QAT_SEL(15);
#undef QAT_SEL
  return hipGetLastError();
}

hipError_t launch_moba_select(const void* q, bool bf, const float* kbar, int32_t* blk, int64_t batch,
                              int64_t seq_len, int64_t hq, int64_t hkv, int64_t d, int64_t nbc,
                              int64_t q_start, int64_t q_len, int block, int topk, hipStream_t s) {
  if (q_len <= 0) return hipSuccess;
  if (bf) {
    if (d == 64)
      return launch_select_d<bf16, 64>((const bf16*)q, kbar, blk, batch, seq_len, hq, hkv, nbc, q_start,
                                       q_len, block, topk, s);
    return launch_select_d<bf16, 128>((const bf16*)q, kbar, blk, batch, seq_len, hq, hkv, nbc, q_start,
                                      q_len, block, topk, s);
  }
  if (d == 64)
    return launch_select_d<float, 64>((const float*)q, kbar, blk, batch, seq_len, hq, hkv, nbc, q_start,
                                      q_len, block, topk, s);
  return launch_select_d<float, 128>((const float*)q, kbar, blk, batch, seq_len, hq, hkv, nbc, q_start,
                                     q_len, block, topk, s);
}

}  // namespace qat
