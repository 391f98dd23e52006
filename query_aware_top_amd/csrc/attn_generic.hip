// Per-row exact attention for the shapes the matrix-core kernels do not take
// (float32 inputs, MoBA's extra local window, head sizes without a tiled
// kernel). One thread owns one (query, head) row and walks its key set in
// ascending position with an online softmax in float32.
//
// Key sets: MoBA write-up (dtcms.com/wzjs/567377.html), sections 2-3 (gated
// earlier blocks whole, own block causal); ESA write-up
// (hlszyjy.com/post/6872.html), four-part split (initial, selected middle,
// local window, chunk causal).
#include "common.h"
#include "launch.h"

namespace qat {

template <typename T, int D>
struct RowAttn {
  float q[D], o[D];
  float m, l, sl2;
  __device__ void init(const T* qr, float scale_log2) {
#pragma unroll
    for (int i = 0; i < D; ++i) { q[i] = to_f32(qr[i]); o[i] = 0.f; }
    m = -__builtin_inff();
    l = 0.f;
    sl2 = scale_log2;
  }
  __device__ void key(const T* kr, const T* vr) {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int i = 0; i < D; i += 2) {
      s0 = fmaf(q[i], to_f32(kr[i]), s0);
      s1 = fmaf(q[i + 1], to_f32(kr[i + 1]), s1);
    }
    const float x = (s0 + s1) * sl2;
    const float m_new = fmaxf(m, x);
    const float alpha = exp2f(m - m_new);
    const float p = exp2f(x - m_new);
    l = l * alpha + p;
#pragma unroll
    for (int i = 0; i < D; ++i) o[i] = o[i] * alpha + p * to_f32(vr[i]);
    m = m_new;
  }
  __device__ void finish(T* dst, float* lse) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int i = 0; i < D; ++i) dst[i] = from_f32<T>(o[i] * inv);
    if (lse) *lse = l > 0.f ? m * 0.6931471805599453f + logf(l) : -__builtin_inff();
  }
};

// MoBA: row = ((bi * q_len) + r) * hq + h.
template <typename T, int D>
__global__ __launch_bounds__(128) void moba_generic_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const int32_t* __restrict__ blk,
    T* __restrict__ out, float* __restrict__ lse, int64_t batch, int64_t seq_len, int64_t hq, int64_t hkv,
    int64_t q_start, int64_t q_len, int block, int topk, int window, float scale_log2) {
  const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= batch * q_len * hq) return;
  const int64_t h = row % hq;
  const int64_t r = (row / hq) % q_len;
  const int64_t bi = row / (hq * q_len);
  const int64_t g = h / (hq / hkv);
  const int64_t t = q_start + r;
  const int64_t cur = t / block;
  const int32_t* br = blk + row * topk;
  RowAttn<T, D> ra;
  ra.init(q + ((bi * seq_len + t) * hq + h) * D, scale_log2);
  auto kv = [&](int64_t pos) {
    const int64_t off = ((bi * seq_len + pos) * hkv + g) * D;
    ra.key(k + off, v + off);
  };
  // earlier blocks sit in the first topk - 1 slots (the last one is taken by
  // the current block)
  auto gated = [&](int64_t b) {
    for (int s = 0; s < topk - 1; ++s)
      if (br[s] == b) return true;
    return false;
  };
  // gated earlier blocks whole; window keys before the own block whose
  // block is not gated; the own block causally. Each key once.
  for (int s = 0; s < topk - 1; ++s) {
    const int32_t b = br[s];
    if (b < 0 || b >= cur) continue;
    for (int64_t p = (int64_t)b * block; p < (int64_t)(b + 1) * block; ++p) kv(p);
  }
  if (window > 0)
    for (int64_t p = max((int64_t)0, t - window + 1); p < cur * block; ++p)
      if (!gated(p / block)) kv(p);
  for (int64_t p = cur * block; p <= t; ++p) kv(p);
  ra.finish(out + row * D, lse ? lse + row : nullptr);
}

// ESA: row = ((bi * m) + i) * H + h.
template <typename T, int D>
__global__ __launch_bounds__(128) void esa_generic_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ n_sel, T* __restrict__ out, float* __restrict__ lse, int64_t batch, int64_t H,
    int64_t ctx_len, int64_t c0, int64_t m, int64_t n_init, int64_t window, int topk, float scale_log2) {
  const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= batch * m * H) return;
  const int64_t h = row % H;
  const int64_t i = (row / H) % m;
  const int64_t bi = row / (H * m);
  RowAttn<T, D> ra;
  ra.init(q + row * D, scale_log2);
  auto kv = [&](int64_t pos) {
    const int64_t off = ((bi * ctx_len + pos) * H + h) * D;
    ra.key(k + off, v + off);
  };
  const int64_t ni = min(n_init, c0);
  for (int64_t p = 0; p < ni; ++p) kv(p);
  const int32_t ns = n_sel[bi];
  for (int s = 0; s < ns; ++s) kv(sel[bi * topk + s]);
  if (c0 > n_init)
    for (int64_t p = max(n_init, c0 - window); p < c0; ++p) kv(p);
  for (int64_t p = c0; p <= c0 + i; ++p) kv(p);
  ra.finish(out + row * D, lse ? lse + row : nullptr);
}

// ---------------------------------------------------------------------------
hipError_t launch_moba_generic(const void* q, const void* k, const void* v, const int32_t* blk, void* out,
                               float* lse, bool bf, int64_t batch, int64_t seq_len, int64_t hq, int64_t hkv,
                               int64_t d, int64_t q_start, int64_t q_len, int block, int topk, int window,
                               float scale, hipStream_t s) {
  const int64_t rows = batch * q_len * hq;
  if (rows == 0) return hipSuccess;
  const float sl2 = scale * 1.4426950408889634f;
  dim3 grid((unsigned)cdiv(rows, 128));
#define QAT_MG(T_, D_)                                                                                       \
  hipLaunchKernelGGL((moba_generic_kernel<T_, D_>), grid, dim3(128), 0, s, (const T_*)q, (const T_*)k,       \
                     (const T_*)v, blk, (T_*)out, lse, batch, seq_len, hq, hkv, q_start, q_len, block, topk, \
                     window, sl2)
  if (bf) {
    if (d == 64) QAT_MG(bf16, 64);
    else QAT_MG(bf16, 128);
  } else {
    if (d == 64) QAT_MG(float, 64);
    else QAT_MG(float, 128);
  }
#undef QAT_MG
  return hipGetLastError();
}

hipError_t launch_esa_generic(const void* q, const void* k, const void* v, const int32_t* sel, const int32_t* n_sel,
                              void* out, float* lse, bool bf, int64_t batch, int64_t H, int64_t d, int64_t ctx_len,
                              int64_t c0, int64_t m, int64_t n_init, int64_t window, int topk, float scale,
                              hipStream_t s) {
  const int64_t rows = batch * m * H;
  if (rows == 0) return hipSuccess;
  const float sl2 = scale * 1.4426950408889634f;
  dim3 grid((unsigned)cdiv(rows, 128));
#define QAT_EG(T_, D_)                                                                                          \
  hipLaunchKernelGGL((esa_generic_kernel<T_, D_>), grid, dim3(128), 0, s, (const T_*)q, (const T_*)k,           \
                     (const T_*)v, sel, n_sel, (T_*)out, lse, batch, H, ctx_len, c0, m, n_init, window, topk, sl2)
  if (bf) {
    if (d == 64) QAT_EG(bf16, 64);
    else QAT_EG(bf16, 128);
  } else {
    if (d == 64) QAT_EG(float, 64);
    else QAT_EG(float, 128);
  }
#undef QAT_EG
  return hipGetLastError();
}

}  // namespace qat
