// Exact attention, one wave per (query, head) row, for the shapes the
// matrix-core kernels do not take (float32 inputs, MoBA's extra local window,
// head sizes without a tiled kernel). The 64 lanes form four groups of 16:
// group g takes keys g, g + 4, g + 8, ... of the row's key sequence (two per
// step), lane i of a group holds dims [i E, (i + 1) E) (E = D / 16) of q, of
// the key's K and V rows and of its accumulator, so each K/V row is read as
// 16 contiguous pieces. Every group runs its own online softmax in float32
// (exp2, scores scaled by scale log2 e); the four are merged at the end.
//
// Key sets: MoBA write-up (dtcms.com/wzjs/567377.html), sections 2-3 (gated
// earlier blocks whole, own block causal); ESA write-up
// (hlszyjy.com/post/6872.html), four-part split (initial, selected middle,
// local window, chunk causal).
#include "common.h"
#include "launch.h"

namespace qat {

template <typename T, int E>
__device__ __forceinline__ void load_piece(const T* p, float (&x)[E]) {
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = to_f32(p[e]);
}

template <typename T, int D>
struct WaveRowAttn {
  static constexpr int E = D / 16;
  float q[E], o[E];
  float m, l, sl2;
  int grp, sub;
  __device__ void init(const T* qr, float scale_log2) {
    const int lane = threadIdx.x & 63;
    grp = lane >> 4;
    sub = lane & 15;
    load_piece<T, E>(qr + sub * E, q);
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = 0.f;
    m = -__builtin_inff();
    l = 0.f;
    sl2 = scale_log2;
  }
  __device__ float score(const float (&kv)[E]) const {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) s = fmaf(q[e], kv[e], s);
    // sum over the 16 lanes of the group (xor offsets below 16 stay inside it)
    s += __shfl_xor(s, 8, 64);
    s += __shfl_xor(s, 4, 64);
    s += __shfl_xor(s, 2, 64);
    s += __shfl_xor(s, 1, 64);
    return s * sl2;
  }
  // The row's keys j = 0 .. n-1; off(j) is key j's element offset in K and V.
  // Two keys per group and step; a group's missing key (past n) reads key 0
  // and enters with weight 0.
  template <typename Off>
  __device__ void keys(const T* __restrict__ K, const T* __restrict__ V, int64_t n, Off off) {
    for (int64_t j0 = 0; j0 < n; j0 += 8) {
      const int64_t ja = j0 + grp, jb = j0 + 4 + grp;
      const bool oka = ja < n, okb = jb < n;
      const int64_t fa = off(oka ? ja : 0), fb = off(okb ? jb : 0);
      float ka[E], kb[E], va[E], vb[E];
      load_piece<T, E>(K + fa + sub * E, ka);
      load_piece<T, E>(K + fb + sub * E, kb);
      load_piece<T, E>(V + fa + sub * E, va);
      load_piece<T, E>(V + fb + sub * E, vb);
      const float xa = oka ? score(ka) : -__builtin_inff();
      const float xb = okb ? score(kb) : -__builtin_inff();
      const float m_new = fmaxf(m, fmaxf(xa, xb));
      if (m_new == -__builtin_inff()) continue;   // this group has no key yet
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);   // 0 while m = -inf
      const float pa = __builtin_amdgcn_exp2f(xa - m_new), pb = __builtin_amdgcn_exp2f(xb - m_new);
      l = fmaf(l, alpha, pa + pb);
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] = fmaf(o[e], alpha, fmaf(pa, va[e], pb * vb[e]));
      m = m_new;
    }
  }
  __device__ void finish(T* dst, float* lse) {
    float mg = fmaxf(m, __shfl_xor(m, 16, 64));
    mg = fmaxf(mg, __shfl_xor(mg, 32, 64));
    const float a = m == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m - mg);
    float lt = l * a;
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float ot = o[e] * a;
      ot += __shfl_xor(ot, 16, 64);
      ot += __shfl_xor(ot, 32, 64);
      if (grp == 0) dst[sub * E + e] = from_f32<T>(ot * inv);
    }
    if (lse && (threadIdx.x & 63) == 0) *lse = lt > 0.f ? mg * 0.6931471805599453f + logf(lt) : -__builtin_inff();
  }
};

// MoBA: row = ((bi * q_len) + r) * hq + h, one wave each.
template <typename T, int D>
__global__ __launch_bounds__(256) void moba_generic_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const int32_t* __restrict__ blk,
    T* __restrict__ out, float* __restrict__ lse, int64_t batch, int64_t seq_len, int64_t hq, int64_t hkv,
    int64_t q_start, int64_t q_len, int block, int topk, int window, float scale_log2) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= batch * q_len * hq) return;
  const int64_t h = row % hq;
  const int64_t r = (row / hq) % q_len;
  const int64_t bi = row / (hq * q_len);
  const int64_t g = h / (hq / hkv);
  const int64_t t = q_start + r;
  const int64_t cur = t / block;
  const int32_t* br = blk + row * topk;
  WaveRowAttn<T, D> ra;
  ra.init(q + ((bi * seq_len + t) * hq + h) * D, scale_log2);
  const int64_t base = (bi * seq_len * hkv + g) * D, stride = hkv * D;
  auto span = [&](int64_t a, int64_t b) {   // keys a .. b-1
    ra.keys(k, v, b - a, [=](int64_t j) { return base + (a + j) * stride; });
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
    span((int64_t)b * block, (int64_t)(b + 1) * block);
  }
  if (window > 0) {
    const int64_t lo = max((int64_t)0, t - window + 1), hi = cur * block;
    for (int64_t bb = lo / block; bb * block < hi; ++bb)
      if (!gated(bb)) span(max(lo, bb * block), min(hi, (bb + 1) * block));
  }
  span(cur * block, t + 1);
  ra.finish(out + row * D, lse ? lse + row : nullptr);
}

// ESA: row = ((bi * m) + i) * H + h, one wave each.
template <typename T, int D>
__global__ __launch_bounds__(256) void esa_generic_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ n_sel, T* __restrict__ out, float* __restrict__ lse, int64_t batch, int64_t H,
    int64_t ctx_len, int64_t c0, int64_t m, int64_t n_init, int64_t window, int topk, float scale_log2) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= batch * m * H) return;
  const int64_t h = row % H;
  const int64_t i = (row / H) % m;
  const int64_t bi = row / (H * m);
  WaveRowAttn<T, D> ra;
  ra.init(q + row * D, scale_log2);
  const int64_t base = (bi * ctx_len * H + h) * D, stride = H * D;
  auto span = [&](int64_t a, int64_t b) {
    ra.keys(k, v, b - a, [=](int64_t j) { return base + (a + j) * stride; });
  };
  span(0, min(n_init, c0));
  const int32_t* s_row = sel + bi * topk;
  ra.keys(k, v, n_sel[bi], [=](int64_t j) { return base + (int64_t)s_row[j] * stride; });
  if (c0 > n_init) span(max(n_init, c0 - window), c0);
  span(c0, c0 + i + 1);
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
  dim3 grid((unsigned)cdiv(rows, 4));
#define QAT_MG(T_, D_)                                                                                     \
  launch_timed("moba_generic_attn", moba_generic_kernel<T_, D_>, grid, dim3(256), 0, s, (const T_*)q,        \
               (const T_*)k, (const T_*)v, blk, (T_*)out, lse, batch, seq_len, hq, hkv, q_start, q_len, block, \
               topk, window, sl2)
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
  dim3 grid((unsigned)cdiv(rows, 4));
#define QAT_EG(T_, D_)                                                                                          \
  launch_timed("esa_generic_attn", esa_generic_kernel<T_, D_>, grid, dim3(256), 0, s, (const T_*)q, (const T_*)k,           \
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
