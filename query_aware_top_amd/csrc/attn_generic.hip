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

constexpr int kMobaDecPiece = 256;   // keys per decode piece
constexpr int kMobaDecKeys = 4;      // keys per 16-lane group and step in a piece

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
  // NK keys per group and step (all their loads issued before any use); a
  // group's missing key (past n) reads key 0 and enters with weight 0.
  template <int NK, typename Off>
  __device__ void keys_n(const T* __restrict__ K, const T* __restrict__ V, int64_t n, Off off) {
    for (int64_t j0 = 0; j0 < n; j0 += 4 * NK) {
      float kx[NK][E], vx[NK][E];
      bool ok[NK];
#pragma unroll
      for (int u = 0; u < NK; ++u) {
        const int64_t j = j0 + 4 * u + grp;
        ok[u] = j < n;
        const int64_t f = off(ok[u] ? j : 0);
        load_piece<T, E>(K + f + sub * E, kx[u]);
        load_piece<T, E>(V + f + sub * E, vx[u]);
      }
      float x[NK];
      float m_new = m;
#pragma unroll
      for (int u = 0; u < NK; ++u) {
        x[u] = ok[u] ? score(kx[u]) : -__builtin_inff();
        m_new = fmaxf(m_new, x[u]);
      }
      if (m_new == -__builtin_inff()) continue;   // this group has no key yet
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);   // 0 while m = -inf
      float ps = 0.f;
#pragma unroll
      for (int u = 0; u < NK; ++u) {
        x[u] = __builtin_amdgcn_exp2f(x[u] - m_new);
        ps += x[u];
      }
      l = fmaf(l, alpha, ps);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float acc = o[e] * alpha;
#pragma unroll
        for (int u = 0; u < NK; ++u) acc = fmaf(x[u], vx[u][e], acc);
        o[e] = acc;
      }
      m = m_new;
    }
  }
  template <typename Off>
  __device__ void keys(const T* __restrict__ K, const T* __restrict__ V, int64_t n, Off off) {
    keys_n<2>(K, V, n, off);
  }
  // As keys_n, software-pipelined: the loads of the next step's 4 NK keys
  // are in flight while the current step is scored and accumulated (two
  // register buffers of raw K and V pieces, used alternately).
  typedef T vec_t __attribute__((ext_vector_type(E)));
  template <int NK, typename Off>
  __device__ __forceinline__ void issue_step(vec_t (&kx)[NK], vec_t (&vx)[NK], const T* __restrict__ K,
                                             const T* __restrict__ V, int64_t j0, int64_t n, Off off) {
#pragma unroll
    for (int u = 0; u < NK; ++u) {
      const int64_t j = j0 + 4 * u + grp;
      const int64_t f = off(j < n ? j : 0) + sub * E;
      kx[u] = *reinterpret_cast<const vec_t*>(K + f);
      vx[u] = *reinterpret_cast<const vec_t*>(V + f);
    }
  }
  template <int NK>
  __device__ __forceinline__ void consume_step(const vec_t (&kx)[NK], const vec_t (&vx)[NK], int64_t j0,
                                               int64_t n) {
    float x[NK];
    float m_new = m;
#pragma unroll
    for (int u = 0; u < NK; ++u) {
      float kf[E];
#pragma unroll
      for (int e = 0; e < E; ++e) kf[e] = to_f32(kx[u][e]);
      x[u] = j0 + 4 * u + grp < n ? score(kf) : -__builtin_inff();
      m_new = fmaxf(m_new, x[u]);
    }
    if (m_new == -__builtin_inff()) return;   // this group has no key yet
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    float ps = 0.f;
#pragma unroll
    for (int u = 0; u < NK; ++u) {
      x[u] = __builtin_amdgcn_exp2f(x[u] - m_new);
      ps += x[u];
    }
    l = fmaf(l, alpha, ps);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float acc = o[e] * alpha;
#pragma unroll
      for (int u = 0; u < NK; ++u) acc = fmaf(x[u], to_f32(vx[u][e]), acc);
      o[e] = acc;
    }
    m = m_new;
  }
  template <int NK, typename Off>
  __device__ void keys_pipe(const T* __restrict__ K, const T* __restrict__ V, int64_t n, Off off) {
    constexpr int S = 4 * NK;
    if (n <= 0) return;
    vec_t ka[NK], va[NK], kb[NK], vb[NK];
    issue_step<NK>(ka, va, K, V, 0, n, off);
    for (int64_t j0 = 0;; j0 += 2 * S) {
      const bool more1 = j0 + S < n;
      if (more1) issue_step<NK>(kb, vb, K, V, j0 + S, n, off);
      consume_step<NK>(ka, va, j0, n);
      if (!more1) break;
      const bool more2 = j0 + 2 * S < n;
      if (more2) issue_step<NK>(ka, va, K, V, j0 + 2 * S, n, off);
      consume_step<NK>(kb, vb, j0 + S, n);
      if (!more2) break;
    }
  }
  template <typename O>
  __device__ void finish(O* dst, float* lse) {
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
      if (grp == 0) dst[sub * E + e] = from_f32<O>(ot * inv);
    }
    if (lse && (threadIdx.x & 63) == 0) *lse = lt > 0.f ? mg * 0.6931471805599453f + logf(lt) : -__builtin_inff();
  }
};

// MoBA: row = ((bi * q_len) + r) * hq + h, one wave each. q holds q_seq
// positions per sequence starting at position q_off (q_seq = seq_len,
// q_off = 0: the whole sequence; q_seq = q_len, q_off = q_start: only the
// processed rows).
template <typename T, int D>
__global__ __launch_bounds__(256) void moba_generic_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const int32_t* __restrict__ blk,
    T* __restrict__ out, float* __restrict__ lse, int64_t batch, int64_t seq_len, int64_t q_seq, int64_t q_off,
    int64_t hq, int64_t hkv, int64_t q_start, int64_t q_len, int block, int topk, int window, float scale_log2) {
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
  ra.init(q + ((bi * q_seq + t - q_off) * hq + h) * D, scale_log2);
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

// MoBA with few query rows (decode): the key set of a row is cut into pieces
// of up to kMobaDecPiece keys (each gated earlier block into ppb pieces, then
// the own block's causal part); one wave per (row, piece) leaves the piece's
// normalised o (float32) and lse, and moba_decode_combine_kernel merges a
// row's pieces by log-sum-exp. A piece past the row's keys leaves lse = -inf.
// q layout as in moba_generic_kernel.
template <typename T, int D>
__global__ __launch_bounds__(256) void moba_decode_piece_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const int32_t* __restrict__ blk,
    float* __restrict__ po, float* __restrict__ plse, int64_t rows, int64_t seq_len, int64_t q_seq, int64_t q_off,
    int64_t hq, int64_t hkv, int64_t q_start, int64_t q_len, int block, int topk, float scale_log2, int ppb,
    int npieces) {
  const int64_t row = (int64_t)blockIdx.y * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int piece = blockIdx.x;
  const int64_t h = row % hq;
  const int64_t r = (row / hq) % q_len;
  const int64_t bi = row / (hq * q_len);
  const int64_t g = h / (hq / hkv);
  const int64_t t = q_start + r;
  const int64_t cur = t / block;
  const int32_t* br = blk + row * topk;
  // the piece's key range [a, e): the s-th earlier block among the first
  // topk - 1 slots (slot order), or the own block from its start to t
  int64_t a = 0, e = 0;
  int s = piece / ppb;
  const int sub = piece % ppb;
  int nth = 0;
  bool found = false;
  for (int sl = 0; sl < topk - 1; ++sl) {
    const int32_t b = br[sl];
    if (b < 0 || b >= cur) continue;
    if (nth++ == s) {
      a = (int64_t)b * block + (int64_t)sub * kMobaDecPiece;
      e = min(a + kMobaDecPiece, (int64_t)(b + 1) * block);
      found = true;
      break;
    }
  }
  if (!found) {   // past the earlier blocks: pieces of the own block
    const int64_t own = piece - (int64_t)nth * ppb;
    a = cur * block + own * kMobaDecPiece;
    e = min(a + kMobaDecPiece, t + 1);
  }
  WaveRowAttn<T, D> ra;
  ra.init(q + ((bi * q_seq + t - q_off) * hq + h) * D, scale_log2);
  const int64_t base = (bi * seq_len * hkv + g) * D, stride = hkv * D;
  ra.template keys_pipe<kMobaDecKeys>(k, v, max((int64_t)0, e - a), [=](int64_t j) { return base + (a + j) * stride; });
  const int64_t pi = row * npieces + piece;
  ra.finish(po + pi * D, plse + pi);
}

// One thread per (row, d): log-sum-exp merge of the row's pieces.
template <typename T, int D>
__global__ void moba_decode_combine_kernel(const float* __restrict__ po, const float* __restrict__ plse,
                                           int npieces, int64_t rows, T* __restrict__ out,
                                           float* __restrict__ lse) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * D) return;
  const int64_t row = idx / D;
  const int d = (int)(idx % D);
  const float* lr = plse + row * npieces;
  float m = -__builtin_inff();
  for (int p = 0; p < npieces; ++p) m = fmaxf(m, lr[p]);
  float l = 0.f, o = 0.f;
  for (int p = 0; p < npieces; ++p) {
    const float w = lr[p] == -__builtin_inff() ? 0.f : expf(lr[p] - m);
    l += w;
    o = fmaf(w, po[(row * npieces + p) * D + d], o);
  }
  out[row * D + d] = from_f32<T>(l > 0.f ? o / l : 0.f);
  if (lse && d == 0) lse[row] = l > 0.f ? m + logf(l) : -__builtin_inff();
}

// ---------------------------------------------------------------------------
hipError_t launch_moba_generic(const void* q, const void* k, const void* v, const int32_t* blk, void* out,
                               float* lse, bool bf, int64_t batch, int64_t seq_len, int64_t q_seq, int64_t q_off,
                               int64_t hq, int64_t hkv, int64_t d, int64_t q_start, int64_t q_len, int block,
                               int topk, int window, float scale, hipStream_t s) {
  const int64_t rows = batch * q_len * hq;
  if (rows == 0) return hipSuccess;
  const float sl2 = scale * 1.4426950408889634f;
  dim3 grid((unsigned)cdiv(rows, 4));
#define QAT_MG(T_, D_)                                                                                     \
  launch_timed("moba_generic_attn", moba_generic_kernel<T_, D_>, grid, dim3(256), 0, s, (const T_*)q,        \
               (const T_*)k, (const T_*)v, blk, (T_*)out, lse, batch, seq_len, q_seq, q_off, hq, hkv, q_start,   \
               q_len, block, topk, window, sl2)
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

int moba_decode_pieces(int block, int topk) {
  const int ppb = (int)cdiv(block, kMobaDecPiece);
  return (topk - 1) * ppb + ppb;
}

hipError_t launch_moba_decode(const void* q, const void* k, const void* v, const int32_t* blk, float* po,
                              float* plse, void* out, float* lse, bool bf, int64_t batch, int64_t seq_len,
                              int64_t q_seq, int64_t q_off, int64_t hq, int64_t hkv, int64_t d, int64_t q_start,
                              int64_t q_len, int block, int topk, float scale, hipStream_t s) {
  const int64_t rows = batch * q_len * hq;
  if (rows == 0) return hipSuccess;
  const float sl2 = scale * 1.4426950408889634f;
  const int ppb = (int)cdiv(block, kMobaDecPiece);
  const int np = moba_decode_pieces(block, topk);
  dim3 grid((unsigned)np, (unsigned)cdiv(rows, 4));
  const unsigned g2 = (unsigned)cdiv(rows * d, 256);
#define QAT_MD(T_, D_)                                                                                          \
  do {                                                                                                          \
    {                                                                                                           \
      KTimer tm_("moba_decode_attn", s);                                                                        \
      launch_timed("moba_decode_attn", moba_decode_piece_kernel<T_, D_>, grid, dim3(256), 0, s, (const T_*)q,    \
                   (const T_*)k, (const T_*)v, blk, po, plse, rows, seq_len, q_seq, q_off, hq, hkv, q_start,      \
                   q_len, block, topk, sl2, ppb, np);                                                           \
    }                                                                                                           \
    hipError_t e_ = hipGetLastError();                                                                          \
    if (e_ != hipSuccess) return e_;                                                                            \
    KTimer tc_("moba_decode_combine", s);                                                                       \
    launch_timed("moba_decode_combine", moba_decode_combine_kernel<T_, D_>, dim3(g2), dim3(256), 0, s,          \
                 (const float*)po, (const float*)plse, np, rows, (T_*)out, lse);                                \
  } while (0)
  if (bf) {
    if (d == 64) QAT_MD(bf16, 64);
    else QAT_MD(bf16, 128);
  } else {
    if (d == 64) QAT_MD(float, 64);
    else QAT_MD(float, 128);
  }
#undef QAT_MD
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
