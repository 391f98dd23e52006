// ESA attention over the fused parts: initial + selected middle tokens
// ("global") and local window + the chunk itself ("window"), one joint
// softmax per head.
//
// ESA write-up (hlszyjy.com/post/6872.html), paragraph on the four-part
// token split: initial tokens and the selected top-k middle tokens form the
// global attention, local tokens the window attention, and the two are fused
// into the final output; decode uses the single current query. CCA write-up
// (m.jxzklqfsx.com/article/817694.html), global-local fusion section: both
// parts' keys and values form one unified K/V, i.e. one softmax.
//
// Key list of a sequence (ascending positions, all before the chunk):
//   j <  n_I                 -> j                      (initial)
//   j <  n_I + n_sel         -> sel[j - n_I]           (selected middle)
//   j <  n_I + n_sel + n_L   -> L0 + (j - n_I - n_sel) (local window)
// followed by the chunk's own keys [c0, t] under the causal mask.
// With per-head selection (ph) head h of sequence b reads selection
// v = b H + h (sel [B, H, topk], n_sel [B, H], one key list per (b, h)).
#include <algorithm>

#include "attn_core.h"
#include "common.h"
#include "launch.h"

namespace qat {

struct EsaKeys {
  const int32_t* sel;
  int64_t n_init, l0, n_l;
  int32_t n_sel;
  __device__ __forceinline__ int64_t count() const { return n_init + n_sel + n_l; }
  __device__ __forceinline__ int64_t pos(int64_t j) const {
    if (j < n_init) return j;
    if (j < n_init + n_sel) return sel[j - n_init];
    return l0 + (j - n_init - n_sel);
  }
};

__device__ __forceinline__ EsaKeys esa_keys(const int32_t* sel, const int32_t* n_sel, int64_t bi, int topk,
                                            int64_t c0, int64_t n_init, int64_t window) {
  EsaKeys kl;
  kl.sel = sel + bi * topk;
  kl.n_sel = n_sel[bi];
  kl.n_init = min(n_init, c0);
  if (c0 > n_init) {
    kl.l0 = max(n_init, c0 - window);
    kl.n_l = c0 - kl.l0;
  } else {
    kl.l0 = c0;
    kl.n_l = 0;
  }
  return kl;
}

// Key positions of one selection in attention order: the gathered keys
// (initial, selected, local) then the chunk [c0, c0 + m). grid (cdiv(len, 256),
// selections).
__global__ void esa_keylist_kernel(const int32_t* __restrict__ sel, const int32_t* __restrict__ n_sel,
                                   int32_t* __restrict__ keylist, int64_t stride, int topk, int64_t c0, int64_t m,
                                   int64_t n_init, int64_t window) {
  const int64_t bi = blockIdx.y;
  const EsaKeys kl = esa_keys(sel, n_sel, bi, topk, c0, n_init, window);
  const int64_t ng = kl.count();
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= ng + m) return;
  keylist[bi * stride + j] = (int32_t)(j < ng ? kl.pos(j) : c0 + (j - ng));
}

// ---------------------------------------------------------------------------
// Prefill / chunk attention on the matrix cores: grid (128-row tiles of the
// chunk, head, sequence).
constexpr int kNW = 8;   // waves per workgroup
constexpr int kThreads = 64 * kNW;
constexpr int kRows = 32 * kNW;

// The sequence's key list is staged in LDS when it fits (kEsaListLds
// entries): the K/V tile loads then take their row positions from LDS
// instead of a global read on the path to every tile's loads.
constexpr int kEsaListLds = 16384;

template <int D, bool LIST_LDS>
__global__ __launch_bounds__(kThreads, 8 / kNW) void esa_prefill_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ kc, const bf16* __restrict__ vc,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ n_sel, const int32_t* __restrict__ keylist,
    int64_t keylist_stride, bf16* __restrict__ out, float* __restrict__ lse_out, int64_t H, int64_t ctx_len,
    int64_t c0, int64_t m, int64_t n_init, int64_t window, int topk, float scale_log2, int ph) {
  QAT_FA_SMEM(D, sm);
  // logical id -> (row tile, head, sequence); the row tiles of one head are
  // adjacent and share an XCD (its L2 holds the head's gathered K/V)
  int64_t id = xcd_logical_id(blockIdx.x, gridDim.x);
  const int64_t ntile = cdiv(m, kRows);
  const int64_t qt = id % ntile;
  id /= ntile;
  const int64_t h = id % H, bi = id / H;
  const int64_t i0 = qt * kRows;
  const int64_t i_last = min(m, i0 + kRows) - 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t i = i0 + wave * 32 + (lane & 31);
  const bool valid = i <= i_last;
  const bf16* qrow = q + ((bi * m + (valid ? i : i0)) * H + h) * D;
  FaState<D> st;
  fa_init<D>(st, qrow, valid);
  const int64_t lv = ph ? bi * H + h : bi;   // the selection this head reads
  const EsaKeys kl = esa_keys(sel, n_sel, lv, topk, c0, n_init, window);
  const bf16* kb = kc + (bi * ctx_len * H + h) * D;
  const bf16* vb = vc + (bi * ctx_len * H + h) * D;
  // one key segment: the gathered keys (all before the chunk, never masked)
  // followed by the chunk's own keys under the causal mask; positions are
  // built here in LDS when they fit, else read from the key list built by
  // esa_keylist_kernel
  const int HD = (int)(H * D);
  const int ng = (int)kl.count();
  const int32_t* lst = keylist + lv * keylist_stride;
  const int lim = ng + (valid ? (int)i : -1);        // this lane attends keys j <= lim
  const int wlim = ng + (int)(i0 + wave * 32);       // every lane of the wave attends j <= wlim
  const int nkeys = ng + (int)(i_last + 1);
  extern __shared__ int32_t s_list[];
  if constexpr (LIST_LDS) {
    for (int j = threadIdx.x; j < nkeys; j += kThreads) s_list[j] = (int32_t)(j < ng ? kl.pos(j) : c0 + (j - ng));
    __syncthreads();
  }
  fa_segment<D, kNW, true>(st, sm, kb, vb, nkeys, scale_log2,
                           [=](int j) { return (LIST_LDS ? s_list[j] : lst[j]) * HD; },
                           [=](int j) { return j <= lim; }, [=](int j0) { return j0 + kKT - 1 <= wlim; });
  float inv_l, lse;
  fa_finish<D>(st, inv_l, lse);
  if (lse_out && valid && (lane >> 5) == 0) lse_out[(bi * m + i) * H + h] = lse;
  constexpr int TPR = D / 8;
  constexpr int RPP = kThreads / TPR;
  const int sub = threadIdx.x % TPR;
  const int nrows = (int)(i_last - i0 + 1);
  for (int half = 0; half < kNW / 4; ++half) {
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
      *(u32x4*)(out + ((bi * m + i0 + tr) * H + h) * D + sub * 8) = w;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Decode (one query per sequence): split-K over the key list. A workgroup of
// 256 threads covers the whole concatenated-head row (E = H*D/256 elements
// per thread, D/E lanes per head) and a contiguous slice of the key list;
// every gathered key row is one contiguous H*D*2-byte read. Partial
// (o, m, l) per (sequence, split, head) go to scratch; a second kernel merges
// them by log-sum-exp.
// keys per split: the fewest whole rounds of resident workgroups (two per CU
// at this kernel's register use) that give splits of 32..256 keys (one round
// of 512 workgroups at the 16-sequence 128k shape: 197 keys each, measured
// faster than two rounds of 98); 64 keys when no round count does
int esa_decode_keys_per_split(int64_t batch, int64_t nkeys_max) {
  constexpr int64_t kSlots = 2 * 256;
  for (int64_t rounds = 1; rounds <= 8; ++rounds) {
    const int64_t ns = std::max<int64_t>(1, rounds * kSlots / batch);
    const int64_t kps = cdiv(nkeys_max, ns);
    if (kps >= 32 && kps <= 256) return (int)kps;
  }
  return 64;
}
constexpr int kDecUnroll = 6;   // keys per batch (4: 1-2 us slower per decode step, 2: slower still)
constexpr int kDecMaxKps = 256;

// The split's key positions are staged in LDS first ([lists][kps], one list,
// or one per head under per-head selection), so the gathers of a batch issue
// back to back instead of each waiting on its own position load; the batches
// alternate between two register sets, the next one in flight while the
// current one is consumed.
template <int E, int D>
__global__ __launch_bounds__(256) void esa_decode_attn_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ kc, const bf16* __restrict__ vc,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ n_sel, float* __restrict__ po,
    float* __restrict__ pm, float* __restrict__ pl, int64_t H, int64_t ctx_len, int64_t c0,
    int64_t n_init, int64_t window, int topk, int nsplit, int kps, float scale_log2, int ph) {
  constexpr int kLph = D / E;   // lanes per head
  extern __shared__ int32_t lpos[];
  const int64_t bi = blockIdx.y;
  const int split = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t HD = H * D;
  const int64_t e0 = (int64_t)tid * E;   // element offset in the row
  const int head = tid / kLph;
  const int64_t j0 = (int64_t)split * kps;
  {
    // per-head selection: each head's lanes walk that head's list (all lists
    // have the same length, min(topk, |M|) selected)
    const int nl = ph ? (int)H : 1;
    for (int i = tid; i < nl * kps; i += 256) {
      const int hh = i / kps;
      const int64_t j = j0 + (i - hh * kps);
      const EsaKeys kh = esa_keys(sel, n_sel, ph ? bi * H + hh : bi, topk, c0, n_init, window);
      lpos[i] = (int32_t)(j < kh.count() ? kh.pos(j) : c0);   // the last key is the query's own position
    }
  }
  const EsaKeys kl = esa_keys(sel, n_sel, ph ? bi * H + head : bi, topk, c0, n_init, window);
  const int64_t nkeys = kl.count() + 1;   // + the query's own position c0
  const int nk = (int)max<int64_t>(0, min<int64_t>(kps, nkeys - j0));
  const int32_t* mypos = lpos + (ph ? head : 0) * kps;
  float qv[E], o[E];
  {
    const bf16* qr = q + bi * HD + e0;
#pragma unroll
    for (int e = 0; e < E; e += 8) {
      const bf16x8 t8 = *(const bf16x8*)(qr + e);
#pragma unroll
      for (int x = 0; x < 8; ++x) qv[e + x] = (float)t8[x];
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;
  float m = -__builtin_inff(), l = 0.f;
  const bf16* kb = kc + bi * ctx_len * HD + e0;
  const bf16* vb = vc + bi * ctx_len * HD + e0;
  __syncthreads();
  using Batch = bf16x8[kDecUnroll][E / 8];
  Batch ka, va, kn, vn;
  // keys past the split's end read the query's own row (always valid) and
  // are masked in the update
  auto load_batch = [&](int jb, Batch& kk, Batch& vv) {
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const int jj = min(jb + u, kps - 1);
      const int64_t p = jb + u < nk ? mypos[jj] : c0;
#pragma unroll
      for (int e = 0; e < E / 8; ++e) {
        kk[u][e] = *(const bf16x8*)(kb + p * HD + 8 * e);
        vv[u][e] = *(const bf16x8*)(vb + p * HD + 8 * e);
      }
    }
  };
  auto consume = [&](int jb, const Batch& kk, const Batch& vv) {
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < E / 8; ++e)
#pragma unroll
        for (int x = 0; x < 8; ++x) s = fmaf(qv[8 * e + x], (float)kk[u][e][x], s);
#pragma unroll
      for (int off = 1; off < kLph; off <<= 1) s += __shfl_xor(s, off, 64);
      const float x = jb + u < nk ? s * scale_log2 : -__builtin_inff();
      const float m_new = fmaxf(m, x);
      const float m_use = m_new == -__builtin_inff() ? 0.f : m_new;
      const float alpha = exp2f(m - m_use);
      const float p = exp2f(x - m_use);
      l = l * alpha + p;
#pragma unroll
      for (int e = 0; e < E / 8; ++e)
#pragma unroll
        for (int xx = 0; xx < 8; ++xx) o[8 * e + xx] = o[8 * e + xx] * alpha + p * (float)vv[u][e][xx];
      m = m_new;
    }
  };
  if (nk > 0) load_batch(0, ka, va);
  for (int jb = 0; jb < nk; jb += 2 * kDecUnroll) {
    if (jb + kDecUnroll < nk) load_batch(jb + kDecUnroll, kn, vn);
    consume(jb, ka, va);
    if (jb + kDecUnroll >= nk) break;
    if (jb + 2 * kDecUnroll < nk) load_batch(jb + 2 * kDecUnroll, ka, va);
    consume(jb + kDecUnroll, kn, vn);
  }
  const int64_t pidx = (bi * nsplit + split) * H + head;
  float* dst = po + pidx * D + (e0 % D);
#pragma unroll
  for (int e = 0; e < E; ++e) dst[e] = o[e];
  if ((e0 % D) == 0) {
    pm[pidx] = m;
    pl[pidx] = l;
  }
}

__global__ void esa_decode_combine_kernel(const float* __restrict__ po, const float* __restrict__ pm,
                                          const float* __restrict__ pl, const int32_t* __restrict__ n_sel,
                                          bf16* __restrict__ out, float* __restrict__ lse_out, int64_t H, int64_t D,
                                          int64_t c0, int64_t n_init, int64_t window, int nsplit_max, int kps,
                                          int ph) {
  const int64_t bi = blockIdx.y;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // element of the H*D row
  if (idx >= H * D) return;
  const int64_t head = idx / D;
  // number of splits actually holding keys for this sequence
  int64_t n_i = min(n_init, c0), n_l = 0;
  if (c0 > n_init) n_l = c0 - max(n_init, c0 - window);
  const int64_t nkeys = n_i + n_sel[ph ? bi * H : bi] + n_l + 1;
  const int ns = (int)min((int64_t)nsplit_max, cdiv(nkeys, kps));
  // online log-sum-exp merge over the splits, 8 splits' loads per round
  // (measured at 32 splits per sequence: rounds of 8 or 4 beat one round of
  // 32 or two of 16 by 2-5 us per decode step; rounds of 2 are slower)
  constexpr int U = 8;
  float M = -__builtin_inff(), L = 0.f, O = 0.f;
  for (int s0 = 0; s0 < ns; s0 += U) {
    float mv[U], lv[U], ov[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sp = min(s0 + u, ns - 1);
      const int64_t p = (bi * nsplit_max + sp) * H + head;
      mv[u] = pm[p];
      lv[u] = pl[p];
      ov[u] = po[p * D + (idx % D)];
      if (s0 + u >= ns) mv[u] = -__builtin_inff();
    }
    float Mn = M;
#pragma unroll
    for (int u = 0; u < U; ++u) Mn = fmaxf(Mn, mv[u]);
    const float a = M == -__builtin_inff() ? 0.f : exp2f(M - Mn);
    L *= a;
    O *= a;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float w = mv[u] == -__builtin_inff() ? 0.f : exp2f(mv[u] - Mn);
      L = fmaf(lv[u], w, L);
      O = fmaf(ov[u], w, O);
    }
    M = Mn;
  }
  out[bi * H * D + idx] = (bf16)(O / L);
  if (lse_out && (idx % D) == 0) lse_out[bi * H + head] = M * kLn2 + logf(L);
}

// ---------------------------------------------------------------------------
int esa_decode_splits(int64_t batch, int64_t n_init, int64_t topk, int64_t window) {
  const int64_t nk = n_init + topk + window + 1;
  return (int)cdiv(nk, esa_decode_keys_per_split(batch, nk));
}

int64_t esa_keylist_len(int64_t n_init, int64_t topk, int64_t window, int64_t m) {
  return n_init + topk + window + m;
}

hipError_t launch_esa_keylist(const int32_t* sel, const int32_t* n_sel, int32_t* keylist, int64_t nsel, int64_t c0,
                              int64_t m, int64_t n_init, int64_t window, int topk, hipStream_t s) {
  const int64_t kls = esa_keylist_len(n_init, topk, window, m);
  hipLaunchKernelGGL(esa_keylist_kernel, dim3((unsigned)cdiv(kls, 256), (unsigned)nsel), dim3(256), 0, s, sel,
                     n_sel, keylist, kls, topk, c0, m, n_init, window);
  return hipGetLastError();
}

hipError_t launch_esa_prefill_attn(const void* q, const void* k, const void* v, const int32_t* sel,
                                   const int32_t* n_sel, int32_t* keylist, void* out, float* lse, int64_t batch,
                                   int64_t H, int64_t D, int64_t ctx_len, int64_t c0, int64_t m, int64_t n_init,
                                   int64_t window, int topk, float scale, bool per_head, hipStream_t s) {
  const int64_t kls = esa_keylist_len(n_init, topk, window, m);
  const int64_t nsel = per_head ? batch * H : batch;
  const bool lds = kls <= kEsaListLds;
  if (!lds) {   // the attention kernel builds a list that fits in LDS itself
    hipLaunchKernelGGL(esa_keylist_kernel, dim3((unsigned)cdiv(kls, 256), (unsigned)nsel), dim3(256), 0, s, sel,
                       n_sel, keylist, kls, topk, c0, m, n_init, window);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  dim3 grid((unsigned)(cdiv(m, kRows) * H * batch));
  const float sl2 = scale * kLog2e;
  const size_t dyn = lds ? (size_t)kls * sizeof(int32_t) : 0;
#define QAT_ESA_PF(D_, L_)                                                                                  \
  launch_timed("esa_prefill_attn", esa_prefill_kernel<D_, L_>, grid, dim3(kThreads), (uint32_t)dyn, s,       \
               (const bf16*)q, (const bf16*)k, (const bf16*)v, sel, n_sel, (const int32_t*)keylist, kls,   \
               (bf16*)out, lse, H, ctx_len, c0, m, n_init, window, topk, sl2, per_head ? 1 : 0)
  if (D == 64) {
    if (lds) QAT_ESA_PF(64, true);
    else QAT_ESA_PF(64, false);
  } else {
    if (lds) QAT_ESA_PF(128, true);
    else QAT_ESA_PF(128, false);
  }
#undef QAT_ESA_PF
  return hipGetLastError();
}

bool esa_decode_supported(int64_t H, int64_t D, bool per_head) {
  const int64_t HD = H * D;
  if (HD % 256 || (D != 64 && D != 128)) return false;
  const int64_t E = HD / 256;
  // the staged positions, one list per head under per-head selection, fit in
  // 64 KiB of LDS
  if ((per_head ? H : 1) * kDecMaxKps * 4 > 65536) return false;
  return (E == 8 || E == 16 || E == 32) && D % E == 0;
}

hipError_t launch_esa_decode_attn(const void* q, const void* k, const void* v, const int32_t* sel,
                                  const int32_t* n_sel, float* po, float* pm, float* pl, void* out, float* lse,
                                  int64_t batch, int64_t H, int64_t D, int64_t ctx_len, int64_t c0, int64_t n_init,
                                  int64_t window, int topk, float scale, bool per_head, hipStream_t s) {
  const int nsplit = esa_decode_splits(batch, n_init, topk, window);
  const int kps = esa_decode_keys_per_split(batch, n_init + topk + window + 1);
  dim3 grid((unsigned)nsplit, (unsigned)batch);
  const float sl2 = scale * kLog2e;
  const int64_t E = H * D / 256;
  const uint32_t lds = (uint32_t)((per_head ? H : 1) * kps * sizeof(int32_t));
#define QAT_DEC(E_, D_)                                                                                     \
  launch_timed("esa_decode_attn", esa_decode_attn_kernel<E_, D_>, grid, dim3(256), lds, s, (const bf16*)q,  \
               (const bf16*)k, (const bf16*)v, sel, n_sel, po, pm, pl, H, ctx_len, c0, n_init, window, topk,   \
               nsplit, kps, sl2, per_head ? 1 : 0)
  if (D == 64) {
    if (E == 8) QAT_DEC(8, 64);
    else if (E == 16) QAT_DEC(16, 64);
    else QAT_DEC(32, 64);
  } else {
    if (E == 8) QAT_DEC(8, 128);
    else if (E == 16) QAT_DEC(16, 128);
    else QAT_DEC(32, 128);
  }
#undef QAT_DEC
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2((unsigned)cdiv(H * D, 256), (unsigned)batch);
  hipLaunchKernelGGL(esa_decode_combine_kernel, g2, dim3(256), 0, s, po, pm, pl, n_sel, (bf16*)out, lse, H, D, c0,
                     n_init, window, nsplit, kps, per_head ? 1 : 0);
  return hipGetLastError();
}

}  // namespace qat
