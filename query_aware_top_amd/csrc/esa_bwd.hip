// ESA attention gradients with the selection held fixed (the selection is a
// discrete top-k over the compressed scores; the compression map is learned
// offline in the ESA write-up, so no gradient flows into it here). Each
// chunk query i of head h attends its sequence's key list: the gathered keys
// (initial, selected, local; never masked) followed by the chunk's own keys
// [c0, c0 + i] (causal) -- ESA write-up, the four-part split. Gradients as
// for any softmax attention over an explicit key set: p = exp(scale q.k -
// lse), dp = dO.v, D = sum p dp, dq = scale sum p (dp - D) k,
// dk += scale p (dp - D) q, dv += p dO.
//
// Two kernels on the bf16 matrix cores (the gradient tile engine):
//   dq  grid (128-query tiles, head, sequence): the forward's layout over
//       the key list; forms D in the same pass and writes dq and D;
//   kv  grid (128-key tiles of the key list, head, sequence): the keys'
//       K^T / V^T fragments in registers, the chunk's query rows of that
//       head streamed through LDS 64 at a time; adds dK, dV into the rows of
//       the caches' gradient at the keys' positions (every position appears
//       once in a sequence's list, so no two workgroups touch one row).
#include "attn_bwd.h"
#include "attn_core.h"
#include "common.h"
#include "launch.h"

namespace qat {

constexpr int kEsaBwdRows = 32 * kBwdNW;

// gathered keys of selection lv (initial + selected + local); with per-head
// selection (ph) head h of sequence b reads selection lv = b H + h
__device__ __forceinline__ int esa_bwd_ngather(const int32_t* n_sel, int64_t bi, int64_t c0, int64_t n_init,
                                               int64_t window) {
  const int64_t ni = min(n_init, c0);
  const int64_t nl = c0 > n_init ? c0 - max(n_init, c0 - window) : 0;
  return (int)(ni + n_sel[bi] + nl);
}

template <int D>
__global__ __launch_bounds__(64 * kBwdNW, 1) void esa_bwd_dq_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const float* __restrict__ lse, const int32_t* __restrict__ keylist,
    int64_t kls, const int32_t* __restrict__ n_sel, float* __restrict__ dq, float* __restrict__ delta, int64_t H,
    int64_t ctx_len, int64_t c0, int64_t m, int64_t n_init, int64_t window, float scale, int ph) {
  QAT_FA_SMEM(D, sm);
  int64_t id = xcd_logical_id(blockIdx.x, gridDim.x);
  const int64_t ntile = cdiv(m, kEsaBwdRows);
  // later row tiles attend more of the chunk's keys: dispatched first
  const int64_t qt = ntile - 1 - id % ntile;
  id /= ntile;
  const int64_t h = id % H, bi = id / H;
  const int64_t i0 = qt * kEsaBwdRows;
  const int64_t i_last = min(m, i0 + kEsaBwdRows) - 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t i = i0 + wave * 32 + (lane & 31);
  const bool valid = i <= i_last;
  const int64_t row = (bi * m + (valid ? i : i0)) * H + h;
  DqState<D> st;
  dq_init<D>(st, q + row * D, dout + row * D, lse[row], valid);
  const int64_t lv = ph ? bi * H + h : bi;
  const int ng = esa_bwd_ngather(n_sel, lv, c0, n_init, window);
  const int HD = (int)(H * D);
  const int32_t* lst = keylist + lv * kls;
  const int lim = ng + (valid ? (int)i : -1);   // this lane attends list entries j <= lim
  dq_segment<D, kBwdNW>(st, sm, k + (bi * ctx_len * H + h) * D, v + (bi * ctx_len * H + h) * D,
                        ng + (int)(i_last + 1), scale * kLog2e, [=](int j) { return lst[j] * HD; },
                        [=](int j) { return j <= lim; });
  const float dsum = xor32_sum(st.dsum);
  if (!valid) return;
  const int hl = lane >> 5;
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

template <int D>
__global__ __launch_bounds__(64 * kBwdNW, 1) void esa_bwd_kv_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    const int32_t* __restrict__ keylist, int64_t kls, const int32_t* __restrict__ n_sel, float* __restrict__ dk,
    float* __restrict__ dv, int64_t H, int64_t ctx_len, int64_t c0, int64_t m, int64_t n_init, int64_t window,
    float scale, int ph) {
  QAT_FA_SMEM(D, sm);
  extern __shared__ __align__(16) char eb_dyn[];   // beyond the 64 KiB of tile buffers
  float* s_lse = reinterpret_cast<float*>(eb_dyn);   // [2][64]
  float* s_di = s_lse + 128;                          // [2][64]
  int64_t id = xcd_logical_id(blockIdx.x, gridDim.x);
  const int64_t nkt = cdiv(kls, kKvKeys);
  const int64_t kt = id % nkt;
  id /= nkt;
  const int64_t h = id % H, bi = id / H;
  const int64_t lv = ph ? bi * H + h : bi;
  const int ng = esa_bwd_ngather(n_sel, lv, c0, n_init, window);
  const int nlist = ng + (int)m;
  const int j0 = (int)kt * kKvKeys;
  if (j0 >= nlist) return;   // uniform
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int j = j0 + wave * 32 + (lane & 31);
  const bool kvalid = j < nlist;
  const int32_t* lst = keylist + lv * kls;
  const int64_t pos = lst[kvalid ? j : j0];
  const int64_t krow = ((bi * ctx_len + pos) * H + h) * D;
  // rows: the chunk's queries of head h; a chunk key j >= ng is seen by
  // queries i >= j - ng only, so the workgroup starts at its first key's row
  const int i_start = j0 > ng ? (j0 - ng) / 64 * 64 : 0;
  const int nrows = (int)m - i_start;
  const int nt = (nrows + 63) / 64;
  const bf16* qbase = q + ((bi * m + i_start) * H + h) * D;
  const bf16* dbase = dout + ((bi * m + i_start) * H + h) * D;
  const int HD = (int)(H * D);
  const float sl2 = scale * kLog2e;
  // the q / dO rows [i_start, m) of head h through buffer resources: per-lane
  // offsets recomputed at each issue (this kernel is at the register limit),
  // the tile start in the range-checked offset (rows past m read as zero;
  // their p is masked)
  const uint32_t region = nrows > 0 ? (uint32_t)(((int64_t)(nrows - 1) * HD + D) * 2) : 0u;
  const __amdgpu_buffer_rsrc_t rq = fa_rsrc(qbase, region), rd = fa_rsrc(dbase, region);
  const float* lrow = lse + (bi * m + i_start) * H + h;     // the rows' lse and D, row stride H
  const float* drow = delta + (bi * m + i_start) * H + h;
  auto issue = [&](bf16* qdst, bf16* ddst, int buf, int rt) {
    const int r0 = rt * 64, n = min(64, nrows - r0);
    FaContig<D, kBwdNW>::issue_checked_fresh(qdst, rq, r0, HD);
    FaContig<D, kBwdNW>::issue_checked_fresh(ddst, rd, r0, HD);
    if (wave == 0) {   // rows past the tile's end repeat its last row (masked)
      const int ro = (r0 + min(fa_fresh_lane(), n - 1)) * (int)H;
      __builtin_amdgcn_global_load_lds((const global_void*)(lrow + ro), (lds_void*)(s_lse + buf * 64), 4, 0, 0);
      __builtin_amdgcn_global_load_lds((const global_void*)(drow + ro), (lds_void*)(s_di + buf * 64), 4, 0, 0);
    }
  };
  // row m_local of tile rt (query i_start + 64 rt + m_local) sees this lane's
  // key iff it exists and, for a chunk key, i >= j - ng
  // (the lane's key index is re-derived per tile from fa_fresh_lane(), and
  // its cache row after the loop: nothing per lane is held across the loop)
  auto row_ok = [=](int rt) {
    const int jf = j0 + wave * 32 + (fa_fresh_lane() & 31);
    const int kfirst = jf >= ng ? jf - ng - i_start : -(1 << 30);
    const int n = min(64, nrows - rt * 64), mm0 = kfirst - rt * 64;
    return [=](int ml) { return ml < n && ml >= mm0; };
  };
  KvState<D> st;
  if (nt > 0) issue(sm.k0, sm.v0, 0, 0);
  kv_load<D>(st, k + krow, v + krow);
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
  fa_wait_loads();
  if (!kvalid) return;
  const int64_t krow_end = ((bi * ctx_len + lst[j0 + wave * 32 + (fa_fresh_lane() & 31)]) * H + h) * D;
  // add into the caches' gradient rows (accumulator layout d = 32 tq + 8 gi + 4 hl + e)
  const int hl = lane >> 5;
#pragma unroll
  for (int tq = 0; tq < D / 32; ++tq)
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const int d0 = 32 * tq + 8 * gi + 4 * hl;
      f32x4 a = *(const f32x4*)(dk + krow_end + d0), b = *(const f32x4*)(dv + krow_end + d0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[e] += scale * st.fa.o[tq][4 * gi + e];
        b[e] += st.dv[tq][4 * gi + e];
      }
      *(f32x4*)(dk + krow_end + d0) = a;
      *(f32x4*)(dv + krow_end + d0) = b;
    }
}

// ---------------------------------------------------------------------------
hipError_t launch_esa_bwd(const void* q, const void* k, const void* v, const int32_t* sel, const int32_t* n_sel,
                          const void* dout, const float* lse, int32_t* keylist, float* dq, float* delta, float* dk,
                          float* dv, int64_t batch, int64_t H, int64_t D, int64_t ctx_len, int64_t c0, int64_t m,
                          int64_t n_init, int64_t window, int topk, float scale, bool per_head, hipStream_t s) {
  const int64_t kls = esa_keylist_len(n_init, topk, window, m);
  hipError_t e = launch_esa_keylist(sel, n_sel, keylist, per_head ? batch * H : batch, c0, m, n_init, window, topk, s);
  if (e != hipSuccess) return e;
  static const bool lds_ok = [] {
    bool ok = hipFuncSetAttribute((const void*)esa_bwd_kv_kernel<64>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  1024) == hipSuccess;
    ok &= hipFuncSetAttribute((const void*)esa_bwd_kv_kernel<128>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              1024) == hipSuccess;
    return ok;
  }();
  if (!lds_ok) return hipErrorInvalidConfiguration;
  dim3 g_dq((unsigned)(cdiv(m, kEsaBwdRows) * H * batch));
  dim3 g_kv((unsigned)(cdiv(kls, kKvKeys) * H * batch));
#define QAT_EB(D_)                                                                                            \
  do {                                                                                                        \
    {                                                                                                         \
      KTimer tm("esa_bwd_dq", s);                                                                             \
      launch_timed("esa_bwd_dq", esa_bwd_dq_kernel<D_>, g_dq, dim3(64 * kBwdNW), 0, s, (const bf16*)q,        \
                   (const bf16*)k, (const bf16*)v, (const bf16*)dout, lse, (const int32_t*)keylist, kls, n_sel, \
                   dq, delta, H, ctx_len, c0, m, n_init, window, scale, per_head ? 1 : 0);                    \
    }                                                                                                         \
    if ((e = hipGetLastError()) != hipSuccess) return e;                                                      \
    KTimer tm("esa_bwd_kv", s);                                                                               \
    launch_timed("esa_bwd_kv", esa_bwd_kv_kernel<D_>, g_kv, dim3(64 * kBwdNW), 1024, s, (const bf16*)q,       \
                 (const bf16*)k, (const bf16*)v, (const bf16*)dout, lse, (const float*)delta,                 \
                 (const int32_t*)keylist, kls, n_sel, dk, dv, H, ctx_len, c0, m, n_init, window, scale,       \
                 per_head ? 1 : 0);                                                                           \
  } while (0)
  if (D == 64) QAT_EB(64);
  else QAT_EB(128);
#undef QAT_EB
  return hipGetLastError();
}

}  // namespace qat
