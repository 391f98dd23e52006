// MoBA block-sparse attention on the bf16 matrix cores.
//
// MoBA write-up (dtcms.com/wzjs/567377.html), section 2: MoBA(q, K, V) =
// Softmax(q K[I]^T) V[I] with I the union of the gated blocks; section 3:
// the query's own block is attended with a causal mask. Section 1 motivates
// the design with the mixture-of-experts analogy: every (token, head) row is
// routed to its gated blocks, which is how the work is laid out here.
//
// Each (token, head) row gates its own blocks, so query tiles of consecutive
// tokens share almost no past blocks. The rows are therefore dispatched like
// mixture-of-experts tokens: a counting sort groups the (row, slot) pairs by
// (sequence, KV head, block); every 128-row group attends the whole block
// (no mask) and leaves a normalised partial (o, lse) in its slot. The
// current-block kernel then runs causal attention over each row's own block
// on plain token tiles and folds the row's partials in by log-sum-exp merge.
#include "attn_core.h"
#include "common.h"
#include "launch.h"

namespace qat {

constexpr int kRowsPerTile = 128;

__global__ void fill_i32_kernel(int32_t* __restrict__ p, int64_t n, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// (row, slot) pairs of earlier blocks -> bucket counts.
__global__ void moba_count_kernel(const int32_t* __restrict__ blk, int64_t nrows, int64_t hq, int64_t hkv,
                                  int64_t q_len, int64_t q_start, int block, int topk, int64_t nbc,
                                  int32_t* __restrict__ counts) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= nrows * topk) return;
  const int64_t row = idx / topk;
  const int32_t b = blk[idx];
  const int64_t h = row % hq;
  const int64_t r = (row / hq) % q_len;
  const int64_t bi = row / (hq * q_len);
  const int64_t cur = (q_start + r) / block;
  if (b < 0 || b >= cur) return;
  const int64_t g = h / (hq / hkv);
  atomicAdd(&counts[(bi * hkv + g) * nbc + b], 1);
}

// Single workgroup: exclusive scans of the bucket counts and of their tile
// counts, the tile table {bucket, first entry}, scatter cursors and the
// number of tiles.
__global__ __launch_bounds__(1024) void moba_scan_kernel(const int32_t* __restrict__ counts, int64_t nb,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ cursor,
                                                         int2* __restrict__ tiles, int32_t* __restrict__ ntiles) {
  __shared__ int32_t s_cnt[1024];
  __shared__ int32_t s_til[1024];
  __shared__ int32_t carry[2];
  if (threadIdx.x == 0) { carry[0] = 0; carry[1] = 0; }
  __syncthreads();
  for (int64_t base = 0; base < nb; base += 1024) {
    const int64_t i = base + threadIdx.x;
    const int32_t c = i < nb ? counts[i] : 0;
    const int32_t tcount = (c + kRowsPerTile - 1) / kRowsPerTile;
    s_cnt[threadIdx.x] = c;
    s_til[threadIdx.x] = tcount;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {   // inclusive Hillis-Steele scan
      const int32_t a = threadIdx.x >= off ? s_cnt[threadIdx.x - off] : 0;
      const int32_t b = threadIdx.x >= off ? s_til[threadIdx.x - off] : 0;
      __syncthreads();
      s_cnt[threadIdx.x] += a;
      s_til[threadIdx.x] += b;
      __syncthreads();
    }
    const int32_t ex_c = carry[0] + s_cnt[threadIdx.x] - c;
    const int32_t ex_t = carry[1] + s_til[threadIdx.x] - tcount;
    if (i < nb) {
      offsets[i] = ex_c;
      cursor[i] = ex_c;
      for (int32_t j = 0; j < tcount; ++j) tiles[ex_t + j] = make_int2((int)i, ex_c + j * kRowsPerTile);
    }
    __syncthreads();
    if (threadIdx.x == 1023) { carry[0] += s_cnt[1023]; carry[1] += s_til[1023]; }
    __syncthreads();
  }
  if (threadIdx.x == 0) { offsets[nb] = carry[0]; ntiles[0] = carry[1]; }
}

// (row, slot) -> entries[cursor[bucket]++] = row * 16 + slot.
__global__ void moba_scatter_kernel(const int32_t* __restrict__ blk, int64_t nrows, int64_t hq, int64_t hkv,
                                    int64_t q_len, int64_t q_start, int block, int topk, int64_t nbc,
                                    int32_t* __restrict__ cursor, int32_t* __restrict__ entries) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= nrows * topk) return;
  const int64_t row = idx / topk;
  const int slot = (int)(idx % topk);
  const int32_t b = blk[idx];
  const int64_t h = row % hq;
  const int64_t r = (row / hq) % q_len;
  const int64_t bi = row / (hq * q_len);
  const int64_t cur = (q_start + r) / block;
  if (b < 0 || b >= cur) return;
  const int64_t g = h / (hq / hkv);
  const int32_t pos = atomicAdd(&cursor[(bi * hkv + g) * nbc + b], 1);
  entries[pos] = (int32_t)(row * 16 + slot);
}

// Past-block attention: one workgroup per tile of up to 128 dispatched rows
// of one (sequence, KV head, block); full block, no mask.
template <int D>
__global__ __launch_bounds__(256, 2) void moba_past_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const int2* __restrict__ tiles, const int32_t* __restrict__ ntiles, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ entries, bf16* __restrict__ part_o, float* __restrict__ part_lse,
    int64_t seq_len, int64_t hq, int64_t hkv, int64_t nbc, int64_t q_start, int64_t q_len, int block,
    int topk, float scale_log2) {
  extern __shared__ __align__(16) char smem_raw[];
  FaSmem<D>& sm = *reinterpret_cast<FaSmem<D>*>(smem_raw);
  const int tile = blockIdx.x;
  if (tile >= ntiles[0]) return;
  const int2 td = tiles[tile];
  const int bucket = td.x;
  const int first = td.y;
  const int count = min(kRowsPerTile, offsets[bucket + 1] - first);
  const int64_t b = bucket % nbc;
  const int64_t g = (bucket / nbc) % hkv;
  const int64_t bi = bucket / (nbc * hkv);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int myrow = wave * 32 + (lane & 31);
  const bool valid = myrow < count;
  const int32_t e = valid ? entries[first + myrow] : 0;
  const int64_t row = e >> 4;
  const int slot = e & 15;
  const int64_t h = row % hq;
  const int64_t r = (row / hq) % q_len;
  const bf16* qrow = q + ((bi * seq_len + q_start + r) * hq + h) * D;

  FaState<D> st;
  fa_init<D>(st, qrow, valid);
  const int64_t kv_row0 = ((bi * seq_len + b * block) * hkv + g) * D;
  const int64_t kv_stride = hkv * D;
  fa_segment<D>(st, sm, k, v, block, scale_log2,
                [=](int64_t j) -> int64_t { return kv_row0 + j * kv_stride; },
                [](int64_t) { return true; });
  float inv_l, lse;
  fa_finish<D>(st, inv_l, lse);
  if (!valid) return;
  const int64_t pidx = row * (topk - 1) + slot;
  bf16* dst = part_o + pidx * D;
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      bf16x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = (bf16)(st.o[t][i4 * 4 + i] * inv_l);
      *(bf16x4*)(dst + fa_d_of(t, i4 * 4)) = w;
    }
  if ((lane >> 5) == 0) part_lse[pidx] = lse;
}

// Current-block attention (causal) plus the log-sum-exp merge of the row's
// past-block partials. grid.x: 128-row tile within the block, grid.y: block
// index relative to the first block touched, grid.z: sequence * Hq + head.
template <int D>
__global__ __launch_bounds__(256, 2) void moba_current_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const int32_t* __restrict__ blk, const bf16* __restrict__ part_o, const float* __restrict__ part_lse,
    bf16* __restrict__ out, float* __restrict__ lse_out, int64_t seq_len, int64_t hq, int64_t hkv,
    int64_t q_start, int64_t q_len, int block, int topk, float scale_log2) {
  extern __shared__ __align__(16) char smem_raw[];
  FaSmem<D>& sm = *reinterpret_cast<FaSmem<D>*>(smem_raw);
  const int64_t bi = blockIdx.z / hq;
  const int64_t h = blockIdx.z % hq;
  const int64_t g = h / (hq / hkv);
  const int64_t c = q_start / block + blockIdx.y;
  const int64_t q_end = q_start + q_len;
  const int64_t lo = max(c * block, q_start);
  const int64_t hi = min((c + 1) * block, q_end);
  const int64_t t0 = lo + (int64_t)blockIdx.x * kRowsPerTile;
  if (t0 >= hi) return;
  const int64_t t_last = min(hi, t0 + kRowsPerTile) - 1;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = t0 + wave * 32 + (lane & 31);
  const bool valid = t <= t_last;
  const bf16* qrow = q + ((bi * seq_len + (valid ? t : t0)) * hq + h) * D;

  FaState<D> st;
  fa_init<D>(st, qrow, valid);
  const int64_t kpos0 = c * block;
  const int64_t kv_row0 = ((bi * seq_len + kpos0) * hkv + g) * D;
  const int64_t kv_stride = hkv * D;
  const int64_t qpos = valid ? t : -1;
  fa_segment<D>(st, sm, k, v, t_last - kpos0 + 1, scale_log2,
                [=](int64_t j) -> int64_t { return kv_row0 + j * kv_stride; },
                [=](int64_t j) { return kpos0 + j <= qpos; });
  float inv_l, lse;
  fa_finish<D>(st, inv_l, lse);
  if (!valid) return;

  // Merge with the past-block partials of this row.
  const int64_t row = (bi * q_len + (t - q_start)) * hq + h;
  const int32_t* br = blk + row * topk;
  float lse_tot = lse;
  for (int s = 0; s < topk; ++s) {
    const int32_t b = br[s];
    if (b >= 0 && b < c) {
      const float l2 = part_lse[row * (topk - 1) + s];
      const float mx = fmaxf(lse_tot, l2);
      lse_tot = mx + logf(expf(lse_tot - mx) + expf(l2 - mx));
    }
  }
  const float w_cur = expf(lse - lse_tot) * inv_l;
  float acc[D / 32][16];
#pragma unroll
  for (int tt = 0; tt < D / 32; ++tt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[tt][i] = st.o[tt][i] * w_cur;
  for (int s = 0; s < topk; ++s) {
    const int32_t b = br[s];
    if (b >= 0 && b < c) {
      const int64_t pidx = row * (topk - 1) + s;
      const float w = expf(part_lse[pidx] - lse_tot);
      const bf16* src = part_o + pidx * D;
#pragma unroll
      for (int tt = 0; tt < D / 32; ++tt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const bf16x4 pv = *(const bf16x4*)(src + fa_d_of(tt, i4 * 4));
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[tt][i4 * 4 + i] += w * (float)pv[i];
        }
    }
  }
  bf16* dst = out + row * D;
#pragma unroll
  for (int tt = 0; tt < D / 32; ++tt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      bf16x4 w4;
#pragma unroll
      for (int i = 0; i < 4; ++i) w4[i] = (bf16)acc[tt][i4 * 4 + i];
      *(bf16x4*)(dst + fa_d_of(tt, i4 * 4)) = w4;
    }
  if (lse_out && (lane >> 5) == 0) lse_out[row] = lse_tot;
}

// ---------------------------------------------------------------------------
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

int64_t moba_max_tiles(int64_t nrows, int topk, int64_t nbuckets) {
  return cdiv(nrows * (topk - 1), kRowsPerTile) + nbuckets;
}

hipError_t launch_moba_dispatch(const int32_t* blk, int64_t batch, int64_t hq, int64_t hkv, int64_t q_start,
                                int64_t q_len, int block, int topk, int64_t nbc, int32_t* counts,
                                int32_t* offsets, int32_t* cursor, int32_t* entries, int2* tiles,
                                int32_t* ntiles, hipStream_t s) {
  const int64_t nrows = batch * q_len * hq;
  const int64_t nbuckets = batch * hkv * nbc;
  hipError_t e = launch_fill_i32(counts, nbuckets, 0, s);
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)cdiv(nrows * topk, 256);
  if (nbuckets > 0) {
    hipLaunchKernelGGL(moba_count_kernel, dim3(grid), dim3(256), 0, s, blk, nrows, hq, hkv, q_len, q_start,
                       block, topk, nbc, counts);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(moba_scan_kernel, dim3(1), dim3(1024), 0, s, counts, nbuckets, offsets, cursor, tiles,
                     ntiles);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (nbuckets > 0) {
    hipLaunchKernelGGL(moba_scatter_kernel, dim3(grid), dim3(256), 0, s, blk, nrows, hq, hkv, q_len, q_start,
                       block, topk, nbc, cursor, entries);
    e = hipGetLastError();
  }
  return e;
}

template <int D>
static hipError_t launch_moba_attn_d(const bf16* q, const bf16* k, const bf16* v, const int32_t* blk,
                                     const int2* tiles, const int32_t* ntiles, const int32_t* offsets,
                                     const int32_t* entries, bf16* part_o, float* part_lse, bf16* out,
                                     float* lse, int64_t batch, int64_t seq_len, int64_t hq, int64_t hkv,
                                     int64_t nbc, int64_t q_start, int64_t q_len, int block, int topk,
                                     float scale, int64_t max_tiles, hipStream_t s) {
  const size_t smem = sizeof(FaSmem<D>);
  const float sl2 = scale * kLog2e;
  hipError_t e;
  if (topk > 1 && max_tiles > 0 && nbc > 0) {
    e = hipFuncSetAttribute((const void*)moba_past_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)smem);
    if (e != hipSuccess) return e;
    {
      KTimer tm("moba_past_attn", s);
      hipLaunchKernelGGL(moba_past_kernel<D>, dim3((unsigned)max_tiles), dim3(256), smem, s, q, k, v, tiles,
                         ntiles, offsets, entries, part_o, part_lse, seq_len, hq, hkv, nbc, q_start, q_len,
                         block, topk, sl2);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  e = hipFuncSetAttribute((const void*)moba_current_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)smem);
  if (e != hipSuccess) return e;
  const int64_t c_first = q_start / block;
  const int64_t c_last = (q_start + q_len - 1) / block;
  dim3 grid((unsigned)cdiv(block, kRowsPerTile), (unsigned)(c_last - c_first + 1), (unsigned)(batch * hq));
  {
    KTimer tm("moba_current_attn", s);
    hipLaunchKernelGGL(moba_current_kernel<D>, grid, dim3(256), smem, s, q, k, v, blk, part_o, part_lse, out,
                       lse, seq_len, hq, hkv, q_start, q_len, block, topk, sl2);
  }
  return hipGetLastError();
}

hipError_t launch_moba_attn_mfma(const void* q, const void* k, const void* v, const int32_t* blk,
                                 const int2* tiles, const int32_t* ntiles, const int32_t* offsets,
                                 const int32_t* entries, void* part_o, float* part_lse, void* out, float* lse,
                                 int64_t batch, int64_t seq_len, int64_t hq, int64_t hkv, int64_t d, int64_t nbc,
                                 int64_t q_start, int64_t q_len, int block, int topk, float scale,
                                 int64_t max_tiles, hipStream_t s) {
  if (d == 64)
    return launch_moba_attn_d<64>((const bf16*)q, (const bf16*)k, (const bf16*)v, blk, tiles, ntiles, offsets,
                                  entries, (bf16*)part_o, part_lse, (bf16*)out, lse, batch, seq_len, hq, hkv,
                                  nbc, q_start, q_len, block, topk, scale, max_tiles, s);
  return launch_moba_attn_d<128>((const bf16*)q, (const bf16*)k, (const bf16*)v, blk, tiles, ntiles, offsets,
                                 entries, (bf16*)part_o, part_lse, (bf16*)out, lse, batch, seq_len, hq, hkv,
                                 nbc, q_start, q_len, block, topk, scale, max_tiles, s);
}

}  // namespace qat
