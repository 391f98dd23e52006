// MoBA block gating: block mean-pool of the keys, block affinity scores and
// top-(k-1) selection plus the forced current block.
//
// MoBA write-up (dtcms.com/wzjs/567377.html), section 3 "block partition and
// selection": blocks of B keys; affinity s_i = <q, mean_pool(K[I_i])>; top-k
// gate; causality (no future blocks); the query's own block is always
// attended. k counts that forced block, so k - 1 earlier blocks are chosen;
// the current block never competes.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace qat {

// ---------------------------------------------------------------------------
// Mean pool, pass 1: a workgroup sums a slice of one block's tokens for all
// Hkv*d columns in float64. A thread owns 8 adjacent columns (one 16-byte
// load per token for bf16) and keeps up to 2 * kMpUnroll token rows in
// flight; the stream of K is read once, in whole rows.
constexpr int kMpThreads = 128;
constexpr int kMpUnroll = 8;

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]);
template <>
__device__ __forceinline__ void load8<bf16>(const bf16* p, float (&v)[8]) {
  const bf16x8 t = *(const bf16x8*)p;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (float)t[i];
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
  const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = a[i];
    v[4 + i] = b[i];
  }
}

// Raw token pieces (8 columns) as loaded, converted only when summed, so the
// loads of the next kMpUnroll rows can be in flight during the sums.
template <typename T>
struct MpRaw;
template <>
struct MpRaw<bf16> {
  bf16x8 v;
};
template <>
struct MpRaw<float> {
  f32x4 a, b;
};
__device__ __forceinline__ MpRaw<bf16> mp_load(const bf16* p) { return {*(const bf16x8*)p}; }
__device__ __forceinline__ MpRaw<float> mp_load(const float* p) {
  return {*(const f32x4*)p, *(const f32x4*)(p + 4)};
}
__device__ __forceinline__ void mp_add(double (&a)[8], const MpRaw<bf16>& r) {
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] += (double)(float)r.v[i];
}
__device__ __forceinline__ void mp_add(double (&a)[8], const MpRaw<float>& r) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] += (double)r.a[i];
    a[4 + i] += (double)r.b[i];
  }
}

template <typename T>
__global__ __launch_bounds__(kMpThreads) void meanpool_partial_kernel(
    const T* __restrict__ k, int64_t seq_len, int64_t cols, int block, int tokens_per_split,
    int nsplit, int64_t nbc, double* __restrict__ partial) {
  const int split = blockIdx.x;
  const int64_t b = blockIdx.y;
  const int64_t bi = blockIdx.z;
  const int64_t t0 = b * block + (int64_t)split * tokens_per_split;
  const int64_t t1 = min(b * block + (int64_t)block, t0 + tokens_per_split);
  const T* base = k + bi * seq_len * cols;
  double* dst = partial + ((bi * nbc + b) * nsplit + split) * cols;
  for (int64_t cg = threadIdx.x; cg < cols / 8; cg += kMpThreads) {
    const T* col = base + cg * 8;
    double a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = 0.0;
    // full groups of kMpUnroll rows, double-buffered: group g + 1 loads while
    // group g is summed (rows still summed in order)
    MpRaw<T> ra[kMpUnroll], rb[kMpUnroll];
    auto load_group = [&](MpRaw<T> (&r)[kMpUnroll], int64_t t) {
#pragma unroll
      for (int u = 0; u < kMpUnroll; ++u) r[u] = mp_load(col + (t + u) * cols);
      __builtin_amdgcn_sched_barrier(0);   // issue the loads here, ahead of the sums
    };
    auto add_group = [&](const MpRaw<T> (&r)[kMpUnroll]) {
#pragma unroll
      for (int u = 0; u < kMpUnroll; ++u) mp_add(a, r[u]);
    };
    const int64_t ng = (t1 - t0) / kMpUnroll;
    int64_t g = 0;
    if (ng > 0) load_group(ra, t0);
    for (; g + 2 < ng; g += 2) {   // both prefetches unconditional, so each wait is for one group
      load_group(rb, t0 + (g + 1) * kMpUnroll);
      add_group(ra);
      load_group(ra, t0 + (g + 2) * kMpUnroll);
      add_group(rb);
    }
    if (g + 1 < ng) {
      load_group(rb, t0 + (g + 1) * kMpUnroll);
      add_group(ra);
      add_group(rb);
    } else if (g < ng) {
      add_group(ra);
    }
    int64_t t = t0 + ng * kMpUnroll;
    for (; t < t1; ++t) mp_add(a, mp_load(col + t * cols));
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[cg * 8 + i] = a[i];
  }
}

// Mean pool in one pass, for launches over few blocks (a cache update, a
// short prefix): a workgroup per (64 columns, block, sequence); thread
// (lane l, column group c) sums tokens l, l + 32, ... of the block over the
// group's 8 columns in float64, and the 32 lane sums of a column are added in
// lane order through LDS. The float64 sums of bfloat16 keys are exact in any
// order, so the means equal those of the two-pass path.
constexpr int kMpdLanes = 32;
template <typename T>
__global__ __launch_bounds__(256) void meanpool_direct_kernel(
    const T* __restrict__ k, int64_t seq_len, int64_t cols, int block, int64_t count, int64_t nbc_total,
    int64_t first, float* __restrict__ kbar, bf16* __restrict__ planes) {
  __shared__ double red[kMpdLanes][65];
  const int cg = threadIdx.x & 7, tl = threadIdx.x >> 3;
  const int64_t c0 = (int64_t)blockIdx.x * 64 + cg * 8;
  const int64_t b = blockIdx.y, bi = blockIdx.z;
  const T* base = k + (bi * seq_len + b * block) * cols + c0;
  double a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = 0.0;
  int t = tl;
  for (; t + (kMpUnroll - 1) * kMpdLanes < block; t += kMpUnroll * kMpdLanes) {
    float v[kMpUnroll][8];
#pragma unroll
    for (int u = 0; u < kMpUnroll; ++u) load8<T>(base + (int64_t)(t + u * kMpdLanes) * cols, v[u]);
#pragma unroll
    for (int u = 0; u < kMpUnroll; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) a[i] += (double)v[u][i];
  }
  for (; t < block; t += kMpdLanes) {
    float v[8];
    load8<T>(base + (int64_t)t * cols, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] += (double)v[i];
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[tl][cg * 8 + i] = a[i];
  __syncthreads();
  if (threadIdx.x >= 64) return;
  const int c = threadIdx.x;
  double s = 0.0;
  for (int l = 0; l < kMpdLanes; ++l) s += red[l][c];
  const float x = (float)(s / (double)block);
  const int64_t col = (int64_t)blockIdx.x * 64 + c;
  kbar[((bi * nbc_total) + first + b) * cols + col] = x;
  if (planes) {   // whole range only: row bi * count + b of the planes
    const int64_t idx = (bi * count + b) * cols + col, total = gridDim.z * count * cols;
    const bf16 hi = (bf16)x;
    const float r1 = x - (float)hi;
    const bf16 mid = (bf16)r1;
    const bf16 lo = (bf16)(r1 - (float)mid);
    planes[idx] = hi;
    planes[total + idx] = mid;
    planes[2 * total + idx] = lo;
  }
}

// Mean pool, pass 2: sum the slices in order and divide by B. Besides the
// float32 means it writes, when `planes` is non-NULL, three bfloat16 planes
// hi/mid/lo with hi + mid + lo == mean exactly (each term is the rounded
// remainder of the previous ones), the operands of the matrix-core scoring.
// The partials cover blocks [first, first + count) of each sequence; the
// means land in a [batch, nbc_total, cols] array.
constexpr int kMpMaxSplits = 32;   // slices per block: see meanpool_tokens_per_split
__global__ void meanpool_finalize_kernel(const double* __restrict__ partial, int nsplit, int64_t count,
                                         int64_t nbc_total, int64_t first, int64_t nrows, int64_t cols, int block,
                                         float* __restrict__ kbar, bf16* __restrict__ planes) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = nrows * cols;
  if (idx >= total) return;
  const int64_t r = idx / cols, c = idx % cols;
  // all of the element's slice sums in flight at once, then added in order
  const double* pp = partial + r * nsplit * cols + c;
  double v[kMpMaxSplits];
#pragma unroll
  for (int i = 0; i < kMpMaxSplits; ++i) v[i] = i < nsplit ? pp[(int64_t)i * cols] : 0.0;
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < kMpMaxSplits; ++i)
    if (i < nsplit) s += v[i];
  const float x = (float)(s / (double)block);
  kbar[((r / count) * nbc_total + first + r % count) * cols + c] = x;
  if (planes) {
    const bf16 hi = (bf16)x;
    const float r1 = x - (float)hi;
    const bf16 mid = (bf16)r1;
    const bf16 lo = (bf16)(r1 - (float)mid);
    planes[idx] = hi;
    planes[total + idx] = mid;
    planes[2 * total + idx] = lo;
  }
}

// ---------------------------------------------------------------------------
// Running top list, descending score. Candidates arrive in ascending block
// order, so an equal score never displaces an earlier (smaller) block: the
// candidate goes before the first entry it strictly exceeds and the entries
// from there on shift down one slot (the scores are sorted, so "strictly
// exceeds" is false up to the insertion point and true after it). -inf
// candidates (not candidates of the row) never enter.
template <int KMAX>
__device__ __forceinline__ void top_insert(float (&tv)[KMAX], int (&ti)[KMAX], float cs, int cb) {
  bool prev = false;
  float pv = 0.f;
  int pi = 0;
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    const bool b = cs > tv[i];
    const float ov = tv[i];
    const int oi = ti[i];
    tv[i] = b ? (prev ? pv : cs) : ov;
    ti[i] = b ? (prev ? pi : cb) : oi;
    prev = b;
    pv = ov;
    pi = oi;
  }
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
    int64_t q_seq, int64_t q_off, int64_t hq, int64_t hkv, int64_t nbc, int64_t q_start, int64_t q_len,
    int block, int topk) {
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
    const T* qp = q + ((bi * q_seq + t - q_off) * hq + h) * D;
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
      top_insert<KMAX>(tv, ti, cs, cb);
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
// Scoring and selection for few query positions over many blocks (decode),
// one workgroup of 16 waves per (sequence, position, KV head): the group's
// query heads share the position, hence the candidate blocks, and each mean
// read. Heads go four at a time. A wave scores four blocks per step, 16 lanes
// per block: lane i of a 16-lane group holds dims [i E, (i + 1) E) (E = D / 16)
// of the four heads' queries in registers and reads the same dims of its
// block's mean (each block's mean row is read as one contiguous piece), and
// the 16 partial sums are added by lane exchanges. Lane j < 4 of a group then
// inserts head j's score into its running top list (score desc, ties to the
// smaller block; each list sees its blocks in ascending order). Each pick is
// the arg-max over all lists of that head: lane exchanges across the wave's
// four groups, then across the 16 waves through LDS.
constexpr int kSelRowsMaxQ = 16;   // positions per sequence up to which this kernel is used
constexpr int kSelGWaves = 16;

template <typename T, int D, int KMAX>
__global__ __launch_bounds__(kSelGWaves * 64) void moba_select_group_kernel(
    const T* __restrict__ q, const float* __restrict__ kbar, int32_t* __restrict__ blk, int64_t q_seq,
    int64_t q_off, int64_t hq, int64_t hkv, int64_t nbc, int64_t q_start, int64_t q_len, int block, int topk) {
  constexpr int E = D / 16;
  __shared__ float red_v[2][kSelGWaves][4];
  __shared__ int red_i[2][kSelGWaves][4];
  const int64_t r = blockIdx.x, g = blockIdx.y, bi = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int grp = lane >> 4, sub = lane & 15;
  const int64_t t = q_start + r;
  const int64_t cur = t / block;
  const int km = topk - 1;
  const int64_t ncand = km > 0 ? min(cur, nbc) : 0;
  const int npick = (int)min((int64_t)km, cur);
  const int64_t G = hq / hkv;
  const float* kb_g = kbar + (bi * nbc * hkv + g) * D + sub * E;   // block b: + b*hkv*D
  int round = 0;
  for (int64_t h0 = 0; h0 < G; h0 += 4) {
    const int nh = (int)min((int64_t)4, G - h0);
    float qv[4][E];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const T* qp = q + ((bi * q_seq + t - q_off) * hq + g * G + h0 + min(j, nh - 1)) * D + sub * E;
#pragma unroll
      for (int e = 0; e < E; ++e) qv[j][e] = to_f32(qp[e]);
    }
    float tv[KMAX];
    int ti[KMAX];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) { tv[i] = -__builtin_inff(); ti[i] = 0x7fffffff; }
    // U steps' mean reads are issued together, then scored in block order
    constexpr int U = KMAX > 7 ? 1 : 4;   // long top lists leave fewer registers
    constexpr int64_t STEP = kSelGWaves * 4;
    for (int64_t b0 = (int64_t)wv * 4; b0 < ncand; b0 += STEP * U) {
      float x[U][E];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t b = b0 + u * STEP + grp;
        const float* kr = kb_g + (b < ncand ? b : 0) * hkv * D;
#pragma unroll
        for (int e = 0; e < E; e += 4) {
          const float4 v = *reinterpret_cast<const float4*>(kr + e);
          x[u][e] = v.x; x[u][e + 1] = v.y; x[u][e + 2] = v.z; x[u][e + 3] = v.w;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t b = b0 + u * STEP + grp;
        float s[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float a = 0.f;
#pragma unroll
          for (int e = 0; e < E; ++e) a = fmaf(qv[j][e], x[u][e], a);
          a += __shfl_xor(a, 8, 64);
          a += __shfl_xor(a, 4, 64);
          a += __shfl_xor(a, 2, 64);
          a += __shfl_xor(a, 1, 64);
          s[j] = a;
        }
        const float mine = sub == 0 ? s[0] : sub == 1 ? s[1] : sub == 2 ? s[2] : s[3];
        if (b < ncand && sub < 4) top_insert<KMAX>(tv, ti, mine, (int)b);
      }
    }
    // picks of head slot j = sub (lanes sub < 4); the same in every such lane
    int pick[KMAX];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      pick[i] = 0x7fffffff;
      if (i < npick) {
        float bv = tv[0];
        int bb = ti[0];
#pragma unroll
        for (int off = 16; off <= 32; off <<= 1) {   // the same lane of the other groups
          const float ov = __shfl_xor(bv, off, 64);
          const int ob = __shfl_xor(bb, off, 64);
          if (ov > bv || (ov == bv && ob < bb)) { bv = ov; bb = ob; }
        }
        const int slot = round & 1;
        if (lane < 4) { red_v[slot][wv][lane] = bv; red_i[slot][wv][lane] = bb; }
        __syncthreads();   // the other slot's last readers are past this barrier too
        const int hs = sub & 3;
        bv = red_v[slot][0][hs];
        bb = red_i[slot][0][hs];
#pragma unroll
        for (int w2 = 1; w2 < kSelGWaves; ++w2) {
          const float ov = red_v[slot][w2][hs];
          const int ob = red_i[slot][w2][hs];
          if (ov > bv || (ov == bv && ob < bb)) { bv = ov; bb = ob; }
        }
        ++round;
        pick[i] = bb;
        if (sub < 4 && ti[0] == bb) {   // the owner of the pick drops its list head
#pragma unroll
          for (int m = 0; m + 1 < KMAX; ++m) { tv[m] = tv[m + 1]; ti[m] = ti[m + 1]; }
          tv[KMAX - 1] = -__builtin_inff();
          ti[KMAX - 1] = 0x7fffffff;
        }
      }
    }
    if (tid < nh) {   // lane j of wave 0 holds head slot j's picks
#pragma unroll
      for (int a2 = 0; a2 < KMAX; ++a2)
#pragma unroll
        for (int b2 = 0; b2 + 1 < KMAX - a2; ++b2) {
          const int lo = min(pick[b2], pick[b2 + 1]);
          const int hi = max(pick[b2], pick[b2 + 1]);
          pick[b2] = lo;
          pick[b2 + 1] = hi;
        }
      int32_t* out = blk + ((bi * q_len + r) * hq + g * G + h0 + tid) * topk;
#pragma unroll
      for (int i = 0; i < KMAX; ++i)
        if (i < npick) out[i] = pick[i];
      out[npick] = (int32_t)cur;
      for (int i = npick + 1; i < topk; ++i) out[i] = -1;
    }
  }
}

// ---------------------------------------------------------------------------
// Scoring and selection on the matrix cores (bfloat16 queries). The block
// means enter as three bfloat16 planes whose sum is the float32 mean exactly,
// so every product is exact and only the float32 accumulation rounds, as in
// a float32 dot product. Transposed tiles S^T = Kbar Q^T: a wave scores 64
// query rows (two 32-column tiles) against 32 blocks per round with
// v_mfma_f32_32x32x16_bf16; the scores go through LDS so that each lane then
// owns one query row and inserts that row's blocks in ascending order into
// its running top list (same order and tie rule as the scalar kernel).
constexpr int kSelWaves = 4;
constexpr int kSelRowsPerWave = 64;
constexpr int kSelBlocks = 32;   // blocks per round (one MFMA row tile)

// Three workgroups per CU fit the registers of top lists up to 3 entries;
// the 7- and 15-entry lists need the register budget of two.
template <int D, int KMAX>
__global__ __launch_bounds__(kSelWaves * 64, (KMAX <= 3 ? 3 : 2)) void moba_select_mfma_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ planes, int64_t plane_stride, int32_t* __restrict__ blk,
    int64_t seq_len, int64_t hq, int64_t hkv, int64_t nbc, int64_t q_start, int64_t q_len, int block, int topk) {
  constexpr int KP = D + 8;   // padded LDS row of one block's mean
  // the block-mean planes and the score transposes share one LDS area (a
  // barrier separates the last plane read from the first score write), so
  // four workgroups fit on a CU
  typedef bf16 PlaneT[kSelBlocks][KP];
  typedef float ScoreT[kSelRowsPerWave][kSelBlocks + 4];
  constexpr size_t kPlaneBytes = 3 * sizeof(PlaneT), kScoreBytes = kSelWaves * sizeof(ScoreT);
  __shared__ __attribute__((aligned(16))) char s_area[kPlaneBytes > kScoreBytes ? kPlaneBytes : kScoreBytes];
  PlaneT* kb_s = reinterpret_cast<PlaneT*>(s_area);
  ScoreT* sc_s = reinterpret_cast<ScoreT*>(s_area);
  const int64_t bi = blockIdx.z;
  const int64_t h = blockIdx.y;
  const int64_t g = h / (hq / hkv);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r0 = (int64_t)blockIdx.x * (kSelWaves * kSelRowsPerWave);
  const int64_t rw = r0 + wave * kSelRowsPerWave;   // first row of this wave
  const int km = topk - 1;

  // B operands: rows rw + lane%32 (tile 0) and rw + 32 + lane%32 (tile 1);
  // lane holds d = 16 ks + 8 (lane/32) .. + 8
  bf16x8 qa[D / 16], qb[D / 16];
  {
    const int64_t ra = min(rw + (lane & 31), q_len - 1), rb = min(rw + 32 + (lane & 31), q_len - 1);
    const bf16* pa = q + ((bi * seq_len + q_start + ra) * hq + h) * D + (lane >> 5) * 8;
    const bf16* pb = q + ((bi * seq_len + q_start + rb) * hq + h) * D + (lane >> 5) * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      qa[ks] = *(const bf16x8*)(pa + ks * 16);
      qb[ks] = *(const bf16x8*)(pb + ks * 16);
    }
  }
  // selection row of this lane
  const int64_t r = rw + lane;
  const bool valid = r < q_len;
  const int64_t t = q_start + (valid ? r : 0);
  const int64_t cur = t / block;
  float tv[KMAX];
  int ti[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) { tv[i] = -__builtin_inff(); ti[i] = 0x7fffffff; }

  const int64_t t_last = q_start + min(q_len, r0 + kSelWaves * kSelRowsPerWave) - 1;
  const int64_t nb_wg = km > 0 ? min(nbc, t_last / block) : 0;
  const bf16* pg = planes + ((bi * nbc) * hkv + g) * D;   // block b at pg + b*hkv*D (+ plane*plane_stride)
  constexpr int kPieces = 3 * kSelBlocks * D / 8;          // 16-byte pieces per round
  constexpr int kPer = kPieces / (kSelWaves * 64);
  static_assert(kPieces % (kSelWaves * 64) == 0, "plane pieces must split evenly over the threads");
  for (int64_t c0 = 0; c0 < nb_wg; c0 += kSelBlocks) {
    bf16x8 piece[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {   // all loads in flight before the first LDS write
      const int i = threadIdx.x + k * kSelWaves * 64;
      const int pl = i / (kSelBlocks * D / 8);
      const int rem = i % (kSelBlocks * D / 8);
      const int bb = rem / (D / 8), dd = (rem % (D / 8)) * 8;
      const int64_t b = min(c0 + bb, nb_wg - 1);
      piece[k] = *(const bf16x8*)(pg + pl * plane_stride + b * hkv * D + dd);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int i = threadIdx.x + k * kSelWaves * 64;
      const int pl = i / (kSelBlocks * D / 8);
      const int rem = i % (kSelBlocks * D / 8);
      const int bb = rem / (D / 8), dd = (rem % (D / 8)) * 8;
      *(bf16x8*)&kb_s[pl][bb][dd] = piece[k];
    }
    __syncthreads();
    f32x16 sa = {}, sb = {};
#pragma unroll
    for (int pl = 0; pl < 3; ++pl)
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 a = *(const bf16x8*)&kb_s[pl][lane & 31][ks * 16 + (lane >> 5) * 8];
        sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qa[ks], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[ks], sb, 0, 0, 0);
      }
    __syncthreads();   // every wave's plane reads are done before scores overwrite them
    // C layout: lane holds query column lane%32, block rows 8*gi + 4*(lane/32) + 0..3
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const int bcol = gi * 8 + (lane >> 5) * 4;
      *(f32x4*)&sc_s[wave][lane & 31][bcol] = f32x4{sa[4 * gi], sa[4 * gi + 1], sa[4 * gi + 2], sa[4 * gi + 3]};
      *(f32x4*)&sc_s[wave][32 + (lane & 31)][bcol] =
          f32x4{sb[4 * gi], sb[4 * gi + 1], sb[4 * gi + 2], sb[4 * gi + 3]};
    }
    __syncthreads();
    // blocks c0 + bb with bb >= nmine are not candidates of this row; they
    // enter as -inf and can only fill slots past the first min(k-1, cur)
    const int64_t nmine = valid ? min((int64_t)kSelBlocks, cur - c0) : 0;
    float scv[kSelBlocks];
#pragma unroll
    for (int j = 0; j < kSelBlocks / 4; ++j) {
      const f32x4 v = *(const f32x4*)&sc_s[wave][lane][4 * j];
#pragma unroll
      for (int x = 0; x < 4; ++x) scv[4 * j + x] = v[x];
    }
#pragma unroll
    for (int bb = 0; bb < kSelBlocks; ++bb) {
      float cs = bb < nmine ? scv[bb] : -__builtin_inff();
      int cb = (int)c0 + bb;
      top_insert<KMAX>(tv, ti, cs, cb);
    }
  }
  if (!valid) return;
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


// Resident variant for up to kSelLdsBytes of block means: a workgroup serves
// one (sequence, KV head) and stages the three planes of every block its rows
// can gate in LDS once; after that its waves run without barriers, each over
// its own strided list of 64-row chunks (chunk c = 64-row slice c / (Hq/Hkv)
// of query head c % (Hq/Hkv) of the group), loading the next chunk's queries
// while it ranks the current one's blocks. The scores stay in the accumulators: the
// lane of query column j holds 16 of each 32 blocks (rows 8gi + 4(lane/32) +
// 0..3), builds a top list over those in ascending block order for both of
// its query columns, and the two half-waves then trade the lists so that
// each lane merges the two halves of one query's candidates. The merge uses
// the full (score desc, block asc) order, so the result equals one pass of
// ordered insertion over all blocks.
constexpr int kSelPWaves = 4;
constexpr int kSelLdsBytes = 53248;   // three workgroups per CU

template <int KMAX>
__device__ __forceinline__ void top_merge(float (&tv)[KMAX], int (&ti)[KMAX], float cs, int cb) {
  bool prev = false;
  float pv = 0.f;
  int pi = 0;
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    const bool b = cs > tv[i] || (cs == tv[i] && cb < ti[i]);
    const float ov = tv[i];
    const int oi = ti[i];
    tv[i] = b ? (prev ? pv : cs) : ov;
    ti[i] = b ? (prev ? pi : cb) : oi;
    prev = b;
    pv = ov;
    pi = oi;
  }
}

__device__ __forceinline__ uint32_t sel_swap_halves(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return r[0] ^ r[1] ^ x;   // the value of lane (l + 32) mod 64
}

// Stages the three planes of blocks 0 .. nb_lds - 1 of one (sequence, KV
// head) into LDS rows of D + 8 elements (the pad spreads a column of rows over
// all banks): [plane][block][D + 8].
template <int D>
__device__ __forceinline__ void sel_stage_planes(bf16* kb_s, const bf16* pg, int64_t plane_stride, int64_t hkv,
                                                 int nb_lds) {
  constexpr int KP = D + 8;
  const int pieces = 3 * nb_lds * (D / 8);
  constexpr int U = 8;
  for (int i0 = threadIdx.x; i0 < pieces; i0 += U * kSelPWaves * 64) {
    bf16x8 pc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {   // clamped index: every load is in bounds, all in flight at once
      const int i = min(i0 + u * kSelPWaves * 64, pieces - 1);
      const int pl = i / (nb_lds * (D / 8)), rem = i % (nb_lds * (D / 8));
      pc[u] = *(const bf16x8*)(pg + pl * plane_stride + (int64_t)(rem / (D / 8)) * hkv * D + (rem % (D / 8)) * 8);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * kSelPWaves * 64;
      if (i < pieces) {
        const int pl = i / (nb_lds * (D / 8)), rem = i % (nb_lds * (D / 8));
        *(bf16x8*)&kb_s[(pl * nb_lds + rem / (D / 8)) * KP + (rem % (D / 8)) * 8] = pc[u];
      }
    }
  }
}

template <int D, int KMAX>
__global__ __launch_bounds__(kSelPWaves * 64, 2) void moba_select_resident_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ planes, int64_t plane_stride, int32_t* __restrict__ blk,
    int64_t seq_len, int64_t hq, int64_t hkv, int64_t nbc, int64_t q_start, int64_t q_len, int block, int topk,
    int nb_lds) {
  constexpr int KP = D + 8;   // padded LDS row of one block's mean
  extern __shared__ __attribute__((aligned(16))) char s_dyn[];
  bf16* kb_s = reinterpret_cast<bf16*>(s_dyn);   // [3][nb_lds][KP]
  const int64_t bi = blockIdx.y / hkv, g = blockIdx.y % hkv;
  const int64_t gs = hq / hkv;
  const int km = topk - 1;
  sel_stage_planes<D>(kb_s, planes + ((bi * nbc) * hkv + g) * D, plane_stride, hkv, nb_lds);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int hl = lane >> 5, l32 = lane & 31;
  // Chunk bookkeeping stays in wave-uniform 32-bit integers (positions and
  // block indices fit in 32 bits, seq_len < 2^31): chunk c is 64-row slice
  // rc = c / gs of group head hh = c % gs, and a wave steps c by `stride`.
  const int gsi = (int)gs;
  const int ql = (int)q_len, qs = (int)q_start;
  const int nrc = (ql + 63) / 64;
  const int stride = (int)gridDim.x * kSelPWaves;
  const int st_rc = stride / gsi, st_hh = stride % gsi;
  const int c_first = (int)blockIdx.x * kSelPWaves + wave;
  int rc = c_first / gsi, hh = c_first % gsi;
  const int64_t row_el = hq * D;   // elements from one position to the next
  const bf16* qg = q + ((bi * seq_len + q_start) * hq + g * gs) * D + hl * 8;
  auto load_q = [&](int rc_, int hh_, bf16x8 (&xa)[D / 16], bf16x8 (&xb)[D / 16]) {
    const int ra = min(rc_ * 64 + l32, ql - 1), rb = min(rc_ * 64 + 32 + l32, ql - 1);
    const bf16* pa = qg + ra * row_el + hh_ * D;
    const bf16* pb = qg + rb * row_el + hh_ * D;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      xa[ks] = *(const bf16x8*)(pa + ks * 16);
      xb[ks] = *(const bf16x8*)(pb + ks * 16);
    }
  };
  bf16x8 qa[D / 16], qb[D / 16];
  if (rc < nrc) load_q(rc, hh, qa, qb);
  while (rc < nrc) {
    int rn = rc + st_rc, hn = hh + st_hh;   // the wave's next chunk
    if (hn >= gsi) {
      hn -= gsi;
      ++rn;
    }
    const bool more = rn < nrc;
    const int h = (int)g * gsi + hh;
    const int ra = rc * 64 + l32, rb = ra + 32;   // query columns of the two score tiles
    const int cur_a = (qs + min(ra, ql - 1)) / block;
    const int cur_b = (qs + min(rb, ql - 1)) / block;
    const int own0 = (qs + rc * 64) / block;   // the chunk's smallest own block
    const int t_last = qs + min(ql, rc * 64 + 64) - 1;
    const int nbr = km > 0 ? min((int)nbc, t_last / block) : 0;   // <= nb_lds
    float tva[KMAX], tvb[KMAX];
    int tia[KMAX], tib[KMAX];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      tva[i] = tvb[i] = -__builtin_inff();
      tia[i] = tib[i] = 0x7fffffff;
    }
    for (int c0 = 0; c0 < nbr; c0 += 32) {
      const bf16* arow = kb_s + min(c0 + l32, nb_lds - 1) * KP + hl * 8;
      f32x16 sa = {}, sb = {};
#pragma unroll
      for (int pl = 0; pl < 3; ++pl)
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const bf16x8 a = *(const bf16x8*)(arow + pl * nb_lds * KP + ks * 16);
          sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qa[ks], sa, 0, 0, 0);
          sb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[ks], sb, 0, 0, 0);
        }
      // plane reads run three fragments ahead of the matrix ops using them
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
      for (int i = 0; i < 3 * (D / 16) - 3; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
      // the next chunk's queries replace these once the last round's matrix
      // ops have read them: their loads overlap the selection work below
      if (c0 + 32 >= nbr && more) load_q(rn, hn, qa, qb);
      // blocks c0 + bb with bb >= n are not candidates of the column's row;
      // when even the chunk's first row (the smallest own block) has all 32
      // as candidates, the round needs no mask (wave-uniform test)
      if (own0 - c0 >= 32) {
#pragma unroll
        for (int gi = 0; gi < 4; ++gi)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int bb = gi * 8 + hl * 4 + i;
            top_insert<KMAX>(tva, tia, sa[4 * gi + i], c0 + bb);
            top_insert<KMAX>(tvb, tib, sb[4 * gi + i], c0 + bb);
          }
      } else {
        const int n_a = cur_a - c0, n_b = cur_b - c0;
#pragma unroll
        for (int gi = 0; gi < 4; ++gi)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int bb = gi * 8 + hl * 4 + i;
            top_insert<KMAX>(tva, tia, bb < n_a ? sa[4 * gi + i] : -__builtin_inff(), c0 + bb);
            top_insert<KMAX>(tvb, tib, bb < n_b ? sb[4 * gi + i] : -__builtin_inff(), c0 + bb);
          }
      }
    }
    if (nbr <= 0 && more) load_q(rn, hn, qa, qb);
    // lane l < 32 keeps query ra (its list of column a), lane l + 32 keeps
    // query rb; each receives the other half's list of its query
    float ov[KMAX], rv[KMAX];
    int oi[KMAX], ri[KMAX];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      ov[i] = hl ? tvb[i] : tva[i];
      oi[i] = hl ? tib[i] : tia[i];
      rv[i] = __builtin_bit_cast(float, sel_swap_halves(__builtin_bit_cast(uint32_t, hl ? tva[i] : tvb[i])));
      ri[i] = (int)sel_swap_halves((uint32_t)(hl ? tia[i] : tib[i]));
    }
#pragma unroll
    for (int i = 0; i < KMAX; ++i) top_merge<KMAX>(ov, oi, rv[i], ri[i]);

    const int r = hl ? rb : ra;
    if (r < ql) {
      const int cur = hl ? cur_b : cur_a;
      const int npick = min(km, cur);
#pragma unroll
      for (int i = 0; i < KMAX; ++i)
        if (i >= npick) oi[i] = 0x7fffffff;
#pragma unroll
      for (int a = 0; a < KMAX; ++a)
#pragma unroll
        for (int b2 = 0; b2 + 1 < KMAX - a; ++b2) {
          const int lo = min(oi[b2], oi[b2 + 1]);
          const int hi = max(oi[b2], oi[b2 + 1]);
          oi[b2] = lo;
          oi[b2 + 1] = hi;
        }
      int32_t* out = blk + ((bi * q_len + r) * hq + h) * topk;
#pragma unroll
      for (int i = 0; i < KMAX; ++i)
        if (i < npick) out[i] = oi[i];
      out[npick] = cur;
      for (int i = npick + 1; i < topk; ++i) out[i] = -1;
    }
    rc = rn;
    hh = hn;
  }
}

// The same resident scheme on the 16x16x32 matrix op, for top lists of up to
// three past blocks. Its B operand gives each query row to four lanes with
// 16 consecutive bytes each, so one load instruction reads 64 contiguous
// bytes of 16 rows (the 32x32x16 layout reads 32 bytes of 32 rows, which
// streams the queries markedly slower from HBM). A wave works through its
// 64-row chunk in half-rounds of 16 blocks: per half-round lane l = j + 16 kg
// holds the scores of blocks 4 kg + 0..3 of the half-round for query rows
// j, j + 16, j + 32, j + 48 of the chunk, and keeps a top list per row. At
// the end of the chunk two exchanges (across lane bit 5, then bit 4) bring
// the four partial lists of row l to lane l, merged in the full (score desc,
// block asc) order, so the result again equals one ordered insertion pass
// over all blocks. Half-rounds past the chunk's last candidate block are
// skipped.
constexpr int kSel16MaxK = 3;   // longest past-block list of the 16x16x32 variant

// int vectors at the 4-byte alignment of a blk row
typedef int i32x2_u __attribute__((ext_vector_type(2), aligned(4)));
typedef int i32x3_u __attribute__((ext_vector_type(3), aligned(4)));
typedef int i32x4_u __attribute__((ext_vector_type(4), aligned(4)));

__device__ __forceinline__ uint32_t sel_swap_rows(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return r[0] ^ r[1] ^ x;   // the value of lane l ^ 16
}

template <int KMAX>
__device__ __forceinline__ void top_merge_from(float (&tv)[KMAX], int (&ti)[KMAX], const float (&rv)[KMAX],
                                               const int (&ri)[KMAX]) {
#pragma unroll
  for (int i = 0; i < KMAX; ++i) top_merge<KMAX>(tv, ti, rv[i], ri[i]);
}

template <int D, int KMAX>
__global__ __launch_bounds__(kSelPWaves * 64, 3) void moba_select_resident16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ planes, int64_t plane_stride, int32_t* __restrict__ blk,
    int64_t seq_len, int64_t hq, int64_t hkv, int64_t nbc, int64_t q_start, int64_t q_len, int block, int topk,
    int nb_lds) {
  constexpr int KP = D + 8;
  constexpr int KS = D / 32;   // k-steps of the matrix op
  static_assert(KMAX <= kSel16MaxK, "per-row lists of the 16x16x32 variant hold at most three blocks");
  extern __shared__ __attribute__((aligned(16))) char s_dyn[];
  bf16* kb_s = reinterpret_cast<bf16*>(s_dyn);   // [3][nb_lds][KP]
  const int64_t bi = blockIdx.y / hkv, g = blockIdx.y % hkv;
  const int64_t gs = hq / hkv;
  const int km = topk - 1;
  sel_stage_planes<D>(kb_s, planes + ((bi * nbc) * hkv + g) * D, plane_stride, hkv, nb_lds);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int j = lane & 15, kg = lane >> 4;
  // wave-uniform chunk bookkeeping, as in the 32x32x16 variant
  const int gsi = (int)gs;
  const int ql = (int)q_len, qs = (int)q_start;
  const int nrc = (ql + 63) / 64;
  const int stride = (int)gridDim.x * kSelPWaves;
  const int st_rc = stride / gsi, st_hh = stride % gsi;
  const int c_first = (int)blockIdx.x * kSelPWaves + wave;
  int rc = c_first / gsi, hh = c_first % gsi;
  const int64_t row_el = hq * D;
  const bf16* qg = q + ((bi * seq_len + q_start) * hq + g * gs) * D + kg * 8;
  // issued in the order the matrix ops consume them (k-step major)
  auto load_q = [&](int rc_, int hh_, bf16x8 (&x)[4][KS]) {
    const bf16* p[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) p[u] = qg + min(rc_ * 64 + 16 * u + j, ql - 1) * row_el + hh_ * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u][ks] = *(const bf16x8*)(p[u] + ks * 32);
  };
  // A chunk's blk rows leave one chunk later, just before the loads of the
  // chunk after: the memory counter retires in issue order, so the store is
  // then older than every load a later wait is for (a store issued behind
  // the loads would be waited for with them).
  int pend[4];
  int32_t* pend_out = nullptr;
  auto store_pending = [&]() {
    if (pend_out) {   // topk <= 4 entries in one store
      if (topk == 4) {
        *(i32x4_u*)pend_out = i32x4_u{pend[0], pend[1], pend[2], pend[3]};
      } else if (topk == 3) {
        *(i32x3_u*)pend_out = i32x3_u{pend[0], pend[1], pend[2]};
      } else if (topk == 2) {
        *(i32x2_u*)pend_out = i32x2_u{pend[0], pend[1]};
      } else {
        pend_out[0] = pend[0];
      }
      pend_out = nullptr;
    }
  };
  bf16x8 qf[4][KS];
  if (rc < nrc) load_q(rc, hh, qf);
  while (rc < nrc) {
    int rn = rc + st_rc, hn = hh + st_hh;   // the wave's next chunk
    if (hn >= gsi) {
      hn -= gsi;
      ++rn;
    }
    const bool more = rn < nrc;
    const int h = (int)g * gsi + hh;
    int cur[4];   // own block of query rows j + 16 u
#pragma unroll
    for (int u = 0; u < 4; ++u) cur[u] = (qs + min(rc * 64 + 16 * u + j, ql - 1)) / block;
    const int own0 = (qs + rc * 64) / block;   // the chunk's smallest own block
    const int t_last = qs + min(ql, rc * 64 + 64) - 1;
    const int nbr = km > 0 ? min((int)nbc, t_last / block) : 0;   // <= nb_lds
    float tv[4][KMAX];
    int ti[4][KMAX];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < KMAX; ++i) {
        tv[u][i] = -__builtin_inff();
        ti[u][i] = 0x7fffffff;
      }
    for (int c0 = 0; c0 < nbr; c0 += 16) {
      const bf16* arow = kb_s + min(c0 + j, nb_lds - 1) * KP + kg * 8;
      f32x4 acc[4] = {};
#pragma unroll
      for (int pl = 0; pl < 3; ++pl)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 a = *(const bf16x8*)(arow + pl * nb_lds * KP + ks * 32);
#pragma unroll
          for (int u = 0; u < 4; ++u) acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[u][ks], acc[u], 0, 0, 0);
        }
      // plane reads run two fragments ahead of the matrix ops using them
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int i = 0; i < 3 * KS - 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      // the last half-round issues the previous chunk's rows, then the next
      // chunk's query loads once its matrix ops have read the current
      // queries: those loads overlap the selection work below
      if (c0 + 16 >= nbr) {
        store_pending();
        if (more) load_q(rn, hn, qf);
      }
      const int b0 = c0 + 4 * kg;   // blocks b0 + 0..3 of this lane
      if (own0 - c0 >= 16) {   // every row of the chunk has all 16 as candidates
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r) top_insert<KMAX>(tv[u], ti[u], acc[u][r], b0 + r);
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            top_insert<KMAX>(tv[u], ti[u], b0 + r < cur[u] ? acc[u][r] : -__builtin_inff(), b0 + r);
      }
    }
    if (nbr <= 0) {
      store_pending();
      if (more) load_q(rn, hn, qf);
    }
    // exchange 1 (lane bit 5): keep the lists of rows 32 * (lane / 32) + j + 0, 16
    const bool hi5 = lane >= 32, hi4 = (lane & 16) != 0;
    float kv[2][KMAX];
    int ki[2][KMAX];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      float rv[KMAX];
      int ri[KMAX];
#pragma unroll
      for (int i = 0; i < KMAX; ++i) {
        kv[x][i] = hi5 ? tv[2 + x][i] : tv[x][i];
        ki[x][i] = hi5 ? ti[2 + x][i] : ti[x][i];
        rv[i] = __builtin_bit_cast(float, sel_swap_halves(__builtin_bit_cast(uint32_t, hi5 ? tv[x][i] : tv[2 + x][i])));
        ri[i] = (int)sel_swap_halves((uint32_t)(hi5 ? ti[x][i] : ti[2 + x][i]));
      }
      top_merge_from<KMAX>(kv[x], ki[x], rv, ri);
    }
    // exchange 2 (lane bit 4): keep the list of row `lane`
    float ov[KMAX];
    int oi[KMAX];
    {
      float rv[KMAX];
      int ri[KMAX];
#pragma unroll
      for (int i = 0; i < KMAX; ++i) {
        ov[i] = hi4 ? kv[1][i] : kv[0][i];
        oi[i] = hi4 ? ki[1][i] : ki[0][i];
        rv[i] = __builtin_bit_cast(float, sel_swap_rows(__builtin_bit_cast(uint32_t, hi4 ? kv[0][i] : kv[1][i])));
        ri[i] = (int)sel_swap_rows((uint32_t)(hi4 ? ki[0][i] : ki[1][i]));
      }
      top_merge_from<KMAX>(ov, oi, rv, ri);
    }

    const int r = rc * 64 + lane;
    if (r < ql) {
      const int cur_own = (qs + r) / block;
      const int npick = min(km, cur_own);
#pragma unroll
      for (int i = 0; i < KMAX; ++i)
        if (i >= npick) oi[i] = 0x7fffffff;
#pragma unroll
      for (int a = 0; a < KMAX; ++a)
#pragma unroll
        for (int b2 = 0; b2 + 1 < KMAX - a; ++b2) {
          const int lo = min(oi[b2], oi[b2 + 1]);
          const int hi = max(oi[b2], oi[b2 + 1]);
          oi[b2] = lo;
          oi[b2 + 1] = hi;
        }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int picked = oi[i < KMAX ? i : KMAX - 1];   // used for i < npick <= KMAX only
        pend[i] = i < npick ? picked : (i == npick ? cur_own : -1);
      }
      pend_out = blk + ((bi * q_len + r) * hq + h) * topk;
    }
    rc = rn;
    hh = hn;
  }
  store_pending();
}

// ---------------------------------------------------------------------------
int meanpool_tokens_per_split(int block) {
  // 64-token slices for blocks up to 2048 tokens, at most kMpMaxSplits beyond
  return (int)std::max<int64_t>(64, cdiv(block, kMpMaxSplits));
}
int meanpool_splits(int block) { return (int)cdiv(block, meanpool_tokens_per_split(block)); }

hipError_t launch_moba_meanpool(const void* k, bool bf, int64_t batch, int64_t seq_len, int64_t hkv,
                                int64_t d, int block, int64_t nbc, double* partial, float* kbar, bf16* planes,
                                hipStream_t s, int64_t first, int64_t count) {
  if (count < 0) count = nbc - first;
  if (count <= 0) return hipSuccess;
  const int nsplit = meanpool_splits(block);
  const int tps = meanpool_tokens_per_split(block);
  if (nsplit > kMpMaxSplits) return hipErrorInvalidValue;   // the finalize pass holds them all
  const int64_t cols = hkv * d;
  bf16* pl = (first == 0 && count == nbc) ? planes : nullptr;
  if (batch * count * nsplit < 1024) {   // few blocks: one pass, no partials
    dim3 g1((unsigned)(cols / 64), (unsigned)count, (unsigned)batch);
    const int64_t shift1 = first * block * cols;
    if (bf)
      hipLaunchKernelGGL(meanpool_direct_kernel<bf16>, g1, dim3(256), 0, s, (const bf16*)k + shift1, seq_len,
                         cols, block, count, nbc, first, kbar, pl);
    else
      hipLaunchKernelGGL(meanpool_direct_kernel<float>, g1, dim3(256), 0, s, (const float*)k + shift1, seq_len,
                         cols, block, count, nbc, first, kbar, pl);
    return hipGetLastError();
  }
  const int64_t shift = first * block * cols;   // elements: block `first` of sequence 0
  dim3 grid((unsigned)nsplit, (unsigned)count, (unsigned)batch);
  if (bf)
    hipLaunchKernelGGL(meanpool_partial_kernel<bf16>, grid, dim3(kMpThreads), 0, s, (const bf16*)k + shift,
                       seq_len, cols, block, tps, nsplit, count, partial);
  else
    hipLaunchKernelGGL(meanpool_partial_kernel<float>, grid, dim3(kMpThreads), 0, s, (const float*)k + shift,
                       seq_len, cols, block, tps, nsplit, count, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t total = batch * count * cols;
  hipLaunchKernelGGL(meanpool_finalize_kernel, dim3((unsigned)cdiv(total, 256)), dim3(256), 0, s,
                     partial, nsplit, count, nbc, first, batch * count, cols, block, kbar, pl);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_select_d(const T* q, const float* kbar, int32_t* blk, int64_t batch,
                                  int64_t q_seq, int64_t q_off, int64_t hq, int64_t hkv, int64_t nbc,
                                  int64_t q_start, int64_t q_len, int block, int topk, hipStream_t s) {
  dim3 grid((unsigned)cdiv(q_len, 256), (unsigned)hq, (unsigned)batch);
  const int km = topk - 1;
#define QAT_SEL(KM_)                                                                                    \
  hipLaunchKernelGGL((moba_score_select_kernel<T, D, KM_>), grid, dim3(256), 0, s, q, kbar, blk, q_seq,   \
                     q_off, hq, hkv, nbc, q_start, q_len, block, topk)
  if (km <= 1) QAT_SEL(1);
  else if (km == 2) QAT_SEL(2);
  else if (km == 3) QAT_SEL(3);
  else if (km <= 7) QAT_SEL(7);
  else QAT_SEL(15);
#undef QAT_SEL
  return hipGetLastError();
}

template <int D>
static hipError_t launch_select_mfma_d(const bf16* q, const bf16* planes, int64_t plane_stride, int32_t* blk,
                                       int64_t batch, int64_t seq_len, int64_t hq, int64_t hkv, int64_t nbc,
                                       int64_t q_start, int64_t q_len, int block, int topk, hipStream_t s) {
  const int km = topk - 1;
  // blocks any row can gate: 0 .. (last position) / block - 1
  const int64_t nb_gate = std::min<int64_t>(nbc, (q_start + q_len - 1) / block);
  const size_t lds = (size_t)3 * nb_gate * (D + 8) * sizeof(bf16);
  // resident kernels for lists of up to 7 past blocks (longer lists would
  // spill their registers); the streaming kernel below takes the rest
  if (lds <= (size_t)kSelLdsBytes && batch * hkv <= 65535 && km <= 7) {
    const int64_t nchunks = (hq / hkv) * cdiv(q_len, 64);
    // one wave of workgroups at the kernel's occupancy (three resident per CU
    // for the 16x16x32 variant, two for the longer lists) over 256 CUs,
    // shared by the groups
    const int64_t slots = km <= kSel16MaxK ? 768 : 512;
    const int64_t per_group = std::max<int64_t>(
        1, std::min<int64_t>(cdiv(slots, batch * hkv), cdiv(nchunks, kSelPWaves)));
    dim3 rgrid((unsigned)per_group, (unsigned)(batch * hkv));
    const size_t lds_launch = std::max<size_t>(lds, 16);
#define QAT_SELR(KM_)                                                                                      \
  hipLaunchKernelGGL((moba_select_resident_kernel<D, KM_>), rgrid, dim3(kSelPWaves * 64), lds_launch, s, q, \
                     planes, plane_stride, blk, seq_len, hq, hkv, nbc, q_start, q_len, block, topk, (int)nb_gate)
#define QAT_SELR16(KM_)                                                                                      \
  hipLaunchKernelGGL((moba_select_resident16_kernel<D, KM_>), rgrid, dim3(kSelPWaves * 64), lds_launch, s, q, \
                     planes, plane_stride, blk, seq_len, hq, hkv, nbc, q_start, q_len, block, topk, (int)nb_gate)
    static_assert(kSel16MaxK == 3, "dispatch below covers lists of 1..3 blocks");
    if (km <= 1) QAT_SELR16(1);
    else if (km == 2) QAT_SELR16(2);
    else if (km == 3) QAT_SELR16(3);
    else QAT_SELR(7);
#undef QAT_SELR
#undef QAT_SELR16
    return hipGetLastError();
  }
  dim3 grid((unsigned)cdiv(q_len, kSelWaves * kSelRowsPerWave), (unsigned)hq, (unsigned)batch);
#define QAT_SEL(KM_)                                                                                        \
  hipLaunchKernelGGL((moba_select_mfma_kernel<D, KM_>), grid, dim3(kSelWaves * 64), 0, s, q, planes,       \
                     plane_stride, blk, seq_len, hq, hkv, nbc, q_start, q_len, block, topk)
  if (km <= 1) QAT_SEL(1);
  else if (km == 2) QAT_SEL(2);
  else if (km == 3) QAT_SEL(3);
  else if (km <= 7) QAT_SEL(7);
  else QAT_SEL(15);
#undef QAT_SEL
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_select_rows_d(const T* q, const float* kbar, int32_t* blk, int64_t batch,
                                       int64_t q_seq, int64_t q_off, int64_t hq, int64_t hkv, int64_t nbc,
                                       int64_t q_start, int64_t q_len, int block, int topk, hipStream_t s) {
  dim3 grid((unsigned)q_len, (unsigned)hkv, (unsigned)batch);
#define QAT_SEL(KM_)                                                                                      \
  hipLaunchKernelGGL((moba_select_group_kernel<T, D, KM_>), grid, dim3(kSelGWaves * 64), 0, s, q, kbar,    \
                     blk, q_seq, q_off, hq, hkv, nbc, q_start, q_len, block, topk)
  const int km = topk - 1;
  if (km <= 1) QAT_SEL(1);
  else if (km == 2) QAT_SEL(2);
  else if (km == 3) QAT_SEL(3);
  else if (km <= 7) QAT_SEL(7);
  else QAT_SEL(15);
#undef QAT_SEL
  return hipGetLastError();
}

// Scoring from a float32 mean cache: few positions per sequence (decode)
// take a workgroup per (sequence, position, KV head); longer ranges the
// workgroup-per-256-rows kernel, which shares each staged mean among its rows.
hipError_t launch_moba_select_means(const void* q, bool bf, const float* kbar, int32_t* blk, int64_t batch,
                                    int64_t seq_len, int64_t q_seq, int64_t q_off, int64_t hq, int64_t hkv,
                                    int64_t d, int64_t nbc, int64_t q_start, int64_t q_len, int block, int topk,
                                    hipStream_t s) {
  (void)seq_len;
  if (q_len <= 0) return hipSuccess;
  const bool few = q_len <= kSelRowsMaxQ;
#define QAT_SM(T_, D_)                                                                                     \
  return few ? launch_select_rows_d<T_, D_>((const T_*)q, kbar, blk, batch, q_seq, q_off, hq, hkv, nbc,     \
                                            q_start, q_len, block, topk, s)                                 \
             : launch_select_d<T_, D_>((const T_*)q, kbar, blk, batch, q_seq, q_off, hq, hkv, nbc, q_start, \
                                       q_len, block, topk, s)
  if (bf) {
    if (d == 64) QAT_SM(bf16, 64);
    QAT_SM(bf16, 128);
  }
  if (d == 64) QAT_SM(float, 64);
  QAT_SM(float, 128);
#undef QAT_SM
}

hipError_t launch_moba_select(const void* q, bool bf, const float* kbar, const bf16* planes, int32_t* blk,
                              int64_t batch, int64_t seq_len, int64_t hq, int64_t hkv, int64_t d, int64_t nbc,
                              int64_t q_start, int64_t q_len, int block, int topk, hipStream_t s) {
  if (q_len <= 0) return hipSuccess;
  if (bf) {
    const int64_t ps = batch * nbc * hkv * d;
    if (d == 64)
      return launch_select_mfma_d<64>((const bf16*)q, planes, ps, blk, batch, seq_len, hq, hkv, nbc, q_start,
                                      q_len, block, topk, s);
    return launch_select_mfma_d<128>((const bf16*)q, planes, ps, blk, batch, seq_len, hq, hkv, nbc, q_start,
                                     q_len, block, topk, s);
  }
  if (d == 64)
    return launch_select_d<float, 64>((const float*)q, kbar, blk, batch, seq_len, 0, hq, hkv, nbc, q_start,
                                      q_len, block, topk, s);
  return launch_select_d<float, 128>((const float*)q, kbar, blk, batch, seq_len, 0, hq, hkv, nbc, q_start,
                                     q_len, block, topk, s);
}

}  // namespace qat
