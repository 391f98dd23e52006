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
#include <algorithm>
#include <type_traits>

#include "attn_core.h"
#include "common.h"
#include "launch.h"

namespace qat {

constexpr int kNW = 8;                    // waves per past-block workgroup
constexpr int kThreads = 64 * kNW;
constexpr int kRowsPerTile = 32 * kNW;    // query rows per attention workgroup

__global__ void fill_i32_kernel(int32_t* __restrict__ p, int64_t n, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// Dispatch keys: (row, slot) pairs whose gated block is an earlier block go
// to bucket (sequence, KV head, block). One thread takes whole rows (the
// row's head, position and block bounds are decoded once for all its slots,
// in 32-bit arithmetic: rows < 2^27 and every index below fits in int32).
// Counting and scattering aggregate in LDS per workgroup first (one global
// atomic per bucket and workgroup), since strongly preferred blocks collect
// most rows of the sequence. Gated lists are ascending with the current
// block last among the valid entries, so earlier blocks sit in the first
// topk - 1 slots; the last slot is never dispatched, which bounds the entry
// and partial arrays at topk - 1 per row whatever the list holds.
constexpr int kDispatchLdsBuckets = 4096;
constexpr int kDispatchRowsPerThread = 8;

struct MobaRowMap {
  uint32_t hq, q_len, q_start, block, group, hkv, nbc, seq_len;
};

struct MobaRow {
  int32_t bucket0;   // bucket of block 0 of the row's (sequence, KV head)
  int32_t cur;       // the row's own block (attended by the current-block pass)
  int32_t qrow;      // index of the row's query vector in q
};

__device__ __forceinline__ MobaRow moba_row(const MobaRowMap& m, uint32_t row) {
  const uint32_t h = row % m.hq, t = row / m.hq;
  const uint32_t r = t % m.q_len, bi = t / m.q_len;
  MobaRow o;
  o.cur = (int32_t)((m.q_start + r) / m.block);
  o.bucket0 = (int32_t)((bi * m.hkv + h / m.group) * m.nbc);
  o.qrow = (int32_t)((bi * m.seq_len + m.q_start + r) * m.hq + h);
  return o;
}

struct MobaNoSkip {
  __device__ void operator()(int32_t, int) const {}
};

// Calls f(row, slot, row descriptor, block) for every dispatched (row, slot)
// pair among this thread's rows, and skip(row, slot) for every other slot
// of those rows. The gated lists of four rows (their first four slots) are
// loaded together, from clamped in-bounds indices, before any of them is
// used, so that the loads overlap.
template <typename F, typename S = MobaNoSkip>
__device__ __forceinline__ void moba_for_each_pair(const int32_t* __restrict__ blk, int32_t r0, int32_t r1,
                                                   const MobaRowMap& m, int topk, F f, S skip = S{}) {
  constexpr int RB = 4, SB = 4;
  const int km = topk - 1;   // >= 1
#pragma unroll 1
  for (int k0 = 0; k0 < kDispatchRowsPerThread; k0 += RB) {
    int32_t bv[RB][SB];
    int32_t rows[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      rows[i] = r0 + (int32_t)threadIdx.x + (k0 + i) * 256;
      const int32_t rc = min(rows[i], r1 - 1);
#pragma unroll
      for (int s = 0; s < SB; ++s) bv[i][s] = blk[rc * topk + min(s, km - 1)];
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      if (rows[i] >= r1) continue;
      const MobaRow mr = moba_row(m, (uint32_t)rows[i]);
#pragma unroll
      for (int s = 0; s < SB; ++s) {
        const int32_t b = bv[i][s];
        if (s < km) {
          if (b >= 0 && b < mr.cur) f(rows[i], s, mr, b);
          else skip(rows[i], s);
        }
      }
      for (int s = SB; s < km; ++s) {
        const int32_t b = blk[rows[i] * topk + s];
        if (b >= 0 && b < mr.cur) f(rows[i], s, mr, b);
        else skip(rows[i], s);
      }
    }
  }
}

// With the counts in LDS, each workgroup also records where its entries
// start inside each bucket (wg_loc, may be NULL): the value its one atomic
// add to the bucket's total returns. The scatter then places its entries
// from there without counting its rows again or taking atomics of its own.
__global__ __launch_bounds__(256) void moba_count_kernel(const int32_t* __restrict__ blk, int32_t nrows,
                                                         MobaRowMap m, int topk, int32_t nbuckets,
                                                         int32_t* __restrict__ counts, int32_t* __restrict__ wg_loc) {
  __shared__ int32_t loc[kDispatchLdsBuckets];
  const bool use_lds = nbuckets <= kDispatchLdsBuckets;
  if (use_lds) {
    for (int i = threadIdx.x; i < nbuckets; i += blockDim.x) loc[i] = 0;
    __syncthreads();
  }
  const int32_t r0 = blockIdx.x * (256 * kDispatchRowsPerThread);
  const int32_t r1 = min(nrows, r0 + 256 * kDispatchRowsPerThread);
  moba_for_each_pair(blk, r0, r1, m, topk, [&](int32_t, int, const MobaRow& mr, int32_t b) {
    if (use_lds) atomicAdd(&loc[mr.bucket0 + b], 1);
    else atomicAdd(&counts[mr.bucket0 + b], 1);
  });
  if (use_lds) {
    __syncthreads();
    for (int i = threadIdx.x; i < nbuckets; i += blockDim.x) {
      const int32_t before = loc[i] ? atomicAdd(&counts[i], loc[i]) : 0;
      if (wg_loc) wg_loc[(int64_t)blockIdx.x * nbuckets + i] = before;
    }
  }
}

// Stable placement, step 2: wg_base[w][b] = offsets[b] + sum of the bucket's
// counts of the workgroups before w (row order). A workgroup takes 64
// buckets; its 16 waves each sum a sixteenth of the workgroup range (16
// loads in flight per lane), then write the running offsets of their part.
constexpr int kScanParts = 16;
__global__ __launch_bounds__(64 * kScanParts) void moba_wg_scan_kernel(const int32_t* __restrict__ wg_counts,
                                                                       int32_t nwg, int32_t nbuckets,
                                                                       const int32_t* __restrict__ offsets,
                                                                       int32_t* __restrict__ wg_base) {
  __shared__ int32_t part[kScanParts][64];
  constexpr int U = 16;
  const int lane = threadIdx.x & 63, pt = threadIdx.x >> 6;
  const int32_t b = blockIdx.x * 64 + lane;
  const int32_t np = (nwg + kScanParts - 1) / kScanParts;
  const int32_t w0 = pt * np, w1 = min(nwg, w0 + np);
  const bool bv = b < nbuckets;
  int32_t sum = 0;
  for (int32_t wb = w0; wb < w1; wb += U) {
    int32_t c[U];
#pragma unroll
    for (int u = 0; u < U; ++u) c[u] = (bv && wb + u < w1) ? wg_counts[(int64_t)(wb + u) * nbuckets + b] : 0;
#pragma unroll
    for (int u = 0; u < U; ++u) sum += c[u];
  }
  part[pt][lane] = sum;
  __syncthreads();
  if (!bv) return;
  int32_t run = offsets[b];
  for (int q2 = 0; q2 < pt; ++q2) run += part[q2][lane];
  for (int32_t wb = w0; wb < w1; wb += U) {
    int32_t c[U];
#pragma unroll
    for (int u = 0; u < U; ++u) c[u] = wb + u < w1 ? wg_counts[(int64_t)(wb + u) * nbuckets + b] : 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (wb + u < w1) wg_base[(int64_t)(wb + u) * nbuckets + b] = run;
      run += c[u];
    }
  }
}

// Exclusive prefix sums of the bucket sizes (entry offsets) and of their tile
// counts; one workgroup, 1024 buckets per pass. `counts` is overwritten with
// the tile prefix (counts[nb] = number of tiles), which the tile pass reads.
__global__ __launch_bounds__(1024) void moba_scan_kernel(int32_t* __restrict__ counts, int32_t nb,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ cursor,
                                                         int32_t* __restrict__ ntiles) {
  __shared__ int32_t s_cnt[1024];
  __shared__ int32_t s_til[1024];
  __shared__ int32_t carry[2];
  if (threadIdx.x == 0) { carry[0] = 0; carry[1] = 0; }
  __syncthreads();
  for (int32_t base = 0; base < nb; base += 1024) {
    const int32_t i = base + threadIdx.x;
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
    if (i < nb) {
      const int32_t ex_c = carry[0] + s_cnt[threadIdx.x] - c;
      offsets[i] = ex_c;
      cursor[i] = ex_c;
      counts[i] = carry[1] + s_til[threadIdx.x] - tcount;
    }
    __syncthreads();
    if (threadIdx.x == 1023) { carry[0] += s_cnt[1023]; carry[1] += s_til[1023]; }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    offsets[nb] = carry[0];
    counts[nb] = carry[1];
    ntiles[0] = carry[1];
  }
}

// Stable placement (the gradient pass): a workgroup owns kStableEntries
// (row, slot) sequence numbers of consecutive rows, seq = (row - r0) * km +
// slot. Step 1 counts its entries per bucket (wg_counts[w][b], and the
// bucket totals); step 2 (moba_wg_scan_kernel) turns the counts into the
// workgroup's first position in every bucket; step 3 sorts the workgroup's
// (bucket, seq) keys in LDS (bitonic) and writes each entry at its bucket's
// base plus its rank among the workgroup's entries of that bucket. A
// bucket's entries thus run in row order, whatever order the hardware
// schedules the workgroups in.
constexpr int kStableEntries = 8192;   // widest sort (32-bit keys: 32 KiB of LDS)
constexpr int kStableSeqBits = 13;     // seq < kStableEntries

int moba_stable_rows_per_wg(int topk) {
  const int km = topk - 1;
  int r = 256;
  while (r * 2 * km <= kStableEntries && r * 2 <= 2048) r *= 2;
  return r;
}

__global__ __launch_bounds__(256) void moba_stable_count_kernel(const int32_t* __restrict__ blk, int32_t nrows,
                                                                MobaRowMap m, int topk, int32_t nbuckets,
                                                                int rows_per_wg, int32_t* __restrict__ counts,
                                                                int32_t* __restrict__ wg_counts) {
  __shared__ int32_t loc[kDispatchLdsBuckets];
  for (int i = threadIdx.x; i < nbuckets; i += blockDim.x) loc[i] = 0;
  __syncthreads();
  const int km = topk - 1;
  const int32_t r0 = blockIdx.x * rows_per_wg;
  const int32_t r1 = min(nrows, r0 + rows_per_wg);
  for (int32_t row = r0 + (int32_t)threadIdx.x; row < r1; row += 256) {
    const MobaRow mr = moba_row(m, (uint32_t)row);
    for (int sl = 0; sl < km; ++sl) {
      const int32_t b = blk[row * topk + sl];
      if (b >= 0 && b < mr.cur) atomicAdd(&loc[mr.bucket0 + b], 1);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nbuckets; i += blockDim.x) {
    if (loc[i]) atomicAdd(&counts[i], loc[i]);
    wg_counts[(int64_t)blockIdx.x * nbuckets + i] = loc[i];
  }
}

// Bitonic sort of 256 * E keys held E per thread (thread t: keys t*E ..
// t*E + E - 1): partners within a thread compare in registers, within a
// wave through lane shuffles, across waves through LDS.
template <int E>
__device__ __forceinline__ void stable_sort_keys(uint32_t (&v)[E], uint32_t* lds) {
  const int tid = threadIdx.x;
  for (int k = 2; k <= 256 * E; k <<= 1) {
    for (int j = k >> 1; j >= E; j >>= 1) {
      const int tj = j / E;   // partner thread: tid ^ tj, same slot
      if (tj >= 64) {
        __syncthreads();
#pragma unroll
        for (int e = 0; e < E; ++e) lds[tid * E + e] = v[e];
        __syncthreads();
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const uint32_t p = tj < 64 ? (uint32_t)__shfl_xor((int)v[e], tj, 64) : lds[(tid ^ tj) * E + e];
        const int i = tid * E + e;
        const bool up = (i & k) == 0, lower = (i & j) == 0;
        v[e] = lower == up ? min(v[e], p) : max(v[e], p);
      }
    }
#pragma unroll
    for (int j = E / 2; j > 0; j >>= 1) {
      if (j >= k) continue;   // uniform
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if ((e & j) == 0) {
          const bool up = ((tid * E + e) & k) == 0;
          const uint32_t x = v[e], y = v[e + j];
          v[e] = up ? min(x, y) : max(x, y);
          v[e + j] = up ? max(x, y) : min(x, y);
        }
      }
    }
  }
}

template <int E>
__global__ __launch_bounds__(256) void moba_stable_scatter_kernel(const int32_t* __restrict__ blk, int32_t nrows,
                                                                  MobaRowMap m, int topk, int32_t nbuckets,
                                                                  int rows_per_wg,
                                                                  const int32_t* __restrict__ wg_base,
                                                                  int2* __restrict__ entries) {
  constexpr int NP = 256 * E;
  __shared__ uint32_t key[NP];
  __shared__ int32_t first[kDispatchLdsBuckets];
  const int km = topk - 1;
  const int32_t r0 = blockIdx.x * rows_per_wg;
  const int32_t r1 = min(nrows, r0 + rows_per_wg);
  const int n = (r1 - r0) * km;   // sequence numbers in use (<= NP)
  uint32_t v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = threadIdx.x * E + e;
    uint32_t kv = 0xffffffffu;   // padding and undispatched slots sort last
    if (i < n) {
      const int32_t row = r0 + i / km;
      const int sl = i % km;
      const MobaRow mr = moba_row(m, (uint32_t)row);
      const int32_t b = blk[row * topk + sl];
      if (b >= 0 && b < mr.cur) kv = ((uint32_t)(mr.bucket0 + b) << kStableSeqBits) | (uint32_t)i;
    }
    v[e] = kv;
  }
  stable_sort_keys<E>(v, key);
  __syncthreads();
#pragma unroll
  for (int e = 0; e < E; ++e) key[threadIdx.x * E + e] = v[e];
  __syncthreads();
  // first sorted index of every bucket present
  for (int i = threadIdx.x; i < NP; i += 256) {
    const uint32_t kv = key[i];
    if (kv != 0xffffffffu && (i == 0 || (key[i - 1] >> kStableSeqBits) != (kv >> kStableSeqBits)))
      first[kv >> kStableSeqBits] = i;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < NP; i += 256) {
    const uint32_t kv = key[i];
    if (kv == 0xffffffffu) continue;
    const int32_t bk = (int32_t)(kv >> kStableSeqBits);
    const int seq = (int)(kv & ((1u << kStableSeqBits) - 1u));
    const int32_t row = r0 + seq / km;
    const int sl = seq % km;
    const MobaRow mr = moba_row(m, (uint32_t)row);
    entries[wg_base[(int64_t)blockIdx.x * nbuckets + bk] + (i - first[bk])] = make_int2(row * 16 + sl, mr.qrow);
  }
}

// Tile table, one thread per tile: the tile's bucket is the last one whose
// first tile is not after it (binary search over the tile prefix, staged in
// LDS when it fits). Tiles of one bucket stay adjacent and in order.
__global__ __launch_bounds__(256) void moba_tiles_kernel(const int32_t* __restrict__ tile_off, int32_t nb,
                                                         const int32_t* __restrict__ offsets, int32_t nbc,
                                                         int32_t hkv, int64_t seq_len, int block, int64_t d,
                                                         int4* __restrict__ tiles) {
  __shared__ int32_t s_off[kDispatchLdsBuckets + 1];
  const int32_t nt = tile_off[nb];
  const int32_t t = blockIdx.x * 256 + threadIdx.x;
  if ((int32_t)(blockIdx.x * 256) >= nt) return;   // uniform per workgroup
  const bool use_lds = nb <= kDispatchLdsBuckets;
  if (use_lds) {
    for (int i = threadIdx.x; i <= nb; i += 256) s_off[i] = tile_off[i];
    __syncthreads();
  }
  if (t >= nt) return;
  const int32_t* off = use_lds ? s_off : tile_off;
  int32_t lo = 0, hi = nb - 1;   // invariant: off[lo] <= t, and off[hi + 1] > t
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if (off[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  const int32_t i = lo, j = t - off[i];
  const int32_t e0 = offsets[i], c = offsets[i + 1] - e0;
  const int64_t b = i % nbc, g = (i / nbc) % hkv, bi = i / (nbc * hkv);
  const int64_t kv = ((bi * seq_len + b * block) * hkv + g) * d;
  tiles[t] = make_int4((int)(uint32_t)kv, (int)(kv >> 32), e0 + j * kRowsPerTile, min(kRowsPerTile, c - j * kRowsPerTile));
}

// (row, slot) -> entries[...] = {row * 16 + slot, index of the row's query
// vector in q (that is (sequence * seq_len + position) * Hq + head)}. Each workgroup reserves one
// range per bucket with a single global atomic and places its entries with
// LDS atomics (the order inside a bucket is irrelevant: every row's result is
// independent of the other rows sharing its tile).
__global__ __launch_bounds__(256) void moba_scatter_kernel(const int32_t* __restrict__ blk, int32_t nrows,
                                                           MobaRowMap m, int topk, int32_t nbuckets,
                                                           const int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ cursor,
                                                           int2* __restrict__ entries,
                                                           const int32_t* __restrict__ wg_loc,
                                                           float* __restrict__ part_lse) {
  __shared__ int32_t loc[kDispatchLdsBuckets];
  __shared__ int32_t base_of[kDispatchLdsBuckets];
  const bool use_lds = nbuckets <= kDispatchLdsBuckets;
  const int32_t r0 = blockIdx.x * (256 * kDispatchRowsPerThread);
  const int32_t r1 = min(nrows, r0 + 256 * kDispatchRowsPerThread);
  if (use_lds) {
    if (wg_loc) {   // this workgroup's start in each bucket, taken by the count pass
      for (int i = threadIdx.x; i < nbuckets; i += blockDim.x) {
        base_of[i] = offsets[i] + wg_loc[(int64_t)blockIdx.x * nbuckets + i];
        loc[i] = 0;
      }
    } else {
      for (int i = threadIdx.x; i < nbuckets; i += blockDim.x) loc[i] = 0;
      __syncthreads();
      moba_for_each_pair(blk, r0, r1, m, topk,
                         [&](int32_t, int, const MobaRow& mr, int32_t b) { atomicAdd(&loc[mr.bucket0 + b], 1); });
      __syncthreads();
      for (int i = threadIdx.x; i < nbuckets; i += blockDim.x) {
        base_of[i] = loc[i] ? atomicAdd(&cursor[i], loc[i]) : 0;
        loc[i] = 0;
      }
    }
    __syncthreads();
  }
  // slots that are not dispatched get no partial: their lse is set to -inf
  // here (part_lse may be NULL), so the current-block pass weights them 0
  const int km = topk - 1;
  moba_for_each_pair(
      blk, r0, r1, m, topk,
      [&](int32_t row, int s, const MobaRow& mr, int32_t b) {
        const int32_t bk = mr.bucket0 + b;
        const int32_t pos = use_lds ? base_of[bk] + atomicAdd(&loc[bk], 1) : atomicAdd(&cursor[bk], 1);
        entries[pos] = make_int2(row * 16 + s, mr.qrow);
      },
      [&](int32_t row, int s) {
        if (part_lse) part_lse[(int64_t)row * km + s] = -__builtin_inff();
      });
}

// Dynamic LDS of the past-block kernels: bf16 staging rows (padded by 8) and
// the output row indices of kNW waves x 32 rows.
template <int D>
constexpr int kPastStageBytes = kNW * 32 * (D + 8) * 2;
template <int D>
constexpr int kPastDynBytes = kPastStageBytes<D> + kNW * 32 * 8;

// Past-block attention: one workgroup per tile of up to 256 dispatched rows
// of one (sequence, KV head, block); full block, no mask. Partials are
// written row-contiguous through LDS. Tiles of one bucket are adjacent in the
// tile table and run on one XCD (shared L2 for the block's K/V).
template <int D, bool FULL>
__global__ __launch_bounds__(kThreads, 8 / kNW) void moba_past_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const int4* __restrict__ tiles, const int32_t* __restrict__ ntiles, const int2* __restrict__ entries,
    bf16* __restrict__ part_o, float* __restrict__ part_lse, int64_t hkv, int block, int topk,
    float scale_log2) {
  QAT_FA_SMEM(D, sm);
  // staging area in dynamic LDS, which is placed after the static tile
  // buffers: those then sit below 64 KiB, where every tile read addresses
  // its buffer through the instruction's immediate offset
  extern __shared__ __align__(16) char s_past_dyn[];
  bf16* s_stage = reinterpret_cast<bf16*>(s_past_dyn);
  int64_t* s_rows = reinterpret_cast<int64_t*>(s_past_dyn + kPastStageBytes<D>);
  const int64_t tile = xcd_logical_id(blockIdx.x, gridDim.x);
  if (tile >= ntiles[0]) return;
  const int4 td = tiles[tile];
  const int64_t kv_off = (int64_t)(uint32_t)td.x | ((int64_t)td.y << 32);
  const int first = td.z;
  const int count = td.w;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int myrow = wave * 32 + (lane & 31);
  const bool valid = myrow < count;
  const int2 e2 = valid ? entries[first + myrow] : make_int2(0, 0);
  const int64_t row = e2.x >> 4;
  const int slot = e2.x & 15;
  const bf16* qrow = q + (int64_t)e2.y * D;

  FaState<D> st;
  fa_init<D>(st, qrow, valid);
  const bf16* kb = k + kv_off;
  const bf16* vb = v + kv_off;
  const int kv_stride = (int)(hkv * D);
  // FULL: block % 64 == 0, so no tile of the block needs masking
  fa_segment<D, kNW, !FULL>(st, sm, kb, vb, block, scale_log2, [=](int j) { return j * kv_stride; },
                            [](int) { return true; }, [](int) { return true; });
  float inv_l, lse;
  fa_finish<D>(st, inv_l, lse);
  const int64_t pidx = row * (topk - 1) + slot;
  if ((lane >> 5) == 0 && valid) __builtin_nontemporal_store(lse, part_lse + pidx);
  fa_store_rows_staged<D>(st, inv_l, s_stage + wave * 32 * (D + 8), s_rows + wave * 32, valid ? pidx : -1, part_o);
}

// Persistent form of the past-block kernel for blocks of a multiple of 128
// keys: a fixed grid of workgroups walks the tile table with stride G (the
// G concurrently processed tiles stay consecutive, so the ones sharing a
// block's K/V share an XCD's L2), and each workgroup overlaps the end of one
// tile with the start of the next: once the last K tile has been scored, the
// next tile's first K/V tiles and its query rows are loaded while the last
// softmax, PV and the partial's store (straight from the accumulators) run.
template <int D>
__global__ __launch_bounds__(kThreads, 8 / kNW) void moba_past_persist_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const int4* __restrict__ tiles, const int32_t* __restrict__ ntiles, const int2* __restrict__ entries,
    bf16* __restrict__ part_o, float* __restrict__ part_lse, int64_t hkv, int block, int topk,
    float scale_log2) {
  QAT_FA_SMEM(D, sm);
  // staging area in dynamic LDS, which is placed after the static tile
  // buffers: those then sit below 64 KiB, where every tile read addresses
  // its buffer through the instruction's immediate offset
  extern __shared__ __align__(16) char s_past_dyn[];
  bf16* s_stage = reinterpret_cast<bf16*>(s_past_dyn);
  int64_t* s_rows = reinterpret_cast<int64_t*>(s_past_dyn + kPastStageBytes<D>);
  const int n_items = ntiles[0];
  const int G = gridDim.x;
  int item = (int)xcd_logical_id(blockIdx.x, G);
  if (item >= n_items) return;
  const int lane = threadIdx.x & 63;
  const int myrow = (threadIdx.x >> 6) * 32 + (lane & 31);
  const int km = topk - 1;
  const int kv_stride = (int)(hkv * D);
  const int nt = block / kKT;   // even
  // whole tiles only (block % 128 == 0): per-lane load offsets fixed; one
  // block's K (or V) rows span (block - 1) * stride + D elements
  FaContig<D, kNW> ctg;
  ctg.init(kv_stride);
  const uint32_t region = (uint32_t)(((int64_t)(block - 1) * kv_stride + D) * 2);
  auto issue = [&](bf16* dst, const bf16* src, int j0) { ctg.issue(dst, fa_rsrc(src, region), j0, kv_stride); };

  // Descriptors run one tile ahead of use, loaded by plain vector loads that
  // the per-tile waits cover: at the top of tile i its own entry and the
  // next tile's descriptor are resident; the next tile's entry and the
  // descriptor after it are then requested.
  struct Tile {
    int64_t kv;   // element offset of the block's K/V rows
    int first, count;
  };
  struct Entry {
    int32_t rs;   // row * 16 + slot, -1 for a padding lane
    int32_t qrow;
  };
  auto tile_at = [=](int it) {
    const int4 t = tiles[it];
    return Tile{(int64_t)(uint32_t)t.x | ((int64_t)t.y << 32), t.z, t.w};
  };
  // loaded unconditionally (a padding lane re-reads the tile's first entry)
  // so that nothing waits for it until its first use
  auto entry_of = [=](Tile t) {
    const int2 x = entries[t.first + (myrow < t.count ? myrow : 0)];
    return Entry{myrow < t.count ? x.x : -1, x.y};
  };
  auto load_q = [=](FaState<D>& st, Entry e) {
    const bf16* qr = q + (int64_t)e.qrow * D;
    const int hh = lane >> 5;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      if (e.rs >= 0) {
        st.q[c] = *(const bf16x8*)(qr + 16 * c + 8 * hh);
      } else {
        const u32x4 z = {0u, 0u, 0u, 0u};
        st.q[c] = __builtin_bit_cast(bf16x8, z);
      }
    }
  };

  // The item loop exists twice, one copy per issue order (the copies hit
  // the same barriers in the same sequence); each wave runs one of them.
  auto run = [&](auto late_c) {
    constexpr bool kLate = decltype(late_c)::value;
    Tile t_cur = tile_at(item);
    Entry e_cur = entry_of(t_cur);
    Tile t_nxt = tile_at(item + G < n_items ? item + G : item);
    FaState<D> st;
    fa_init<D>(st, q, false);
    load_q(st, e_cur);
    {
      const int64_t kv = t_cur.kv;
      issue(sm.k0, k + kv, 0);
      issue(sm.k1, k + kv, kKT);
      issue(sm.v0, v + kv, 0);
      issue(sm.v1, v + kv, kKT);
    }
    // load instructions of one tile per wave: the waits below leave that many
    // (the most recent tile) in flight
    constexpr int kNI = FaContig<D, kNW>::NI;
    auto ok = [](int) { return true; };
    // A tile's partial output is written at the top of the next tile, once
    // that tile's first K/V and query rows have been waited for: writes are
    // never waited on by the wait that guards those loads.
    auto epilogue = [&](const Entry& e) {
      float inv_l, lse;
      fa_finish<D>(st, inv_l, lse);
      const bool mine = e.rs >= 0;
      const int64_t pidx = mine ? (int64_t)(e.rs >> 4) * km + (e.rs & 15) : 0;
      if ((lane >> 5) == 0 && mine) __builtin_nontemporal_store(lse, part_lse + pidx);
      const int wv = threadIdx.x >> 6;
      fa_store_rows_staged<D>(st, inv_l, s_stage + wv * 32 * (D + 8), s_rows + wv * 32, mine ? pidx : -1, part_o);
  #pragma unroll
      for (int t = 0; t < D / 32; ++t)
  #pragma unroll
        for (int i = 0; i < 16; ++i) st.o[t][i] = 0.f;
      st.m = -__builtin_inff();
      st.l = 0.f;
    };
    // Per tile: the scores of the next tile (matrix cores) and the softmax of
    // this one (vector ALUs) are independent; the two waves that share a SIMD
    // (waves w and w + kNW/2) issue them in opposite orders, so that one
    // wave's matrix ops run under the other's vector work; then O += P V.
    auto step = [&](const bf16* ks_next, f32x16* s_next, f32x16* s_now, const bf16* vs) {
      u32x4 pw[4];
      if constexpr (kLate) {
        fa_softmax<D, false>(st, s_now, pw, scale_log2);
        fa_scores<D>(st, ks_next, s_next);
      } else {
        fa_scores<D>(st, ks_next, s_next);
        fa_softmax<D, false>(st, s_now, pw, scale_log2);
      }
      fa_pv<D>(st, vs, pw);
    };
    bool pending = false;
    Entry e_prev = e_cur;
    while (true) {
      const int nxt_item = item + G;
      const bool has_next = nxt_item < n_items;
      const int64_t kv = t_cur.kv;
      const bf16* kb = k + kv;
      const bf16* vb = v + kv;
      // the query rows, K0, K1, V0 and (last) V1 are in flight: V1 is not
      // needed before the first pair and stays in flight
      fa_wait_loads_keep<kNI>();
      fa_lds_barrier();
      if (pending) epilogue(e_prev);
      // the next tile's descriptors, first used at this tile's last pair (no
      // select on the loaded values: that would wait for them right here; when
      // there is no next tile, t_nxt repeats the current one and e_nxt is unused)
      const Entry e_nxt = entry_of(t_nxt);
      const Tile t_nn = tile_at(nxt_item + G < n_items ? nxt_item + G : item);
      f32x16 s_cur[2], s_nxt[2];
      fa_scores<D>(st, sm.k0, s_cur);
      fa_lds_barrier();
      const int64_t kv_n = t_nxt.kv;
      // K0 of the next tile goes into buffer k0 as soon as the buffer is free,
      // after every load that this tile still waits for
      if (nt > 2) {
        issue(sm.k0, kb, 2 * kKT);
        int j = 0;
        do {   // at least one pair (a do loop, so the waits in it cover every path to the last pair)
          step(sm.k1, s_nxt, s_cur, sm.v0);
          fa_wait_loads();
          fa_lds_barrier();
          issue(sm.k1, kb, (j + 3) * kKT);
          issue(sm.v0, vb, (j + 2) * kKT);
          step(sm.k0, s_cur, s_nxt, sm.v1);
          fa_wait_loads();
          fa_lds_barrier();
          issue(sm.v1, vb, (j + 3) * kKT);
          if (j + 4 < nt) issue(sm.k0, kb, (j + 4) * kKT);
          else if (has_next) issue(sm.k0, k + kv_n, 0);
          j += 2;
        } while (j + 2 < nt);
      } else {
        // no pair loop: everything this tile still needs (V1, the
        // descriptors) is waited for here, so that only K0 of the next tile
        // is in flight where the paths join
        fa_wait_loads();
        if (has_next) issue(sm.k0, k + kv_n, 0);
      }
      // last pair: tiles nt-2 (V in v0) and nt-1 (K in k1, V in v1)
      step(sm.k1, s_nxt, s_cur, sm.v0);
      if (has_next) fa_wait_loads_keep<kNI>();   // the next tile's K0 (issued last) stays in flight
      else fa_wait_loads();
      fa_lds_barrier();
      // every K tile is scored and V_{nt-2} consumed: k1, v0 and the query
      // registers are free for the next tile
      if (has_next) {
        issue(sm.k1, k + kv_n, kKT);
        issue(sm.v0, v + kv_n, 0);
        load_q(st, e_nxt);
      }
      fa_finish_tile<D, false>(st, s_nxt, sm.v1, scale_log2, (nt - 1) * kKT, block, ok, ok);
      if (!has_next) {
        epilogue(e_cur);
        break;
      }
      fa_lds_barrier();   // every wave is done with V_{nt-1}
      issue(sm.v1, v + kv_n, kKT);
      pending = true;
      e_prev = e_cur;
      t_cur = t_nxt;
      e_cur = e_nxt;
      t_nxt = t_nn;
      item = nxt_item;
    }
  };
  if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) >= kNW / 2) run(std::true_type{});
  else run(std::false_type{});
}

// Current-block attention (causal) merged with the row's past-block
// partials: the partials seed the online-softmax state (running max, sum and
// accumulator), so the merge costs no pass of its own and its loads overlap
// the first K/V tiles. A workgroup holds 32*NW rows = 32*NW/P consecutive
// tokens x P query heads of one KV group (GQA packing: the heads share K/V).
// Logical id -> (token tile, block, sequence, KV head, head pack).
constexpr int kCurNW = 4;
constexpr int kCurRows = 32 * kCurNW;
constexpr int kPreSlots = 2;   // past partials loaded ahead of the tiles (more: folded in one by one)

template <int D>
__global__ __launch_bounds__(64 * kCurNW, 2) void moba_current_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const int32_t* __restrict__ blk, const bf16* __restrict__ part_o, const float* __restrict__ part_lse,
    bf16* __restrict__ out, float* __restrict__ lse_out, int64_t seq_len, int64_t hq, int64_t hkv,
    int64_t q_start, int64_t q_len, int block, int topk, float scale_log2, int pack, int tiles_per_block,
    int64_t nblocks) {
  constexpr int NW = kCurNW;
  constexpr int THREADS = 64 * NW;
  QAT_FA_SMEM(D, sm);
  int64_t id = xcd_logical_id(blockIdx.x, gridDim.x);
  // a block's last token tiles attend the most keys: they are dispatched
  // first, so the launch ends on short tiles
  const int tt = tiles_per_block - 1 - (int)(id % tiles_per_block);
  id /= tiles_per_block;
  const int64_t cb = id % nblocks;
  id /= nblocks;
  const int64_t gs = hq / hkv;
  const int64_t npk = gs / pack;
  const int64_t hp = id % npk;
  id /= npk;
  const int64_t g = id % hkv;
  const int64_t bi = id / hkv;
  const int64_t c = q_start / block + cb;
  const int64_t q_end = q_start + q_len;
  const int64_t lo = max(c * block, q_start);
  const int64_t hi = min((c + 1) * block, q_end);
  const int tok_per_tile = kCurRows / pack;
  const int64_t t0 = lo + (int64_t)tt * tok_per_tile;
  if (t0 >= hi) return;
  const int64_t t_last = min(hi, t0 + tok_per_tile) - 1;
  const int64_t h0 = g * gs + hp * pack;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hl = lane >> 5;
  const int myrow = wave * 32 + (lane & 31);
  const int64_t t = t0 + myrow / pack;
  const int64_t h = h0 + myrow % pack;
  const bool valid = t <= t_last;
  const int64_t row = (bi * q_len + ((valid ? t : t0) - q_start)) * hq + h;
  const int km = topk - 1;

  const int64_t kpos0 = c * block;
  const bf16* kb = k + ((bi * seq_len + kpos0) * hkv + g) * D;
  const bf16* vb = v + ((bi * seq_len + kpos0) * hkv + g) * D;
  const int kv_stride = (int)(hkv * D);
  const int nkeys = (int)(t_last - kpos0 + 1);
  // The block's rows [kpos0, t_last] through buffer resources: fixed
  // per-lane offsets, the tile's start added to the range-checked vector
  // offset, so rows of the last tile past t_last read as zero (their scores
  // are masked) and nothing past the region is touched.
  FaContig<D, NW> ctg;
  ctg.init(kv_stride);
  const uint32_t region = (uint32_t)(((int64_t)(nkeys - 1) * kv_stride + D) * 2);
  const __amdgpu_buffer_rsrc_t rk = fa_rsrc(kb, region), rv = fa_rsrc(vb, region);
  auto issue = [&](bf16* dst, bool is_v, int tile) { ctg.issue_checked(dst, is_v ? rv : rk, tile * kKT, kv_stride); };
  fa_segment_begin_tiles<D>(sm, nkeys, issue);

  FaState<D> st;
  fa_init<D>(st, q + ((bi * seq_len + (valid ? t : t0)) * hq + h) * D, valid);
  // Seed the online softmax with the row's past-block partials (normalised o
  // in bf16, natural-log lse): m = max lse in log2 units, l = sum of
  // 2^(lse - m) (kept by the lower half-wave only: l is summed over the two
  // halves at the end), o = sum of 2^(lse - m) o_p. The lane's accumulator
  // holds d = 32 tq + 8 gi + 4 hl + 0..3. These loads are younger than the
  // tiles', so waiting for them costs no extra latency. Every (row, slot)
  // partial lse is -inf unless the slot's block was dispatched (the
  // dispatch's scatter writes -inf for the slots it leaves out), so the
  // loads need no look at the gating; the o rows of such slots were never written (whatever the
  // workspace held, NaN included) and are replaced by zeros as they load.
  auto unpack = [](const uint2 u, float* f) {
    f[0] = __builtin_bit_cast(float, u.x << 16);
    f[1] = __builtin_bit_cast(float, u.x & 0xffff0000u);
    f[2] = __builtin_bit_cast(float, u.y << 16);
    f[3] = __builtin_bit_cast(float, u.y & 0xffff0000u);
  };
  auto load_slots = [&](int s0, float* plse, uint2 (*po)[D / 8]) {
#pragma unroll
    for (int sl = 0; sl < kPreSlots; ++sl) {
      const int64_t pidx = row * km + min(s0 + sl, km - 1);
      const float lv = part_lse[pidx];
      plse[sl] = (valid && s0 + sl < km) ? lv * kLog2e : -__builtin_inff();
      const bool live = plse[sl] != -__builtin_inff();
      // partial rows are stored in split halves: this lane's D/2 values are
      // contiguous, in accumulator order
      const bf16* src = part_o + pidx * D + hl * (D / 2);
#pragma unroll
      for (int i = 0; i < D / 16; ++i) {
        const u32x4 w = *(const u32x4*)(src + 8 * i);
        po[sl][2 * i] = live ? make_uint2(w[0], w[1]) : make_uint2(0u, 0u);
        po[sl][2 * i + 1] = live ? make_uint2(w[2], w[3]) : make_uint2(0u, 0u);
      }
    }
  };
  if (km > 0) {   // topk = 1: no past slots, nothing to load
    // first round: the state is empty, so o = sum_s w_s o_s under one max
    // (no rescale of a zero accumulator)
    float plse[kPreSlots];
    uint2 po[kPreSlots][D / 8];
    load_slots(0, plse, po);
    float mx = plse[0];
#pragma unroll
    for (int sl = 1; sl < kPreSlots; ++sl) mx = fmaxf(mx, plse[sl]);
    const float base = mx == -__builtin_inff() ? 0.f : mx;   // all empty: every weight 0
    float w[kPreSlots], wsum = 0.f;
#pragma unroll
    for (int sl = 0; sl < kPreSlots; ++sl) {
      w[sl] = __builtin_amdgcn_exp2f(plse[sl] - base);
      wsum += w[sl];
    }
    st.m = mx;
    st.l = hl == 0 ? wsum : 0.f;
#pragma unroll
    for (int tq = 0; tq < D / 32; ++tq)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        float f[4];
        unpack(po[0][tq * 4 + gi], f);
#pragma unroll
        for (int e = 0; e < 4; ++e) st.o[tq][4 * gi + e] = w[0] * f[e];
#pragma unroll
        for (int sl = 1; sl < kPreSlots; ++sl) {
          unpack(po[sl][tq * 4 + gi], f);
#pragma unroll
          for (int e = 0; e < 4; ++e) st.o[tq][4 * gi + e] = __builtin_fmaf(w[sl], f[e], st.o[tq][4 * gi + e]);
        }
      }
  }
  // later rounds (k > kPreSlots + 1): folded into the running state
  for (int s0 = kPreSlots; s0 < km; s0 += kPreSlots) {
    float plse[kPreSlots];
    uint2 po[kPreSlots][D / 8];
    load_slots(s0, plse, po);
#pragma unroll
    for (int sl = 0; sl < kPreSlots; ++sl) {
      if (plse[sl] == -__builtin_inff()) continue;
      const float m_new = fmaxf(st.m, plse[sl]);
      const float a = st.m == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(st.m - m_new);
      const float wt = __builtin_amdgcn_exp2f(plse[sl] - m_new);
      st.l = st.l * a + (hl == 0 ? wt : 0.f);
#pragma unroll
      for (int tq = 0; tq < D / 32; ++tq)
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          float f[4];
          unpack(po[sl][tq * 4 + gi], f);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            st.o[tq][4 * gi + e] = __builtin_fmaf(wt, f[e], st.o[tq][4 * gi + e] * a);
        }
      st.m = m_new;
    }
  }

  // keys are block-relative: this lane attends keys j <= lim, and every lane
  // of the wave attends keys j <= wlim
  const int lim = valid ? (int)(t - kpos0) : -1;
  const int wlim = (int)(t0 - kpos0) + (wave * 32) / pack;
  fa_segment_run_tiles<D, true>(st, sm, nkeys, scale_log2, issue, [=](int j) { return j <= lim; },
                                [=](int j0) { return j0 + kKT - 1 <= wlim; });
  float inv_l, lse;
  fa_finish<D>(st, inv_l, lse);
  if (lse_out && valid && hl == 0) lse_out[row] = lse;
  fa_rows_to_lds<D>(st, sm, inv_l, 0);
  __syncthreads();
  constexpr int TPR = D / 8;
  constexpr int RPP = THREADS / TPR;
  const int sub = threadIdx.x % TPR;
  const int nrows = (int)(t_last - t0 + 1) * pack;
  for (int rr = threadIdx.x / TPR; rr < nrows; rr += RPP) {
    const int64_t orow = (bi * q_len + (t0 + rr / pack - q_start)) * hq + h0 + rr % pack;
    const f32x4 a = fa_row_chunk<D>(sm, rr, 2 * sub), cc = fa_row_chunk<D>(sm, rr, 2 * sub + 1);
    u32x4 w;
    w[0] = pack_bf16x2(a[0], a[1]);
    w[1] = pack_bf16x2(a[2], a[3]);
    w[2] = pack_bf16x2(cc[0], cc[1]);
    w[3] = pack_bf16x2(cc[2], cc[3]);
    // non-temporal: nothing in this pass reads out again, and a cached copy
    // would leave dirty lines whose write-back slows the next kernel's reads
    __builtin_nontemporal_store(w, (u32x4*)(out + orow * D + sub * 8));
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

int moba_rows_per_tile() { return kRowsPerTile; }

int64_t moba_max_tiles(int64_t nrows, int topk, int64_t nbuckets) {
  return cdiv(nrows * (topk - 1), kRowsPerTile) + nbuckets;
}

int64_t moba_dispatch_wg_ints(int64_t nrows, int64_t nbuckets) {
  if (nbuckets > kDispatchLdsBuckets) return 0;
  return cdiv(nrows, 256 * kDispatchRowsPerThread) * nbuckets;
}

int64_t moba_dispatch_stable_ints(int64_t nrows, int64_t nbuckets, int topk) {
  // bucket ids and sequence numbers share a 32-bit sort key
  if (nbuckets > kDispatchLdsBuckets || topk < 2 || topk - 1 > 16) return 0;
  return cdiv(nrows, moba_stable_rows_per_wg(topk)) * nbuckets;
}

hipError_t launch_moba_dispatch(const int32_t* blk, int64_t batch, int64_t seq_len, int64_t hq, int64_t hkv,
                                int64_t d, int64_t q_start, int64_t q_len, int block, int topk, int64_t nbc,
                                int32_t* counts, int32_t* offsets, int32_t* cursor, int2* entries, int4* tiles,
                                int32_t* ntiles, hipStream_t s, int32_t* wg_counts, int32_t* wg_base,
                                int32_t* wg_loc, float* part_lse) {
  const int64_t nrows = batch * q_len * hq;
  const int64_t nbuckets = batch * hkv * nbc;
  const bool stable = wg_counts && wg_base && moba_dispatch_stable_ints(nrows, nbuckets, topk) > 0;
  const int srows = moba_stable_rows_per_wg(topk);
  const unsigned sgrid = (unsigned)cdiv(nrows, srows);
  const MobaRowMap m{(uint32_t)hq, (uint32_t)q_len, (uint32_t)q_start, (uint32_t)block, (uint32_t)(hq / hkv),
                     (uint32_t)hkv, (uint32_t)nbc, (uint32_t)seq_len};
  hipError_t e = launch_fill_i32(counts, nbuckets, 0, s);
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)cdiv(nrows, 256 * kDispatchRowsPerThread);
  if (nbuckets > 0) {
    if (stable)
      hipLaunchKernelGGL(moba_stable_count_kernel, dim3(sgrid), dim3(256), 0, s, blk, (int32_t)nrows, m, topk,
                         (int32_t)nbuckets, srows, counts, wg_counts);
    else
      hipLaunchKernelGGL(moba_count_kernel, dim3(grid), dim3(256), 0, s, blk, (int32_t)nrows, m, topk,
                         (int32_t)nbuckets, counts, nbuckets <= kDispatchLdsBuckets ? wg_loc : nullptr);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(moba_scan_kernel, dim3(1), dim3(1024), 0, s, counts, (int32_t)nbuckets, offsets, cursor,
                     ntiles);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (stable && nbuckets > 0) {
    hipLaunchKernelGGL(moba_wg_scan_kernel, dim3((unsigned)cdiv(nbuckets, 64)), dim3(64 * kScanParts), 0, s,
                       (const int32_t*)wg_counts, (int32_t)sgrid, (int32_t)nbuckets, (const int32_t*)offsets,
                       wg_base);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (nbuckets > 0) {
    const int64_t max_tiles = moba_max_tiles(nrows, topk, nbuckets);
    hipLaunchKernelGGL(moba_tiles_kernel, dim3((unsigned)cdiv(max_tiles, 256)), dim3(256), 0, s, counts,
                       (int32_t)nbuckets, offsets, (int32_t)nbc, (int32_t)hkv, seq_len, block, d, tiles);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (stable) {
      // sort width: the workgroup's sequence numbers rounded up to a power of two
      int np = 256;
      while (np < srows * (topk - 1)) np <<= 1;
#define QAT_STS(E_)                                                                                         \
  hipLaunchKernelGGL(moba_stable_scatter_kernel<E_>, dim3(sgrid), dim3(256), 0, s, blk, (int32_t)nrows, m, \
                     topk, (int32_t)nbuckets, srows, (const int32_t*)wg_base, entries)
      if (np <= 256) QAT_STS(1);
      else if (np <= 512) QAT_STS(2);
      else if (np <= 1024) QAT_STS(4);
      else if (np <= 2048) QAT_STS(8);
      else if (np <= 4096) QAT_STS(16);
      else QAT_STS(32);
#undef QAT_STS
    } else
      hipLaunchKernelGGL(moba_scatter_kernel, dim3(grid), dim3(256), 0, s, blk, (int32_t)nrows, m, topk,
                         (int32_t)nbuckets, (const int32_t*)offsets, cursor, entries,
                         (const int32_t*)(nbuckets <= kDispatchLdsBuckets ? wg_loc : nullptr), part_lse);
    e = hipGetLastError();
  }
  return e;
}

template <int D>
static hipError_t launch_moba_attn_d(const bf16* q, const bf16* k, const bf16* v, const int32_t* blk,
                                     const int4* tiles, const int32_t* ntiles, const int2* entries, bf16* part_o,
                                     float* part_lse, bf16* out, float* lse, int64_t batch, int64_t seq_len,
                                     int64_t hq, int64_t hkv, int64_t nbc, int64_t q_start, int64_t q_len, int block,
                                     int topk, float scale, int64_t max_tiles, hipStream_t s) {
  const float sl2 = scale * kLog2e;
  hipError_t e;
  // dynamic LDS beyond 64 KiB is declared once per kernel
  static const bool lds_ok = [] {
    bool ok = hipFuncSetAttribute((const void*)moba_past_persist_kernel<D>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, kPastDynBytes<D>) == hipSuccess;
    ok &= hipFuncSetAttribute((const void*)moba_past_kernel<D, true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              kPastDynBytes<D>) == hipSuccess;
    ok &= hipFuncSetAttribute((const void*)moba_past_kernel<D, false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              kPastDynBytes<D>) == hipSuccess;
    return ok;
  }();
  if (!lds_ok) return hipErrorInvalidConfiguration;
  // past partials exist only if the past-block pass runs (no complete block
  // before the rows: none is written, and the current-block pass must fold
  // none)
  const bool past = topk > 1 && max_tiles > 0 && nbc > 0;
  if (past) {
    {
      KTimer tm("moba_past_attn", s);
      // every (row, slot) lse is written before the current-block pass reads
      // it without consulting the gating: by this pass for the dispatched
      // slots, as -inf by the dispatch's scatter for the others
      if (block % (2 * kKT) == 0 && (int64_t)block * hkv * D * 2 < (1ll << 31)) {
        // persistent grid: the workgroups that fit at once (256 CUs x 8 waves), never more than the tiles
        const int64_t grid = std::min<int64_t>(max_tiles, 2048 / kNW);
        launch_timed("moba_past_attn", moba_past_persist_kernel<D>, dim3((unsigned)grid), dim3(kThreads),
                     kPastDynBytes<D>, s, q, k, v, tiles, ntiles, entries, part_o, part_lse, hkv, block, topk, sl2);
      } else if (block % kKT == 0) {
        launch_timed("moba_past_attn", moba_past_kernel<D, true>, dim3((unsigned)max_tiles), dim3(kThreads),
                     kPastDynBytes<D>, s, q, k, v, tiles, ntiles, entries, part_o, part_lse, hkv, block, topk, sl2);
      } else {
        launch_timed("moba_past_attn", moba_past_kernel<D, false>, dim3((unsigned)max_tiles), dim3(kThreads),
                     kPastDynBytes<D>, s, q, k, v, tiles, ntiles, entries, part_o, part_lse, hkv, block, topk, sl2);
      }
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int64_t gs = hq / hkv;
  const int pack = (kCurRows % gs == 0) ? (int)gs : 1;
  const int tok_per_tile = kCurRows / pack;
  const int tiles_per_block = (int)cdiv(block, tok_per_tile);
  const int64_t c_first = q_start / block;
  const int64_t nblocks = (q_start + q_len - 1) / block - c_first + 1;
  const int64_t nwg = (int64_t)tiles_per_block * nblocks * batch * hkv * (gs / pack);
  {
    KTimer tm("moba_current_attn", s);
    launch_timed("moba_current_attn", moba_current_kernel<D>, dim3((unsigned)nwg), dim3(64 * kCurNW), 0, s, q, k,
                 v, blk, (const bf16*)part_o, (const float*)part_lse, out, lse, seq_len, hq, hkv, q_start, q_len,
                 block, past ? topk : 1, sl2, pack, tiles_per_block, nblocks);
  }
  return hipGetLastError();
}

hipError_t launch_moba_attn_mfma(const void* q, const void* k, const void* v, const int32_t* blk,
                                 const int4* tiles, const int32_t* ntiles, const int2* entries, void* part_o,
                                 float* part_lse, void* out, float* lse, int64_t batch, int64_t seq_len, int64_t hq,
                                 int64_t hkv, int64_t d, int64_t nbc, int64_t q_start, int64_t q_len, int block,
                                 int topk, float scale, int64_t max_tiles, hipStream_t s) {
  if (d == 64)
    return launch_moba_attn_d<64>((const bf16*)q, (const bf16*)k, (const bf16*)v, blk, tiles, ntiles, entries,
                                  (bf16*)part_o, part_lse, (bf16*)out, lse, batch, seq_len, hq, hkv, nbc, q_start,
                                  q_len, block, topk, scale, max_tiles, s);
  return launch_moba_attn_d<128>((const bf16*)q, (const bf16*)k, (const bf16*)v, blk, tiles, ntiles, entries,
                                 (bf16*)part_o, part_lse, (bf16*)out, lse, batch, seq_len, hq, hkv, nbc, q_start,
                                 q_len, block, topk, scale, max_tiles, s);
}

}  // namespace qat
