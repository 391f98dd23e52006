// Flash-style exact softmax attention tile engine on the bf16 matrix cores
// (v_mfma_f32_32x32x16_bf16), shared by the MoBA and ESA attention kernels.
//
// Exact attention over an explicit key set is the standard definition
// (MoBA write-up, sections 1-2: Softmax(q K[I]^T) V[I]); the key set is fed
// as segments (a contiguous range or a gathered index list, optionally
// causal), processed 64 keys at a time with an online softmax, so the
// result equals one joint softmax over the union of the segments (the
// fusion of the ESA write-up and the CCA write-up's unified K/V).
//
// Layout (one workgroup = NW waves = 32*NW query rows; one wave = 32 rows):
// the wave computes S^T = K Q^T (A = K tile from LDS, B = Q from
// registers) so that each lane owns ONE query (lane % 32) and 16 key
// scores per 32-key subtile; row max / row sum are lane-local plus one
// exchange with lane ^ 32. Then O^T += V^T P^T (A = V^T, B = P from
// registers). The probabilities a lane holds for a 16-key chunk are the
// keys 16kc + 8(j/4) + 4h + j%4 (j = 0..7, h = lane / 32); V stays row-major
// in LDS and the matching V^T operand is fetched with two transposing LDS
// reads (ds_read_b64_tr_b16), each giving a lane 4 keys of one d column.
//
// K/V tiles go from global memory straight into LDS (global_load_lds, 16
// bytes per lane, no staging registers); rows are unpadded and the 16-byte
// chunks of row r are stored at chunk ^ swz(r), which spreads both the
// K-operand reads and the transposing V reads over all LDS banks.
#pragma once

#include "common.h"

namespace qat {

constexpr int kKT = 64;          // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.f;   // log2 units a stale running max may lag

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void global_void;

// The four LDS tile buffers (K and V, double-buffered) are separate
// __shared__ variables so that alias analysis can see that reads of one
// buffer never depend on the in-flight direct loads into the other; with a
// single array the compiler would wait for those loads before every read.
template <int D>
struct FaSmem {
  bf16* k0;
  bf16* v0;
  bf16* k1;
  bf16* v1;
};

#define QAT_FA_SMEM(D, name)                                         \
  __shared__ __align__(16) qat::bf16 name##_k0[qat::kKT * (D)];      \
  __shared__ __align__(16) qat::bf16 name##_v0[qat::kKT * (D)];      \
  __shared__ __align__(16) qat::bf16 name##_k1[qat::kKT * (D)];      \
  __shared__ __align__(16) qat::bf16 name##_v1[qat::kKT * (D)];      \
  qat::FaSmem<D> name{name##_k0, name##_v0, name##_k1, name##_v1}

// Chunk swizzle of row r. D = 128 (16 chunks per 256-byte row = all 64
// banks): swz swaps the two 2-bit halves of r & 15, so (a) rows r & 15 =
// 0..15 read at one chunk index land on 16 distinct chunks (K-operand
// reads), and (b) the 4 consecutive rows 4a..4a+3 read by one transposing
// group get distinct bits 2-3, so their chunks 4t..4t+3 never collide.
template <int D>
__device__ __forceinline__ int fa_swz(int r) {
  if (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  return (((r & 3) << 1) | ((r >> 2) & 1)) & (D / 8 - 1);
}

template <int D>
struct FaState {
  f32x16 o[D / 32];   // O^T: lane's query (lane%32), d = 32*t + 8*(i/4) + 4*(lane/32) + i%4
  bf16x8 q[D / 16];   // B operand of S^T: q[row][16c + 8*(lane/32) .. +8]
  float m;            // running max of scaled scores, log2 units (may lag by kRescaleSlack)
  float l;            // lane-partial running sum (combine with lane^32 at the end)
  int kofs[D / 16];   // LDS byte offsets of this lane's K-operand reads
  int vofs[D / 32][2];   // LDS byte offsets of this lane's transposing V reads
};

template <int D>
__device__ __forceinline__ void fa_init(FaState<D>& st, const bf16* qrow, bool valid) {
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5, r32 = lane & 31;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    if (valid) {
      st.q[c] = *(const bf16x8*)(qrow + 16 * c + 8 * h);
    } else {
      const u32x4 z = {0u, 0u, 0u, 0u};
      st.q[c] = __builtin_bit_cast(bf16x8, z);
    }
  }
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) st.o[t][i] = 0.f;
  st.m = -__builtin_inff();
  st.l = 0.f;
  constexpr int RB = D * 2;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) st.kofs[c] = r32 * RB + 16 * ((2 * c + h) ^ fa_swz<D>(r32));
  const int i16 = lane & 15, dh = (lane >> 4) & 1;
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int row = 4 * h + (i16 >> 2) + 8 * hi;
      const int chunk = 4 * t + 2 * dh + ((i16 & 3) >> 1);
      st.vofs[t][hi] = row * RB + 16 * (chunk ^ fa_swz<D>(row)) + 8 * (i16 & 1);
    }
}

// The lane id as a value the compiler cannot hoist out of a loop: address
// terms derived from it are recomputed where a load is issued (a few vector
// ops per tile) instead of being held in registers, or spilled, across a
// whole tile loop. For kernels at the register limit.
__device__ __forceinline__ int fa_fresh_lane() {
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  return t & 63;
}

// Issue the direct-to-LDS loads of one 64-key tile of K or V for the calling
// wave: wave w of NW fills rows [w*64/NW, (w+1)*64/NW). row_ofs(j) gives key
// j's element offset from src (32-bit: one sequence's K or V holds fewer
// than 2^31 elements); rows at or beyond n are clamped to row n - 1 (a valid
// row whose scores the caller masks).
template <int D, int NW, typename RowOfs, bool CLAMP = true, bool FRESH = false>
__device__ __forceinline__ void fa_issue_one(bf16* __restrict__ dst, const bf16* __restrict__ src, int j0, int n,
                                             RowOfs row_ofs) {
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;       // rows per wave instruction
  constexpr int RPW = kKT / NW;       // rows per wave
  static_assert(RPW % RPI == 0, "tile rows must split evenly over the waves");
  const int lane = FRESH ? fa_fresh_lane() : (int)(threadIdx.x & 63);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int i = 0; i < RPW / RPI; ++i) {
    const int r0 = RPW * wave + i * RPI;
    const int r = r0 + lane / CPR;
    const int c = (lane % CPR) ^ fa_swz<D>(r);
    const int j = j0 + r;
    const int off = row_ofs(CLAMP ? (j < n ? j : n - 1) : j) + c * 8;
    __builtin_amdgcn_global_load_lds((const global_void*)(src + off), (lds_void*)(dst + r0 * D), 16, 0, 0);
  }
}

// Contiguous rows at a fixed element stride, whole tiles, through a buffer
// resource: the lane's byte offset inside a tile (row times stride plus its
// swizzled 16-byte chunk) is fixed, the tile's start goes in the scalar
// offset, so a load costs no vector instruction and no 64-bit address
// registers. The resource's record count bounds every access to the region
// it describes (out-of-range reads return zero).
constexpr uint32_t kBufWord3 = 0x00020000u;   // raw buffer, gfx9-family format

template <int D, int NW>
struct FaContig {
  static constexpr int CPR = D / 8;
  static constexpr int RPI = 64 / CPR;
  static constexpr int RPW = kKT / NW;
  static constexpr int NI = RPW / RPI;   // load instructions per wave per tile
  int off[NI];                           // bytes
  __device__ __forceinline__ void init(int stride) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = RPW * wave + i * RPI + lane / CPR;
      off[i] = (r * stride + ((lane % CPR) ^ fa_swz<D>(r)) * 8) * 2;
    }
  }
  // issue_checked with the per-lane offsets recomputed from fa_fresh_lane()
  // (for kernels at the register limit: nothing held across the tile loop)
  __device__ __forceinline__ static void issue_checked_fresh(bf16* __restrict__ dst, __amdgpu_buffer_rsrc_t rsrc,
                                                             int j0, int stride) {
    const int lane = fa_fresh_lane();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int base = j0 * stride * 2;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = RPW * wave + i * RPI + lane / CPR;
      const int o = (r * stride + ((lane % CPR) ^ fa_swz<D>(r)) * 8) * 2;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + (RPW * wave + i * RPI) * D), 16, o + base, 0, 0,
                                               0);
    }
  }
  // As issue, with the tile's start in the per-lane offset, which the
  // resource's range check covers (the scalar offset is not checked): rows
  // of the tile past the region read as zero.
  __device__ __forceinline__ void issue_checked(bf16* __restrict__ dst, __amdgpu_buffer_rsrc_t rsrc, int j0,
                                                int stride) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int base = j0 * stride * 2;
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + (RPW * wave + i * RPI) * D), 16,
                                               off[i] + base, 0, 0, 0);
  }
  // rows [j0, j0 + 64) of the region (row j at j * stride elements) into dst
  __device__ __forceinline__ void issue(bf16* __restrict__ dst, __amdgpu_buffer_rsrc_t rsrc, int j0,
                                        int stride) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int soff = __builtin_amdgcn_readfirstlane(j0 * stride * 2);
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + (RPW * wave + i * RPI) * D), 16, off[i],
                                               soff, 0, 0);
  }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t fa_rsrc(const bf16* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, (int)kBufWord3);
}

// Waits for every outstanding vector memory operation of the wave. The
// builtin (encoding of vmcnt(0), other counters untouched) lets the compiler's
// own wait insertion know the counter is drained; the empty asm statements
// keep memory accesses from moving across it.
__device__ __forceinline__ void fa_wait_loads() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);
  asm volatile("" ::: "memory");
}

// Waits until at most N vector memory operations of the wave are outstanding
// (the N most recently issued ones may still be in flight).
template <int N>
__device__ __forceinline__ void fa_wait_loads_keep() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
  asm volatile("" ::: "memory");
}

// Workgroup barrier for LDS hand-offs only: the wave's LDS operations are
// complete when it arrives (lgkmcnt), but its global stores are not waited
// for (a __syncthreads would wait for every outstanding memory operation).
// Direct-to-LDS loads must be waited for with fa_wait_loads() first. The
// memory clobber keeps memory accesses from moving across it.
__device__ __forceinline__ void fa_lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = (bf16)a;
  v[1] = (bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// Online-softmax step for one 64-key tile held in s[0..1] (16 scores per
// lane per 32-key half): rescale if the running max moved by more than
// kRescaleSlack for any lane, then p = exp2(s * scale_log2 - m) packed to
// bf16 in pw[kc] (the B operand of the PV chunk of keys [16kc, 16kc + 16));
// the row sum is accumulated in float32 from the unrounded probabilities.
template <int D, bool MASKED>
__device__ __forceinline__ void fa_softmax(FaState<D>& st, f32x16* s, u32x4* pw, float scale_log2) {
  float mx = __builtin_fmaxf(s[0][0], s[0][1]);
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int i = (sb == 0 ? 2 : 0); i < 16; ++i) mx = __builtin_fmaxf(mx, s[sb][i]);
  mx = xor32_max(mx);
  const float mx_s = mx * scale_log2;   // scale_log2 > 0
  if (__builtin_amdgcn_ballot_w64(mx_s > st.m + kRescaleSlack) != 0) {
    const float m_new = __builtin_fmaxf(st.m, mx_s);
    const float alpha = (m_new == -__builtin_inff()) ? 1.f : __builtin_amdgcn_exp2f(st.m - m_new);
    st.l *= alpha;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) st.o[t][i] *= alpha;
    st.m = m_new;
  }
  const float m_use = MASKED ? ((st.m == -__builtin_inff()) ? 0.f : st.m) : st.m;
  float psum = 0.f;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][i], scale_log2, -m_use));
      const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][i + 1], scale_log2, -m_use));
      pw[sb * 2 + (i >> 3)][(i & 7) >> 1] = pack_bf16x2(e0, e1);
      psum += e0 + e1;
    }
  st.l += psum;
}

// S^T = K Q^T for one 64-key tile in LDS (two 32-key halves); all K
// fragments are read before the matrix ops (one LDS latency per tile).
template <int D>
__device__ __forceinline__ void fa_scores(const FaState<D>& st, const bf16* __restrict__ ks, f32x16* s) {
  const char* kb = reinterpret_cast<const char*>(ks);
  constexpr int RB = D * 2;
  bf16x8 ka[2][D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c)
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) ka[sb][c] = *(const bf16x8*)(kb + st.kofs[c] + sb * 32 * RB);
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int i = 0; i < 16; ++i) s[sb][i] = 0.f;
#pragma unroll
  for (int c = 0; c < D / 16; ++c)
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[sb][c], st.q[c], s[sb], 0, 0, 0);
  // K reads run two k-steps ahead of the matrix ops that use them (at most
  // six fragments live, which keeps the register budget for two waves/SIMD)
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int c = 0; c < D / 16 - 2; ++c) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
}

// O^T += V^T P^T for one 64-key tile in LDS.
template <int D>
__device__ __forceinline__ void fa_pv(FaState<D>& st, const bf16* __restrict__ vs, const u32x4* pw) {
  const char* vb = reinterpret_cast<const char*>(vs);
  constexpr int RB = D * 2;
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) {
    const bf16x8 p = __builtin_bit_cast(bf16x8, pw[kc]);
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + st.vofs[t][0] + 16 * kc * RB));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + st.vofs[t][1] + 16 * kc * RB));
      const i16x4 both[2] = {lo, hi};
      st.o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, both), p, st.o[t], 0, 0, 0);
    }
  }
}

// Masking of a tile's scores: key_ok(kidx) for key kidx of the tile.
template <typename KeyOk>
__device__ __forceinline__ void fa_mask(f32x16* s, KeyOk key_ok) {
  const int h = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kidx = sb * 32 + (i >> 2) * 8 + h * 4 + (i & 3);
      if (!key_ok(kidx)) s[sb][i] = -__builtin_inff();
    }
}

// Softmax + PV of tile j (scores in s), masked when needed.
template <int D, bool CAN_MASK, typename KeyOk, typename TileFull>
__device__ __forceinline__ void fa_finish_tile(FaState<D>& st, f32x16* s, const bf16* __restrict__ vs,
                                               float scale_log2, int base, int n, KeyOk key_ok, TileFull tile_full) {
  u32x4 pw[4];
  if (CAN_MASK && !(base + kKT <= n && tile_full(base)))
    fa_mask(s, [&](int kidx) { return base + kidx < n && key_ok(base + kidx); });
  fa_softmax<D, CAN_MASK>(st, s, pw, scale_log2);
  fa_pv<D>(st, vs, pw);
}

// Runs all tiles of one key segment of n keys. row_ofs(j) -> element offset
// of key j (0 <= j < n) from K / V; key_ok(j) -> whether this lane's query
// attends key j; tile_full(j0) -> whether every lane of the calling wave
// attends all keys [j0, j0 + 64) (wave-uniform; lets the tile skip masking).
// CAN_MASK = false promises n % 64 == 0 and every key attended by every
// lane (no masking code is generated).
//
// Software pipeline, one barrier per tile: iteration j computes the scores
// of tile j+1 on the matrix cores while the softmax of tile j runs on the
// vector ALUs, then O += P_j V_j. K tiles live in two buffers (K_t in
// buffer t % 2), V tiles in two others (V_t in buffer t % 2); at the end of
// iteration j the buffers of K_{j+1} and V_j are free and receive K_{j+3} and
// V_{j+2}, so every direct load has a whole iteration to land. Must be
// called by all NW*64 threads of the workgroup.
//
// Split form: fa_segment_begin issues the first tiles' direct loads (no
// registers held), after which the caller may issue loads of its own and
// fold them into the state (their wait also covers the tiles, which are
// older); fa_segment_run then computes.
//
// The _tiles forms take an issuer: issue(dst, is_v, t) loads tile t of K
// (is_v false) or V into the LDS buffer dst for the calling wave.
template <int D, typename Issue>
__device__ __forceinline__ void fa_segment_begin_tiles(const FaSmem<D>& sm, int n, Issue issue) {
  if (n <= 0) return;
  const int nt = (n + kKT - 1) / kKT;
  issue(sm.k0, false, 0);
  issue(sm.v0, true, 0);
  if (nt > 1) {
    issue(sm.k1, false, 1);
    issue(sm.v1, true, 1);
  }
}

// One pipeline step: scores of the next tile (matrix cores) and the
// softmax of this one (vector ALUs), then O += P V. LATE issues the softmax
// first: with eight-wave workgroups the two waves that share a SIMD (w and
// w + 4) take opposite orders, so one wave's matrix ops run under the
// other's vector work.
template <int D, bool CAN_MASK, bool LATE, typename KeyOk, typename TileFull>
__device__ __forceinline__ void fa_step(FaState<D>& st, f32x16* s_now, f32x16* s_next, const bf16* __restrict__ ks_next,
                                        const bf16* __restrict__ vs, float scale_log2, int base, int n, KeyOk key_ok,
                                        TileFull tile_full) {
  u32x4 pw[4];
  if constexpr (!LATE) fa_scores<D>(st, ks_next, s_next);
  if (CAN_MASK && !(base + kKT <= n && tile_full(base)))
    fa_mask(s_now, [&](int kidx) { return base + kidx < n && key_ok(base + kidx); });
  fa_softmax<D, CAN_MASK>(st, s_now, pw, scale_log2);
  if constexpr (LATE) fa_scores<D>(st, ks_next, s_next);
  fa_pv<D>(st, vs, pw);
}

template <int D, bool CAN_MASK, bool LATE, typename Issue, typename KeyOk, typename TileFull>
__device__ __forceinline__ void fa_segment_loop(FaState<D>& st, const FaSmem<D>& sm, int n, float scale_log2,
                                                Issue issue, KeyOk key_ok, TileFull tile_full) {
  const int nt = (n + kKT - 1) / kKT;
  auto issue_k = [&](bf16* dst, int t) {
    if (t < nt) issue(dst, false, t);
  };
  auto issue_v = [&](bf16* dst, int t) {
    if (t < nt) issue(dst, true, t);
  };
  // prologue (K0, V0, K1, V1 issued by fa_segment_begin): S(0) computed,
  // then K2 into K0's buffer (after every wave has read K0)
  fa_wait_loads();
  fa_lds_barrier();
  f32x16 s_cur[2], s_nxt[2];
  fa_scores<D>(st, sm.k0, s_cur);
  fa_lds_barrier();
  issue_k(sm.k0, 2);
  for (int j = 0; j < nt; j += 2) {
    // ---- even j: S(j+1) from K buffer 1, PV(j) from V buffer 0. The score
    // tile is computed unconditionally (past the end it reads a buffer no
    // load is writing and the result is unused) so that it shares a basic
    // block with the softmax it should overlap.
    fa_step<D, CAN_MASK, LATE>(st, s_cur, s_nxt, sm.k1, sm.v0, scale_log2, j * kKT, n, key_ok, tile_full);
    if (j + 1 >= nt) break;
    fa_wait_loads();
    fa_lds_barrier();
    issue_k(sm.k1, j + 3);
    issue_v(sm.v0, j + 2);
    // ---- odd j+1: S(j+2) from K buffer 0, PV(j+1) from V buffer 1
    fa_step<D, CAN_MASK, LATE>(st, s_nxt, s_cur, sm.k0, sm.v1, scale_log2, (j + 1) * kKT, n, key_ok, tile_full);
    if (j + 2 >= nt) break;
    fa_wait_loads();
    fa_lds_barrier();
    issue_k(sm.k0, j + 4);
    issue_v(sm.v1, j + 3);
  }
  fa_wait_loads();
  fa_lds_barrier();
}

template <int D, bool CAN_MASK, int NW = 0, typename Issue, typename KeyOk, typename TileFull>
__device__ __forceinline__ void fa_segment_run_tiles(FaState<D>& st, const FaSmem<D>& sm, int n, float scale_log2,
                                                     Issue issue, KeyOk key_ok, TileFull tile_full) {
  if (n <= 0) return;
  if constexpr (NW == 8) {
    // one copy of the loop per issue order (same barriers in the same sequence)
    if (__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) >= NW / 2)
      fa_segment_loop<D, CAN_MASK, true>(st, sm, n, scale_log2, issue, key_ok, tile_full);
    else
      fa_segment_loop<D, CAN_MASK, false>(st, sm, n, scale_log2, issue, key_ok, tile_full);
  } else {
    fa_segment_loop<D, CAN_MASK, false>(st, sm, n, scale_log2, issue, key_ok, tile_full);
  }
}

// Row-offset forms: key j of the segment at element offset row_ofs(j) from
// K / V (fa_issue_one).
template <int D, int NW, typename RowOfs>
__device__ __forceinline__ void fa_segment_begin(const FaSmem<D>& sm, const bf16* __restrict__ K,
                                                 const bf16* __restrict__ V, int n, RowOfs row_ofs) {
  fa_segment_begin_tiles<D>(sm, n, [&](bf16* dst, bool is_v, int t) {
    fa_issue_one<D, NW>(dst, is_v ? V : K, t * kKT, n, row_ofs);
  });
}

// SPLIT: the two issue orders of fa_segment_run_tiles for eight-wave
// workgroups (false: one order, fewer registers: a kernel with several
// segments keeps one loop copy per segment and order).
template <int D, int NW, bool CAN_MASK, bool SPLIT = true, typename RowOfs, typename KeyOk, typename TileFull>
__device__ __forceinline__ void fa_segment_run(FaState<D>& st, const FaSmem<D>& sm, const bf16* __restrict__ K,
                                               const bf16* __restrict__ V, int n, float scale_log2,
                                               RowOfs row_ofs, KeyOk key_ok, TileFull tile_full) {
  fa_segment_run_tiles<D, CAN_MASK, SPLIT ? NW : 0>(st, sm, n, scale_log2, [&](bf16* dst, bool is_v, int t) {
    fa_issue_one<D, NW>(dst, is_v ? V : K, t * kKT, n, row_ofs);
  }, key_ok, tile_full);
}

template <int D, int NW, bool CAN_MASK, bool SPLIT = true, typename RowOfs, typename KeyOk, typename TileFull>
__device__ __forceinline__ void fa_segment(FaState<D>& st, const FaSmem<D>& sm, const bf16* __restrict__ K,
                                           const bf16* __restrict__ V, int n, float scale_log2, RowOfs row_ofs,
                                           KeyOk key_ok, TileFull tile_full) {
  fa_segment_begin<D, NW>(sm, K, V, n, row_ofs);
  fa_segment_run<D, NW, CAN_MASK, SPLIT>(st, sm, K, V, n, scale_log2, row_ofs, key_ok, tile_full);
}

// Final normalisation: returns the lane's 1/l and natural-log lse.
template <int D>
__device__ __forceinline__ void fa_finish(FaState<D>& st, float& inv_l, float& lse) {
  const float l = xor32_sum(st.l);
  inv_l = l > 0.f ? 1.f / l : 0.f;
  lse = l > 0.f ? st.m * kLn2 + logf(l) : -__builtin_inff();
}

// Epilogue staging, one group of 4 waves (128 rows) at a time: waves
// [4*half, 4*half + 4) write their rows of O (each scaled by `mul`) to LDS as
// float rows of D, wave w%4 into tile buffer w%4 (32 rows of D floats fit in
// one 64-key bf16 tile), with the 16-byte chunk q of row r stored at
// q ^ (r & 31); read back with fa_row_chunk. Call after the last fa_segment
// (whose trailing barrier frees the buffers) or after the previous half has
// been consumed; follow with __syncthreads().
template <int D>
__device__ __forceinline__ float* fa_row_buf(const FaSmem<D>& sm, int r) {
  bf16* b = (r >> 5) == 0 ? sm.k0 : (r >> 5) == 1 ? sm.v0 : (r >> 5) == 2 ? sm.k1 : sm.v1;
  return reinterpret_cast<float*>(b) + (r & 31) * D;
}

template <int D>
__device__ __forceinline__ void fa_rows_to_lds(FaState<D>& st, const FaSmem<D>& sm, float mul, int half) {
  static_assert(kKT * D * sizeof(bf16) >= 32 * D * sizeof(float), "tile buffer too small for 32 float rows");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if ((wave >> 2) != half) return;
  const int h = lane >> 5;
  const int row = (wave & 3) * 32 + (lane & 31);
  float* dst = fa_row_buf<D>(sm, row);
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      f32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = st.o[t][i4 * 4 + e] * mul;
      const int q = 8 * t + 2 * i4 + h;
      *(f32x4*)(dst + 4 * (q ^ (row & 31) & (D / 4 - 1))) = w;
    }
}

// Partner value across the two half-waves (lane l <-> l ^ 32): the swap
// returns the own and the partner value in some order, so xor-ing both with
// the own value leaves the partner's.
__device__ __forceinline__ uint32_t xchg32(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return r[0] ^ r[1] ^ x;
}

// Stores the lane's query row of O (times mul) as bf16 at dst, straight from
// the accumulators: the two half-waves trade 4-element groups so that each
// lane writes whole 16-byte pieces (D/16 stores per lane, no LDS).
template <int D>
__device__ __forceinline__ void fa_store_row_bf16(const FaState<D>& st, float mul, bf16* dst, bool ok) {
  const int h = (threadIdx.x >> 5) & 1;
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      // elements 8p..8p+3: d = 32t + 16p + 4h + 0..3; 8p+4..8p+7: d + 8
      const uint32_t a0 = pack_bf16x2(st.o[t][8 * p + 0] * mul, st.o[t][8 * p + 1] * mul);
      const uint32_t a1 = pack_bf16x2(st.o[t][8 * p + 2] * mul, st.o[t][8 * p + 3] * mul);
      const uint32_t b0 = pack_bf16x2(st.o[t][8 * p + 4] * mul, st.o[t][8 * p + 5] * mul);
      const uint32_t b1 = pack_bf16x2(st.o[t][8 * p + 6] * mul, st.o[t][8 * p + 7] * mul);
      // lower half keeps d 16p+0..3 and takes the partner's 4..7; upper half
      // keeps 12..15 and takes the partner's 8..11
      const uint32_t r0 = xchg32(h ? a0 : b0), r1 = xchg32(h ? a1 : b1);
      u32x4 w;
      w[0] = h ? r0 : a0;
      w[1] = h ? r1 : a1;
      w[2] = h ? b0 : r0;
      w[3] = h ? b1 : r1;
      if (ok) *(u32x4*)(dst + 32 * t + 16 * p + 8 * h) = w;
    }
}

// Stores the wave's 32 query rows of O (times mul) as bf16 rows through an
// LDS staging area: each lane first writes its accumulator groups into its
// row (rows padded by 16 bytes, so the writes spread over the banks), then
// 16 lanes per row read back whole 16-byte chunks and write them out, so
// each store instruction covers four complete 2*D-byte rows instead of 32
// fragments. stage: this wave's 32 rows of D + 8 bf16; rows: its 32 output
// row indices (a lane's row index < 0 skips that row).
//
// Row layout ("split halves"): the D/2 values a lower-half lane holds (d with
// d % 8 < 4, in accumulator order) come first, then the upper half's, so a
// reader with the same register layout fetches its values as D/16
// contiguous 16-byte pieces.
//
// The stores are non-temporal: the rows are read back only by a later
// kernel, after the whole pass has written far more than the memory-side
// cache holds, so caching them would leave dirty lines whose write-back
// then competes with that kernel's reads (a plain 512 MiB write followed by
// a 1 GiB read runs the read at about 4.3 TB/s, against 6.2 TB/s after a
// non-temporal write of the same bytes).
template <int D>
__device__ __forceinline__ void fa_store_rows_staged(const FaState<D>& st, float mul, bf16* stage, int64_t* rows,
                                                     int64_t my_row, bf16* __restrict__ out) {
  constexpr int RS = D + 8;   // padded row stride (elements)
  const int lane = threadIdx.x & 63, h = lane >> 5, r = lane & 31;
  if (h == 0) rows[r] = my_row;
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      uint2 w;
      w.x = pack_bf16x2(st.o[t][4 * gi + 0] * mul, st.o[t][4 * gi + 1] * mul);
      w.y = pack_bf16x2(st.o[t][4 * gi + 2] * mul, st.o[t][4 * gi + 3] * mul);
      *(uint2*)(stage + r * RS + h * (D / 2) + 4 * (4 * t + gi)) = w;
    }
  constexpr int CPR = D / 8;    // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;
#pragma unroll
  for (int k = 0; k < 32 / RPI; ++k) {
    const int row = k * RPI + lane / CPR, c = lane % CPR;
    const int64_t dst = rows[row];
    const u32x4 v = *(const u32x4*)(stage + row * RS + 8 * c);
    if (dst >= 0) __builtin_nontemporal_store(v, (u32x4*)(out + dst * D + 8 * c));
  }
}

// Workgroup id remapped so that consecutive logical ids run on the same XCD:
// the hardware deals workgroups to the 8 XCDs round-robin, and tiles that
// share K/V then share that XCD's L2.
__device__ __forceinline__ int64_t xcd_logical_id(int64_t bid, int64_t nwg) {
  constexpr int kXcd = 8;
  const int64_t x = bid % kXcd, local = bid / kXcd;
  const int64_t per = nwg / kXcd, rem = nwg % kXcd;
  const int64_t start = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
  return start + local;
}

// 4 floats [4q, 4q + 4) of staged row r (0 <= r < 128).
template <int D>
__device__ __forceinline__ f32x4 fa_row_chunk(const FaSmem<D>& sm, int r, int q) {
  return *(const f32x4*)(fa_row_buf<D>(sm, r) + 4 * (q ^ (r & 31) & (D / 4 - 1)));
}

}  // namespace qat
