// Gradient tile engine on the bf16 matrix cores, shared by the MoBA and ESA
// sparse-attention gradients (gradients of softmax attention over an
// explicit key set: p = exp(scale q.k - lse), dp = dO.v, D = sum p dp,
// dq = scale sum p (dp - D) k, dk += scale p (dp - D) q, dv += p dO).
// Built on the forward tile engine (attn_core.h): the same LDS tiles,
// swizzle, direct loads and transposing reads.
#pragma once

#include "attn_core.h"
#include "common.h"

namespace qat {

// ---------------------------------------------------------------------------
// dq on the bf16 matrix cores (bfloat16 inputs), with the tile engine's
// layout: per 64-key tile, S^T = K Q^T and dP^T = V dO^T (A = K or V tile
// from LDS, B = the row's q or dO in registers, so each lane owns one row
// and 16 keys per 32-key half) and p = exp2(S scale log2e - lse log2e) from
// the forward's lse. D is not known before the row's last key, so the pass
// accumulates D = sum p dp, A = sum p dp k and B = sum p k, and
// dq = scale (A - D B) at the end: A^T += K^T (p dp)^T and B^T += K^T p^T
// with A = K^T by transposing reads of the same K tile (as V^T in the
// forward), each B operand split into bfloat16 hi + lo (their sum carries
// the value to 2^-17 relative, so A - D B keeps its accuracy).
constexpr int kBwdNW = 4;   // waves of the matrix-core gradient kernels (one per SIMD: 512 registers)

template <int D>
struct DqState {
  FaState<D> fa;          // q as B operand, A^T accumulator in fa.o, LDS offsets
  f32x16 b[D / 32];       // B^T accumulator (same layout as fa.o)
  bf16x8 dob[D / 16];     // dO as B operand
  float lse2, dsum;       // dsum: this lane's keys only (halves joined at the end)
};

template <int D>
__device__ __forceinline__ void dq_init(DqState<D>& st, const bf16* qrow, const bf16* drow, float lse, bool valid) {
  fa_init<D>(st.fa, qrow, valid);
  const int h = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    if (valid) {
      st.dob[c] = *(const bf16x8*)(drow + 16 * c + 8 * h);
    } else {
      const u32x4 z = {0u, 0u, 0u, 0u};
      st.dob[c] = __builtin_bit_cast(bf16x8, z);
    }
  }
#pragma unroll
  for (int tq = 0; tq < D / 32; ++tq)
#pragma unroll
    for (int i = 0; i < 16; ++i) st.b[tq][i] = 0.f;
  st.lse2 = valid ? lse * kLog2e : 0.f;
  st.dsum = 0.f;
}

// S^T-shaped product of one 64-row LDS tile (A) with per-lane B fragments.
template <int D>
__device__ __forceinline__ void dq_tile_prod(const int* kofs, const bf16* __restrict__ tile, const bf16x8* b,
                                             f32x16* s) {
  const char* kb = reinterpret_cast<const char*>(tile);
  constexpr int RB = D * 2;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int i = 0; i < 16; ++i) s[sb][i] = 0.f;
#pragma unroll
  for (int c = 0; c < D / 16; ++c)
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const bf16x8 a = *(const bf16x8*)(kb + kofs[c] + sb * 32 * RB);
      s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[c], s[sb], 0, 0, 0);
    }
}

// The 32-key (or 32-row) half sb of two such products at once, S from tile
// a with fragments b and dP from tile c with fragments d (the two chains
// interleaved; the same operands and order as dq_tile_prod).
template <int D>
__device__ __forceinline__ void dq_half_prod(const int* kofs, const bf16* __restrict__ a_tile, const bf16x8* b,
                                             const bf16* __restrict__ c_tile, const bf16x8* d, int sb, f32x16& s,
                                             f32x16& dp) {
  const char* ab = reinterpret_cast<const char*>(a_tile);
  const char* cb = reinterpret_cast<const char*>(c_tile);
  constexpr int RB = D * 2;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    s[i] = 0.f;
    dp[i] = 0.f;
  }
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    const bf16x8 x = *(const bf16x8*)(ab + kofs[c] + sb * 32 * RB);
    const bf16x8 y = *(const bf16x8*)(cb + kofs[c] + sb * 32 * RB);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, b[c], s, 0, 0, 0);
    dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(y, d[c], dp, 0, 0, 0);
  }
}

// bfloat16 hi + lo split of a pair: .x = packed hi, .y = packed lo
__device__ __forceinline__ uint2 split_pack(float x0, float x1) {
  const bf16 h0 = (bf16)x0, h1 = (bf16)x1;
  return make_uint2(pack_bf16x2((float)h0, (float)h1), pack_bf16x2(x0 - (float)h0, x1 - (float)h1));
}

// One 64-key tile: keys with key_ok(kidx) false (kidx 0..63 within the tile)
// get p = 0.
template <int D, typename KeyOk>
__device__ __forceinline__ void dq_tile(DqState<D>& st, const bf16* __restrict__ ks, const bf16* __restrict__ vs,
                                        float sl2, KeyOk key_ok) {
  f32x16 s[2], dp[2];
  dq_tile_prod<D>(st.fa.kofs, ks, st.fa.q, s);
  dq_tile_prod<D>(st.fa.kofs, vs, st.dob, dp);
  const int h = (threadIdx.x & 63) >> 5;
  u32x4 pdh[4], pdl[4], ph[4], pl[4];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      float p2[2], pd2[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int kidx = sb * 32 + ((i + u) >> 2) * 8 + h * 4 + ((i + u) & 3);
        p2[u] = key_ok(kidx) ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][i + u], sl2, -st.lse2)) : 0.f;
        pd2[u] = p2[u] * dp[sb][i + u];
        st.dsum += pd2[u];
      }
      const int kc = sb * 2 + (i >> 3), w = (i & 7) >> 1;
      const uint2 a2 = split_pack(pd2[0], pd2[1]), b2 = split_pack(p2[0], p2[1]);
      pdh[kc][w] = a2.x;
      pdl[kc][w] = a2.y;
      ph[kc][w] = b2.x;
      pl[kc][w] = b2.y;
    }
  const char* kb = reinterpret_cast<const char*>(ks);
  constexpr int RB = D * 2;
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
    for (int tq = 0; tq < D / 32; ++tq) {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(kb + st.fa.vofs[tq][0] + 16 * kc * RB));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(kb + st.fa.vofs[tq][1] + 16 * kc * RB));
      const i16x4 both[2] = {lo, hi};
      const bf16x8 a = __builtin_bit_cast(bf16x8, both);
      st.fa.o[tq] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, pdh[kc]), st.fa.o[tq], 0, 0, 0);
      st.fa.o[tq] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, pdl[kc]), st.fa.o[tq], 0, 0, 0);
      st.b[tq] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, ph[kc]), st.b[tq], 0, 0, 0);
      st.b[tq] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, pl[kc]), st.b[tq], 0, 0, 0);
    }
  }
}

// All tiles of n keys from K / V (row_ofs(j): key j's element offset), K and
// V tiles double-buffered in LDS, one barrier per tile. Called by all NW*64
// threads of the workgroup.
template <int D, int NW, typename RowOfs, typename KeyOk>
__device__ __forceinline__ void dq_segment(DqState<D>& st, const FaSmem<D>& sm, const bf16* __restrict__ K,
                                           const bf16* __restrict__ V, int n, float sl2, RowOfs row_ofs,
                                           KeyOk key_ok) {
  if (n <= 0) return;
  const int nt = (n + kKT - 1) / kKT;
  fa_issue_one<D, NW>(sm.k0, K, 0, n, row_ofs);
  fa_issue_one<D, NW>(sm.v0, V, 0, n, row_ofs);
  for (int j = 0; j < nt; j += 2) {
    fa_wait_loads();
    fa_lds_barrier();
    if (j + 1 < nt) {
      fa_issue_one<D, NW>(sm.k1, K, (j + 1) * kKT, n, row_ofs);
      fa_issue_one<D, NW>(sm.v1, V, (j + 1) * kKT, n, row_ofs);
    }
    dq_tile<D>(st, sm.k0, sm.v0, sl2, [&](int kidx) { return j * kKT + kidx < n && key_ok(j * kKT + kidx); });
    if (j + 1 >= nt) break;
    fa_wait_loads();
    fa_lds_barrier();
    if (j + 2 < nt) {
      fa_issue_one<D, NW>(sm.k0, K, (j + 2) * kKT, n, row_ofs);
      fa_issue_one<D, NW>(sm.v0, V, (j + 2) * kKT, n, row_ofs);
    }
    dq_tile<D>(st, sm.k1, sm.v1, sl2,
               [&](int kidx) { return (j + 1) * kKT + kidx < n && key_ok((j + 1) * kKT + kidx); });
  }
  fa_wait_loads();
  fa_lds_barrier();
}

// ---------------------------------------------------------------------------
// dK and dV on the matrix cores (bfloat16 inputs): the tile engine with the
// roles of rows and keys exchanged. A wave holds 32 keys of the block as B
// operands (K^T and V^T fragments, lane = key) and its dK^T, dV^T
// accumulators; the rows stream through LDS 64 at a time (q and dO tiles,
// double-buffered direct loads, with each row's lse and D). Per row tile:
// S = Q K^T and dP = dO V^T (A = the q / dO tile, so each lane holds one key
// and 16 rows per 32-row half), p = exp2(S scale log2e - lse log2e),
// ds = p (dp - D), then dV^T += dO^T p and dK^T += Q^T ds with A = dO^T /
// Q^T by transposing reads of the tiles (as V^T in the forward) and p, ds
// split into bfloat16 hi + lo.
constexpr int kKvKeys = 32 * kBwdNW;   // keys per workgroup (32 per wave)

template <int D>
struct KvState {
  FaState<D> fa;          // K^T fragments in fa.q, dK^T in fa.o, LDS offsets
  bf16x8 vq[D / 16];      // V^T fragments
  f32x16 dv[D / 32];      // dV^T
};

template <int D>
__device__ __forceinline__ void kv_load(KvState<D>& st, const bf16* krow, const bf16* vrow) {
  fa_init<D>(st.fa, krow, true);
  const int h = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) st.vq[c] = *(const bf16x8*)(vrow + 16 * c + 8 * h);
#pragma unroll
  for (int tq = 0; tq < D / 32; ++tq)
#pragma unroll
    for (int i = 0; i < 16; ++i) st.dv[tq][i] = 0.f;
}

// One tile of up to 64 rows: rows m with row_ok(m) false get p = 0. lse_t /
// di_t: the tile's lse (natural log) and D per row, in LDS.
template <int D, typename RowOk>
__device__ __forceinline__ void kv_tile(KvState<D>& st, const bf16* __restrict__ qt, const bf16* __restrict__ dt,
                                        const float* lse_t, const float* di_t, float sl2, RowOk row_ok) {
  const int h = (threadIdx.x & 63) >> 5;
  const char* qb = reinterpret_cast<const char*>(qt);
  const char* db = reinterpret_cast<const char*>(dt);
  constexpr int RB = D * 2;
  // one 32-row half at a time, from its S and dP products to the row chunks
  // kc = 2 sb, 2 sb + 1 of the accumulations (only one half's scores live)
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    // the second half's products are not hoisted above the first half's work
    if (sb) __builtin_amdgcn_sched_barrier(0);
    f32x16 s[2], dp[2];
    dq_half_prod<D>(st.fa.kofs, qt, st.fa.q, dt, st.vq, sb, s[sb], dp[sb]);
    u32x4 pph[2], ppl[2], dsh[2], dsl[2];
    // the half's 16 rows of this lane are 4 runs of 4 consecutive rows
    f32x4 l4[4], d4[4];
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      l4[gi] = *(const f32x4*)(lse_t + sb * 32 + gi * 8 + h * 4);
      d4[gi] = *(const f32x4*)(di_t + sb * 32 + gi * 8 + h * 4);
    }
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      float p2[2], ds2[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int m = sb * 32 + ((i + u) >> 2) * 8 + h * 4 + ((i + u) & 3);
        const float l2 = l4[(i + u) >> 2][(i + u) & 3] * kLog2e, di = d4[(i + u) >> 2][(i + u) & 3];
        p2[u] = row_ok(m) ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][i + u], sl2, -l2)) : 0.f;
        ds2[u] = p2[u] * (dp[sb][i + u] - di);
      }
      const int kk = i >> 3, w = (i & 7) >> 1;
      const uint2 a2 = split_pack(p2[0], p2[1]), b2 = split_pack(ds2[0], ds2[1]);
      pph[kk][w] = a2.x;
      ppl[kk][w] = a2.y;
      dsh[kk][w] = b2.x;
      dsl[kk][w] = b2.y;
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int kc = 2 * sb + kk;
#pragma unroll
      for (int tq = 0; tq < D / 32; ++tq) {
        const i16x4 d0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(db + st.fa.vofs[tq][0] + 16 * kc * RB));
        const i16x4 d1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(db + st.fa.vofs[tq][1] + 16 * kc * RB));
        const i16x4 q0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(qb + st.fa.vofs[tq][0] + 16 * kc * RB));
        const i16x4 q1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(qb + st.fa.vofs[tq][1] + 16 * kc * RB));
        const i16x4 dd[2] = {d0, d1}, qq[2] = {q0, q1};
        const bf16x8 ad = __builtin_bit_cast(bf16x8, dd), aq = __builtin_bit_cast(bf16x8, qq);
        st.dv[tq] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad, __builtin_bit_cast(bf16x8, pph[kk]), st.dv[tq], 0, 0, 0);
        st.dv[tq] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad, __builtin_bit_cast(bf16x8, ppl[kk]), st.dv[tq], 0, 0, 0);
        st.fa.o[tq] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, __builtin_bit_cast(bf16x8, dsh[kk]), st.fa.o[tq], 0, 0, 0);
        st.fa.o[tq] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, __builtin_bit_cast(bf16x8, dsl[kk]), st.fa.o[tq], 0, 0, 0);
      }
    }
  }
}

// This lane's key's dK, dV (accumulator layout d = 32 tq + 8 gi + 4 h + e)
// stored (ADD = false) or added with float atomics.
template <int D, bool ADD>
__device__ __forceinline__ void kv_write(const KvState<D>& st, float* dkr, float* dvr, float scale) {
  const int h = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int tq = 0; tq < D / 32; ++tq)
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const int d0 = 32 * tq + 8 * gi + 4 * h;
      if constexpr (ADD) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          unsafeAtomicAdd(dkr + d0 + e, scale * st.fa.o[tq][4 * gi + e]);
          unsafeAtomicAdd(dvr + d0 + e, st.dv[tq][4 * gi + e]);
        }
      } else {
        f32x4 a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = scale * st.fa.o[tq][4 * gi + e];
          b[e] = st.dv[tq][4 * gi + e];
        }
        *(f32x4*)(dkr + d0) = a;
        *(f32x4*)(dvr + d0) = b;
      }
    }
}

}  // namespace qat
