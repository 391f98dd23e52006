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
// Layout (one workgroup = 4 waves = 128 query rows; one wave = 32 rows):
// the wave computes S^T = K Q^T (A = K tile from LDS, B = Q from
// registers) so that each lane owns ONE query (lane % 32) and 16 key
// scores per 32-key subtile; row max / row sum are lane-local plus one
// exchange with lane ^ 32. Then O^T += V^T P^T (A = V^T from LDS, B = P
// from registers); the key order inside each 16-key chunk is permuted
// (bits 2 and 3 of the key offset swapped) so that the probabilities a lane
// already holds form its B operand without any data movement, and V is
// stored transposed in LDS in that permuted order.
#pragma once

#include "common.h"

namespace qat {

constexpr int kKT = 64;          // keys per tile
constexpr int kKPad = 8;         // bf16 padding of a K row in LDS
constexpr int kVPad = 8;         // bf16 padding of a V^T row in LDS
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D>
struct FaSmem {
  bf16 k[2][kKT][D + kKPad];
  bf16 vt[2][D][kKT + kVPad];
};

template <int D>
struct FaState {
  f32x16 o[D / 32];   // O^T: lane's query (lane%32), d = 32*dt + 8*(i/4) + 4*(lane/32) + i%4
  bf16x8 q[D / 16];   // B operand of S^T: q[row][16c + 8*(lane/32) .. +8]
  float m;            // running max of scaled scores, log2 units
  float l;            // lane-partial running sum (combine with lane^32 at the end)
};

__device__ __forceinline__ int swap23(int o) {
  return (o & ~0xC) | ((o & 4) << 1) | ((o & 8) >> 1);
}

template <int D>
__device__ __forceinline__ void fa_init(FaState<D>& st, const bf16* qrow, bool valid) {
  const int h = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    if (valid) {
      st.q[c] = *(const bf16x8*)(qrow + 16 * c + 8 * h);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) st.q[c][j] = (bf16)0.f;
    }
  }
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) st.o[t][i] = 0.f;
  st.m = -__builtin_inff();
  st.l = 0.f;
}

// Global -> register staging of one 64-key tile for the whole workgroup
// (256 threads). K: 4 chunks of 16 B per thread (D = 128), V: 4 keys x 8 d
// per thread. `row_of(j)` returns the element offset of key j's row (or -1
// when j is beyond the segment: zeros are staged and the key is masked).
template <int D>
struct FaStage {
  static constexpr int kChunks = kKT * D / 8;            // 16 B chunks of K
  static constexpr int kKPer = kChunks / 256;             // per thread
  static constexpr int kVGroups = (kKT / 4) * (D / 8);    // 4 keys x 8 d groups
  bf16x8 kr[kKPer > 0 ? kKPer : 1];
  bf16x8 vr[4];
};

template <int D, typename RowOf>
__device__ __forceinline__ void fa_load(FaStage<D>& sg, const bf16* __restrict__ K,
                                        const bf16* __restrict__ V, RowOf row_of) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < FaStage<D>::kKPer; ++i) {
    const int c = tid + 256 * i;
    const int key = c / (D / 8), part = c % (D / 8);
    const int64_t off = row_of(key);
    if (off >= 0) {
      sg.kr[i] = *(const bf16x8*)(K + off + part * 8);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) sg.kr[i][j] = (bf16)0.f;
    }
  }
  if (tid < FaStage<D>::kVGroups) {
    const int kg = tid / (D / 8), dc = tid % (D / 8);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t off = row_of(4 * kg + r);
      if (off >= 0) {
        sg.vr[r] = *(const bf16x8*)(V + off + dc * 8);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) sg.vr[r][j] = (bf16)0.f;
      }
    }
  }
}

template <int D>
__device__ __forceinline__ void fa_store(const FaStage<D>& sg, FaSmem<D>& sm, int buf) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < FaStage<D>::kKPer; ++i) {
    const int c = tid + 256 * i;
    const int key = c / (D / 8), part = c % (D / 8);
    *(bf16x8*)&sm.k[buf][key][part * 8] = sg.kr[i];
  }
  if (tid < FaStage<D>::kVGroups) {
    const int kg = tid / (D / 8), dc = tid % (D / 8);
    const int kp = swap23(4 * kg);   // 4 consecutive keys stay consecutive
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      bf16x4 v4;
      v4[0] = sg.vr[0][j];
      v4[1] = sg.vr[1][j];
      v4[2] = sg.vr[2][j];
      v4[3] = sg.vr[3][j];
      *(bf16x4*)&sm.vt[buf][dc * 8 + j][kp] = v4;
    }
  }
}

// One 64-key tile for one wave. `key_ok(kidx)` says whether key kidx of the
// tile may be attended by this lane's query (segment bound and causality).
template <int D, typename KeyOk>
__device__ __forceinline__ void fa_tile(FaState<D>& st, const FaSmem<D>& sm, int buf, float scale_log2,
                                        KeyOk key_ok) {
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5, r32 = lane & 31;
  f32x16 s[2];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const bf16x8 a = *(const bf16x8*)&sm.k[buf][sb * 32 + r32][16 * c + 8 * h];
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, st.q[c], acc, 0, 0, 0);
    }
    s[sb] = acc;
  }
  // scale, mask, tile max
  float mx = -__builtin_inff();
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kidx = sb * 32 + (i >> 2) * 8 + h * 4 + (i & 3);
      const float x = key_ok(kidx) ? s[sb][i] * scale_log2 : -__builtin_inff();
      s[sb][i] = x;
      mx = fmaxf(mx, x);
    }
  mx = fmaxf(mx, shfl_xor_f(mx, 32));
  const float m_new = fmaxf(st.m, mx);
  const float m_use = (m_new == -__builtin_inff()) ? 0.f : m_new;
  const float alpha = exp2f(st.m - m_use);
  float psum = 0.f;
  bf16x8 p[4];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float e = exp2f(s[sb][i] - m_use);
      psum += e;
      p[sb * 2 + (i >> 3)][i & 7] = (bf16)e;
    }
  st.l = st.l * alpha + psum;
  st.m = m_new;
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) st.o[t][i] *= alpha;
#pragma unroll
  for (int kc = 0; kc < 4; ++kc)
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
      const bf16x8 a = *(const bf16x8*)&sm.vt[buf][32 * t + r32][16 * kc + 8 * h];
      st.o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p[kc], st.o[t], 0, 0, 0);
    }
}

// Runs all tiles of one key segment of n keys. row_of(j) -> element offset of
// key j (0 <= j < n) in K/V; key_ok(j) -> whether this lane's query attends
// key j. Must be called by all 256 threads of the workgroup.
template <int D, typename RowOf, typename KeyOk>
__device__ __forceinline__ void fa_segment(FaState<D>& st, FaSmem<D>& sm, const bf16* __restrict__ K,
                                           const bf16* __restrict__ V, int64_t n, float scale_log2,
                                           RowOf row_of, KeyOk key_ok) {
  if (n <= 0) return;
  const int64_t ntiles = cdiv(n, kKT);
  FaStage<D> sg;
  auto tile_rows = [&](int64_t tile) {
    return [=](int j) -> int64_t {
      const int64_t jj = tile * kKT + j;
      return jj < n ? row_of(jj) : (int64_t)-1;
    };
  };
  fa_load<D>(sg, K, V, tile_rows(0));
  fa_store<D>(sg, sm, 0);
  __syncthreads();
  for (int64_t tile = 0; tile < ntiles; ++tile) {
    const int buf = (int)(tile & 1);
    if (tile + 1 < ntiles) fa_load<D>(sg, K, V, tile_rows(tile + 1));
    const int64_t base = tile * kKT;
    fa_tile<D>(st, sm, buf, scale_log2, [&](int kidx) { return base + kidx < n && key_ok(base + kidx); });
    if (tile + 1 < ntiles) fa_store<D>(sg, sm, buf ^ 1);
    __syncthreads();
  }
}

// Final normalisation: returns the lane's 1/l and natural-log lse.
template <int D>
__device__ __forceinline__ void fa_finish(FaState<D>& st, float& inv_l, float& lse) {
  const float l = st.l + shfl_xor_f(st.l, 32);
  inv_l = l > 0.f ? 1.f / l : 0.f;
  lse = l > 0.f ? st.m * kLn2 + logf(l) : -__builtin_inff();
}

// d index held in st.o[t][i] by this lane.
__device__ __forceinline__ int fa_d_of(int t, int i) {
  const int h = (threadIdx.x & 63) >> 5;
  return 32 * t + 8 * (i >> 2) + 4 * h + (i & 3);
}

}  // namespace qat
