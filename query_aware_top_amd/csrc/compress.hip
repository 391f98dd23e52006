// Compression of concatenated-head rows by one affine map, accumulated in
// float64 on the fp64 matrix cores and rounded once.
//
// ESA write-up (hlszyjy.com/post/6872.html), paragraph on compressing query
// and key from 4096 to 128 dimensions with a one-layer MLP: read as one
// affine map out = W x + b. The products of two bf16 (or two fp32) values are
// exact in float64 and the float64 sum of d_model of them is far below the
// bf16 rounding grid, so the bf16 compressed-key cache written here is the
// correctly rounded value of the exact product.
#include "common.h"
#include "launch.h"

namespace qat {

// The fp64 MFMA 16x16x4 takes A[row = lane%16][k-slot = lane/16],
// B[k-slot = lane/16][col = lane%16] and returns D[row = lane/16 + 4i][col =
// lane%16]. Any assignment of k to the four slots works if both operands use
// it: lane slot j takes k = kb + 8 j + s at step s of a 32-k chunk, so each
// lane reads 8 consecutive k of its x row and of each W row with one 16-byte
// load. A wave owns 16 rows x 64 columns (four accumulators sharing the x
// operand); a workgroup stacks 4 waves over 64 rows. The next chunk's loads
// are issued before the current chunk's 32 matrix ops.
constexpr int kCmpRows = 64;
constexpr int kCmpCols = 64;

template <typename T>
struct Raw8;   // 8 consecutive elements as loaded
template <>
struct Raw8<bf16> {
  u32x4 v;
  __device__ __forceinline__ void load(const bf16* p) { v = *(const u32x4*)p; }
  __device__ __forceinline__ double get(int s) const {
    const uint32_t w = v[s >> 1];
    return (double)__builtin_bit_cast(float, (s & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};
template <>
struct Raw8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *(const f32x4*)p;
    b = *(const f32x4*)(p + 4);
  }
  __device__ __forceinline__ double get(int s) const { return (double)(s < 4 ? a[s] : b[s - 4]); }
};

template <typename TX, typename TW>
__global__ __launch_bounds__(256) void compress_partial_kernel(
    const TX* __restrict__ x, int64_t n, int64_t x_stride, int64_t d_model,
    const TW* __restrict__ W, int64_t d_c, int64_t k_per_split, double* __restrict__ partial) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t row0 = (int64_t)blockIdx.x * kCmpRows + wave * 16;
  const int64_t col0 = (int64_t)blockIdx.y * kCmpCols;
  const int split = blockIdx.z;
  const int64_t k0 = (int64_t)split * k_per_split;
  const int64_t k1 = min(d_model, k0 + k_per_split);
  const int r = lane & 15, j = lane >> 4;
  const int64_t row = row0 + r;
  const TX* xr = x + (row < n ? row : 0) * x_stride + 8 * j;
  const int ncb = (int)min((int64_t)4, (d_c - col0) / 16);   // column blocks of 16 in range
  const TW* wr[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) wr[cb] = W + (col0 + 16 * min(cb, ncb - 1) + r) * d_model + 8 * j;
  f64x4 acc[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) acc[cb] = f64x4{0.0, 0.0, 0.0, 0.0};
  Raw8<TX> xa;
  Raw8<TW> wa[4];
  if (k0 < k1) {
    xa.load(xr + k0);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) wa[cb].load(wr[cb] + k0);
  }
  for (int64_t kb = k0; kb < k1; kb += 32) {
    const Raw8<TX> xc = xa;
    Raw8<TW> wc[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) wc[cb] = wa[cb];
    if (kb + 32 < k1) {
      xa.load(xr + kb + 32);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) wa[cb].load(wr[cb] + kb + 32);
    }
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const double av = row < n ? xc.get(st) : 0.0;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) acc[cb] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, wc[cb].get(st), acc[cb], 0, 0, 0);
    }
  }
  double* dst = partial + (int64_t)split * n * d_c;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    if (cb >= ncb) break;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t orow = row0 + j + 4 * i;
      if (orow < n) dst[orow * d_c + col0 + 16 * cb + r] = acc[cb][i];
    }
  }
}

// Few rows (decode: one row per sequence): the four waves of a workgroup
// take four 16-column blocks of the same 16 rows, one accumulator each, so a
// wave runs a quarter of the matrix ops of the row-stacked layout above over
// the same k range and no wave computes rows past n. Same operand order,
// same partial layout.
constexpr int kCmpColRows = 32;   // at most this many rows use the column layout

template <typename TX, typename TW>
__global__ __launch_bounds__(256) void compress_partial_cols_kernel(
    const TX* __restrict__ x, int64_t n, int64_t x_stride, int64_t d_model,
    const TW* __restrict__ W, int64_t d_c, int64_t k_per_split, double* __restrict__ partial) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t row0 = (int64_t)blockIdx.x * 16;
  const int64_t col0 = ((int64_t)blockIdx.y * 4 + wave) * 16;
  if (col0 >= d_c) return;   // wave-uniform; no barrier below
  const int split = blockIdx.z;
  const int64_t k0 = (int64_t)split * k_per_split;
  const int64_t k1 = min(d_model, k0 + k_per_split);
  const int r = lane & 15, j = lane >> 4;
  const int64_t row = row0 + r;
  const TX* xr = x + (row < n ? row : 0) * x_stride + 8 * j;
  const TW* wr = W + (col0 + r) * d_model + 8 * j;
  f64x4 acc = f64x4{0.0, 0.0, 0.0, 0.0};
  Raw8<TX> xa;
  Raw8<TW> wa;
  if (k0 < k1) {
    xa.load(xr + k0);
    wa.load(wr + k0);
  }
  for (int64_t kb = k0; kb < k1; kb += 32) {
    const Raw8<TX> xc = xa;
    const Raw8<TW> wc = wa;
    if (kb + 32 < k1) {
      xa.load(xr + kb + 32);
      wa.load(wr + kb + 32);
    }
#pragma unroll
    for (int st = 0; st < 8; ++st)
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64(row < n ? xc.get(st) : 0.0, wc.get(st), acc, 0, 0, 0);
  }
  double* dst = partial + (int64_t)split * n * d_c;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t orow = row0 + j + 4 * i;
    if (orow < n) dst[orow * d_c + col0 + r] = acc[i];
  }
}

// Sum the split partials in split order, add the bias, round once.
// kind 0: float32 out; 1: bf16 out; 2: float32 out plus bf16 hi/lo split
// (hi = bf16(v), lo = bf16(v - hi)) used by the two-term bf16 scoring.
__global__ void compress_finalize_kernel(const double* __restrict__ partial, int nsplit, int64_t n,
                                         int64_t d_c, const float* __restrict__ bias, void* out,
                                         int64_t out_stride, int kind, bf16* __restrict__ hi,
                                         bf16* __restrict__ lo) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n * d_c) return;
  const int64_t row = idx / d_c, col = idx % d_c;
  // in split order; sixteen partials are loaded at a time so that their
  // loads overlap
  double v = 0.0;
  int s = 0;
  for (; s + 16 <= nsplit; s += 16) {
    double t[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) t[u] = partial[(int64_t)(s + u) * n * d_c + idx];
#pragma unroll
    for (int u = 0; u < 16; ++u) v += t[u];
  }
  for (; s < nsplit; ++s) v += partial[(int64_t)s * n * d_c + idx];
  if (bias) v += (double)bias[col];
  if (kind == 1) {
    ((bf16*)out)[row * out_stride + col] = f64_to_bf16_rne(v);
  } else {
    const float f = (float)v;
    ((float*)out)[row * out_stride + col] = f;
    if (kind == 2) {
      const bf16 h = (bf16)f;
      hi[idx] = h;
      lo[idx] = (bf16)(f - (float)h);
    }
  }
}

// Query compression of a chunk (many rows, bf16 x and W) on the bf16
// matrix cores with float32 accumulation: the products of two bf16 values
// are exact in float32 and only the accumulation rounds (about 2^-18
// relative over 4096 terms, far below what the scores summed over the
// chunk's queries can resolve), so the fp64 path is kept for the key cache
// (which must be correctly rounded) and for decode rows. One launch; a
// workgroup takes 32 rows and 32 output columns (so a CU streams a quarter
// of W, not all of it), its four waves each a quarter of d_model, computing
// out^T = W x^T on the 16x16x32 op (A = 16 rows of W, B = 16 rows of x; each
// lane loads 16 contiguous bytes, four lanes 64 of one row); the quarters are
// added in wave order in LDS, plus the bias, and the same pass writes the
// bf16 hi/lo split of the scoring passes.
constexpr int kCqRows = 32;    // rows per workgroup
constexpr int kCqWaves = 4;    // d_model quarters
constexpr int kCqBatch = 2;    // k-steps of 32 whose loads are issued together
constexpr int kCqCols = 32;    // output columns per workgroup

__global__ __launch_bounds__(kCqWaves * 64) void compress_bf16_rows_kernel(
    const bf16* __restrict__ x, int64_t n, int64_t x_stride, int64_t d_model, const bf16* __restrict__ W,
    int64_t d_c, const float* __restrict__ bias, float* __restrict__ out, bf16* __restrict__ hi,
    bf16* __restrict__ lo) {
  constexpr int NI = kCqCols / 16;   // output-column tiles
  __shared__ float red[kCqWaves][kCqRows][kCqCols + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, kg = lane >> 4;
  const int64_t row0 = (int64_t)blockIdx.x * kCqRows;
  const int64_t kq = d_model / kCqWaves;
  const int64_t k0 = wave * kq + kg * 8;
  const bf16* xp[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) xp[t] = x + min(row0 + 16 * t + j, n - 1) * x_stride + k0;
  const int64_t c0 = (int64_t)blockIdx.y * kCqCols;
  const bf16* wp = W + (c0 + j) * d_model + k0;
  f32x4 acc[2][NI];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int it = 0; it < NI; ++it) acc[t][it] = f32x4{0.f, 0.f, 0.f, 0.f};
  // groups of kCqBatch k-steps, double-buffered: group g + 1 loads while
  // group g runs on the matrix cores (kq / step is even, see _ok)
  constexpr int64_t step = 32 * kCqBatch;
  bf16x8 wa0[kCqBatch][NI], xb0[kCqBatch][2], wa1[kCqBatch][NI], xb1[kCqBatch][2];
  auto load = [&](int64_t kk, bf16x8 (&wa)[kCqBatch][NI], bf16x8 (&xb)[kCqBatch][2]) {
#pragma unroll
    for (int b = 0; b < kCqBatch; ++b) {
#pragma unroll
      for (int t = 0; t < 2; ++t) xb[b][t] = *(const bf16x8*)(xp[t] + kk + 32 * b);
#pragma unroll
      for (int it = 0; it < NI; ++it) wa[b][it] = *(const bf16x8*)(wp + (int64_t)16 * it * d_model + kk + 32 * b);
    }
    __builtin_amdgcn_sched_barrier(0);   // the whole group in flight before the matrix ops
  };
  auto mma = [&](const bf16x8 (&wa)[kCqBatch][NI], const bf16x8 (&xb)[kCqBatch][2]) {
#pragma unroll
    for (int b = 0; b < kCqBatch; ++b)
#pragma unroll
      for (int it = 0; it < NI; ++it)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          acc[t][it] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[b][it], xb[b][t], acc[t][it], 0, 0, 0);
  };
  const int64_t ng = kq / step;
  load(0, wa0, xb0);
  int64_t g = 0;
  for (; g + 2 < ng; g += 2) {
    load((g + 1) * step, wa1, xb1);
    mma(wa0, xb0);
    load((g + 2) * step, wa0, xb0);
    mma(wa1, xb1);
  }
  load((g + 1) * step, wa1, xb1);
  mma(wa0, xb0);
  mma(wa1, xb1);
  // lane: row 16 t + j, output columns 16 it + 4 kg + 0..3
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int it = 0; it < NI; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][16 * t + j][16 * it + 4 * kg + r] = acc[t][it][r];
  __syncthreads();
  for (int idx = threadIdx.x; idx < kCqRows * kCqCols; idx += kCqWaves * 64) {
    const int rr = idx / kCqCols, c = idx % kCqCols;
    const int64_t orow = row0 + rr;
    if (orow >= n) continue;
    float v = ((red[0][rr][c] + red[1][rr][c]) + red[2][rr][c]) + red[3][rr][c];
    if (bias) v += bias[c0 + c];
    const int64_t o = orow * d_c + c0 + c;
    out[o] = v;
    const bf16 hv = (bf16)v;
    hi[o] = hv;
    lo[o] = (bf16)(v - (float)hv);
  }
}

bool compress_bf16_rows_ok(int64_t n, int64_t d_model, int64_t d_c) {
  // whole, even numbers of load groups per wave quarter
  return n >= 64 && d_c % kCqCols == 0 && d_c <= 4096 && d_model % (kCqWaves * 32 * kCqBatch * 2) == 0;
}

hipError_t launch_compress_bf16_rows(const void* x, int64_t n, int64_t x_stride, int64_t d_model, const void* W,
                                     int64_t d_c, const float* bias, float* out, bf16* hi, bf16* lo,
                                     hipStream_t s) {
  dim3 grid((unsigned)cdiv(n, kCqRows), (unsigned)(d_c / kCqCols));
  hipLaunchKernelGGL(compress_bf16_rows_kernel, grid, dim3(kCqWaves * 64), 0, s, (const bf16*)x, n, x_stride,
                     d_model, (const bf16*)W, d_c, bias, out, hi, lo);
  return hipGetLastError();
}

int compress_splits(int64_t n, int64_t d_model, int64_t d_c) {
  // about 2048 waves (two per SIMD; 4096 and 8192 measured slower, 1024 the
  // same, 512 much slower at 2048 rows x 4096 -> 128), chunks of at least 64 k
  const int64_t waves = cdiv(n, 16) * cdiv(d_c, kCmpCols);
  int64_t ns = cdiv(2048, waves);
  const int64_t max_ns = d_model / 64 > 0 ? d_model / 64 : 1;
  if (ns > max_ns) ns = max_ns;
  if (ns < 1) ns = 1;
  return (int)ns;
}

hipError_t launch_compress_partial(const void* x, int64_t n, int64_t x_stride, int64_t d_model,
                                   bool x_bf16, const void* W, bool w_bf16, int64_t d_c, int nsplit,
                                   double* partial, hipStream_t s) {
  const int64_t k_per_split = cdiv(d_model / 32, nsplit) * 32;
  if (n <= kCmpColRows && d_c % 16 == 0) {
    dim3 grid((unsigned)cdiv(n, 16), (unsigned)cdiv(d_c, 64), (unsigned)nsplit);
    if (x_bf16 && w_bf16)
      hipLaunchKernelGGL((compress_partial_cols_kernel<bf16, bf16>), grid, dim3(256), 0, s, (const bf16*)x, n,
                         x_stride, d_model, (const bf16*)W, d_c, k_per_split, partial);
    else if (!x_bf16 && !w_bf16)
      hipLaunchKernelGGL((compress_partial_cols_kernel<float, float>), grid, dim3(256), 0, s, (const float*)x, n,
                         x_stride, d_model, (const float*)W, d_c, k_per_split, partial);
    else if (x_bf16)
      hipLaunchKernelGGL((compress_partial_cols_kernel<bf16, float>), grid, dim3(256), 0, s, (const bf16*)x, n,
                         x_stride, d_model, (const float*)W, d_c, k_per_split, partial);
    else
      hipLaunchKernelGGL((compress_partial_cols_kernel<float, bf16>), grid, dim3(256), 0, s, (const float*)x, n,
                         x_stride, d_model, (const bf16*)W, d_c, k_per_split, partial);
    return hipGetLastError();
  }
  dim3 grid((unsigned)cdiv(n, kCmpRows), (unsigned)cdiv(d_c, kCmpCols), (unsigned)nsplit);
  if (x_bf16 && w_bf16)
    hipLaunchKernelGGL((compress_partial_kernel<bf16, bf16>), grid, dim3(256), 0, s, (const bf16*)x, n,
                       x_stride, d_model, (const bf16*)W, d_c, k_per_split, partial);
  else if (!x_bf16 && !w_bf16)
    hipLaunchKernelGGL((compress_partial_kernel<float, float>), grid, dim3(256), 0, s, (const float*)x,
                       n, x_stride, d_model, (const float*)W, d_c, k_per_split, partial);
  else if (x_bf16)
    hipLaunchKernelGGL((compress_partial_kernel<bf16, float>), grid, dim3(256), 0, s, (const bf16*)x, n,
                       x_stride, d_model, (const float*)W, d_c, k_per_split, partial);
  else
    hipLaunchKernelGGL((compress_partial_kernel<float, bf16>), grid, dim3(256), 0, s, (const float*)x,
                       n, x_stride, d_model, (const bf16*)W, d_c, k_per_split, partial);
  return hipGetLastError();
}

hipError_t launch_compress_finalize(const double* partial, int nsplit, int64_t n, int64_t d_c,
                                    const float* bias, void* out, int64_t out_stride, int kind,
                                    bf16* hi, bf16* lo, hipStream_t s) {
  const int64_t total = n * d_c;
  hipLaunchKernelGGL(compress_finalize_kernel, dim3((unsigned)cdiv(total, 256)), dim3(256), 0, s,
                     partial, nsplit, n, d_c, bias, out, out_stride, kind, hi, lo);
  return hipGetLastError();
}

}  // namespace qat
