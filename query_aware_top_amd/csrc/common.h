// Internal helpers shared by the HIP kernels of the library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

namespace qat {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// Round a finite double to the nearest bfloat16 (ties to even) without an
// intermediate float rounding: add half an ulp of the 45 discarded mantissa
// bits (plus the kept LSB for ties-to-even) and truncate.
__device__ __forceinline__ bf16 f64_to_bf16_rne(double x) {
  uint64_t b = (uint64_t)__double_as_longlong(x);
  uint64_t lsb = (b >> 45) & 1ull;
  b += ((1ull << 44) - 1ull) + lsb;
  b &= ~((1ull << 45) - 1ull);
  return (bf16)(float)__longlong_as_double((long long)b);   // exact from here
}

// Order-preserving map float -> uint32 (larger float, larger key).
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, kWave); }

// Combine lanes l and l ^ 32 without LDS: v_permlane32_swap exchanges the
// upper half of its first operand with the lower half of its second, so
// for (v, v) the two results hold v[l] and v[l ^ 32] in some order.
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__host__ __device__ __forceinline__ int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Workspace carving helper: 256-byte aligned regions.
struct Carver {
  char* base;
  size_t off;
  __host__ explicit Carver(void* b) : base((char*)b), off(0) {}
  template <typename T>
  __host__ T* take(size_t count) {
    off = (off + 255) & ~(size_t)255;
    T* p = base ? (T*)(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
  __host__ size_t bytes() const { return (off + 255) & ~(size_t)255; }
};

// Optional per-kernel timing with HIP events on the launch stream (enabled
// through qat_timing_enable); no-ops when disabled.
void ktimer_start(const char* name, hipStream_t s);
void ktimer_stop(const char* name, hipStream_t s);

struct KTimer {
  const char* name;
  hipStream_t s;
  KTimer(const char* n, hipStream_t st) : name(n), s(st) { ktimer_start(name, s); }
  ~KTimer() { ktimer_stop(name, s); }
};

// Kernel-level timing of the one stage chosen with qat_timing_select: that
// stage's main kernel is launched with start/stop events filled from its own
// dispatch (hipExtLaunchKernel), so no marker packets enter the stream.
bool ktimer_kernel_events(const char* name, hipEvent_t* a, hipEvent_t* b);
void ktimer_kernel_record(const char* name, hipEvent_t a, hipEvent_t b);

template <typename F, typename... Args>
inline void launch_timed(const char* name, F kernel, dim3 grid, dim3 block, uint32_t shm, hipStream_t s,
                         Args... args) {
  hipEvent_t a, b;
  if (ktimer_kernel_events(name, &a, &b)) {
    hipExtLaunchKernelGGL(kernel, grid, block, shm, s, a, b, 0, args...);
    ktimer_kernel_record(name, a, b);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, shm, s, args...);
  }
}

}  // namespace qat
