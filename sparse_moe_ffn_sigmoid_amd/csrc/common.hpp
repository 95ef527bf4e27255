// Shared device helpers for the MI355X (gfx950) kernels of the latent MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_mi355x.h"

#define MOE_WAVE 64

#define MOE_HIP_CHECK(expr)                          \
  do {                                               \
    hipError_t _e = (expr);                          \
    if (_e != hipSuccess) return MOE_EHIP;           \
  } while (0)

#define MOE_LAUNCH_CHECK()                           \
  do {                                               \
    if (hipGetLastError() != hipSuccess) return MOE_EHIP; \
  } while (0)

namespace moe {

typedef uint16_t bf16_t;

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// Round to nearest even; NaN stays NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

template <typename T>
__device__ __forceinline__ float to_f32(T v);
template <>
__device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }

template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + __expf(-z)); }

// One gradient-descent step on one value: w - lr * g as two fp32 operations,
// each rounded to nearest even (no fused multiply-add), so that every kernel
// that applies the step produces the same bits.
__device__ __forceinline__ float sgd_value(float w, float g, float lr) {
#pragma clang fp contract(off)
  const float t = lr * g;
  return w - t;
}

// tanh(x) = 1 - 2 / (e^(2x) + 1) with the hardware exponential: the limits
// are exact (e^(2x) overflowing gives 1, underflowing gives -1), the result
// stays in [-1, 1], and the absolute error near 0 is a few ulp of 1 -- far
// below the bf16 rounding the outputs receive.
__device__ __forceinline__ float tanh_fast(float x) {
  const float e = __expf(2.0f * x);
  return 1.0f - __fdividef(2.0f, e + 1.0f);
}

// SiTU-GLU: SiLU(4 tanh(g/4)) * 25 tanh(u/25), evaluated in fp32.
__device__ __forceinline__ float situ_glu(float g, float u) {
  const float gc = 4.0f * tanh_fast(g * 0.25f);
  const float uc = 25.0f * tanh_fast(u * 0.04f);
  return __fdividef(gc, 1.0f + __expf(-gc)) * uc;
}

__host__ __device__ __forceinline__ size_t align_up(size_t v, size_t a) {
  return (v + a - 1) / a * a;
}

// Bump allocator over a caller-provided workspace.
struct Carver {
  char* base;
  size_t off;
  explicit Carver(void* b) : base(static_cast<char*>(b)), off(0) {}
  template <typename T>
  T* take(size_t count) {
    off = align_up(off, 256);
    T* p = reinterpret_cast<T*>(base ? base + off : nullptr);
    off += count * sizeof(T);
    return p;
  }
  size_t bytes() const { return align_up(off, 256); }
};

}  // namespace moe
