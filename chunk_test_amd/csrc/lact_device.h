// Device helpers shared by the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lact {

__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// float -> bfloat16, round to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <bool BF16>
__device__ __forceinline__ float load_io(const void* base, int64_t i) {
  if constexpr (BF16) {
    return bf16_to_f32(static_cast<const uint16_t*>(base)[i]);
  } else {
    return static_cast<const float*>(base)[i];
  }
}

template <bool BF16>
__device__ __forceinline__ void store_io(void* base, int64_t i, float v) {
  if constexpr (BF16) {
    static_cast<uint16_t*>(base)[i] = f32_to_bf16(v);
  } else {
    static_cast<float*>(base)[i] = v;
  }
}

// logistic function without overflow for either sign (full-precision expf)
__device__ __forceinline__ float sigmoid_f(float z) {
  if (z >= 0.f) return 1.f / (1.f + expf(-z));
  float e = expf(z);
  return e / (1.f + e);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// sum over aligned groups of `width` lanes (a power of two <= 64)
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int off = width >> 1; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace lact
