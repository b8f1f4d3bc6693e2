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

// Offset of element (r, c) of a rows x cols matrix (rows a multiple of 32,
// cols of 16) in the bf16 operand copy of the fast weights.  The copy is
// stored in the order the query read loads it as 32x32x16 MFMA operands:
// blocks of 32 rows x 16 columns, row-block major, each block as the 64
// 16-byte slices of its lanes (lane 32 (c / 8 % 2) + r % 32 holds the eight
// columns 16 (c / 16) + 8 (c / 8 % 2) .. +7 of row r), so a wavefront reads
// one block as 1 KiB of consecutive bytes.  Four elements c .. c + 3 with
// c % 4 == 0 stay adjacent.
__device__ __forceinline__ int64_t wb_tiled(int r, int c, int cols) {
  return ((static_cast<int64_t>(r >> 5) * (cols >> 4) + (c >> 4)) * 64 + ((c >> 3) & 1) * 32 + (r & 31)) * 8 +
         (c & 7);
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

// v from another lane of the same 16-lane row (DPP lane permutation; no LDS
// round trip): quad_perm [1,0,3,2] (xor 1), quad_perm [2,3,0,1] (xor 2),
// row_half_mirror (i <-> 7 - i within 8), row_mirror (i <-> 15 - i).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sums over aligned groups of W lanes (W a power of two <= 64) of N values
// at once, every lane of a group receiving its group's sum.  Inside a
// 16-lane row the butterfly runs on DPP moves (after the two quad steps
// every lane holds its quad's sum, the half-mirror adds the other quad of
// its half-row, the mirror the other half-row); wider groups add lane
// shuffles.  The N reductions are independent, so their latencies overlap.
template <int W, int N>
__device__ __forceinline__ void group_sums(float (&v)[N]) {
  static_assert(W >= 1 && W <= 64 && (W & (W - 1)) == 0, "group width");
  if constexpr (W >= 2) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += dpp_mov<0xB1>(v[i]);
  }
  if constexpr (W >= 4) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += dpp_mov<0x4E>(v[i]);
  }
  if constexpr (W >= 8) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += dpp_mov<0x141>(v[i]);
  }
  if constexpr (W >= 16) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += dpp_mov<0x140>(v[i]);
  }
  if constexpr (W >= 32) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += __shfl_xor(v[i], 16, 64);
  }
  if constexpr (W >= 64) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += __shfl_xor(v[i], 32, 64);
  }
}

}  // namespace lact
