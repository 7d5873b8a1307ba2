// Device-side helpers shared by the tree-verification kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tree_verify.h"

namespace tv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kPage = 16;
constexpr int kWave = 64;

// Workspace header: status word at byte 0, the rest of the first 256 bytes
// reserved. Counters and partial buffers follow at 256-byte boundaries.
constexpr size_t kHeaderBytes = 256;

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

__device__ inline void raise_status(uint32_t* status, uint32_t bit) {
  if (status) atomicOr(status, bit);
}

__device__ inline float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(uint32_t(b) << 16);
}

// Round to nearest even; NaN stays a quiet NaN.
__device__ inline uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f32_to_bf16_bits(lo)) | (uint32_t(f32_to_bf16_bits(hi)) << 16);
}

template <typename T>
__device__ inline T shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

__device__ inline double shfl_xor_d(double v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

}  // namespace tv
