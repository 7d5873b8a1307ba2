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

// The value that lane (lane ^ M) of the wave holds, M = 1, 2, 4, 8, 16 or
// 32, by VALU cross-lane moves rather than an LDS permute: DPP quad
// permutes (1, 2) and row rotations (4: one rotation each way, 8: half a
// row) inside each 16-lane row, and the row-swap permutes across rows (16,
// 32). Every lane of the wave must be active.
template <int M>
__device__ inline uint32_t lane_xor_bits(uint32_t x) {
  static_assert(M == 1 || M == 2 || M == 4 || M == 8 || M == 16 || M == 32, "lane mask");
  const int lane = threadIdx.x & (kWave - 1);
  const int xi = int(x);
  if constexpr (M == 1) {
    return uint32_t(__builtin_amdgcn_mov_dpp(xi, 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
  } else if constexpr (M == 2) {
    return uint32_t(__builtin_amdgcn_mov_dpp(xi, 0x4E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
  } else if constexpr (M == 4) {
    const int from_below = __builtin_amdgcn_mov_dpp(xi, 0x124, 0xF, 0xF, false);  // row_ror:4, lane - 4
    const int from_above = __builtin_amdgcn_mov_dpp(xi, 0x12C, 0xF, 0xF, false);  // row_ror:12, lane + 4
    return uint32_t((lane & 4) ? from_below : from_above);
  } else if constexpr (M == 8) {
    return uint32_t(__builtin_amdgcn_mov_dpp(xi, 0x128, 0xF, 0xF, false));  // row_ror:8
  } else if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);  // [0]: even rows copied up
    return (lane & 16) ? r[0] : r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);  // [0]: low half copied up
    return (lane & 32) ? r[0] : r[1];
  }
}

// Runtime mask: the switch folds away where the mask is a constant after
// unrolling (the butterfly loops over 32, 16, ..., 1).
__device__ inline uint32_t lane_xor_bits(uint32_t x, int m) {
  switch (m) {
    case 1: return lane_xor_bits<1>(x);
    case 2: return lane_xor_bits<2>(x);
    case 4: return lane_xor_bits<4>(x);
    case 8: return lane_xor_bits<8>(x);
    case 16: return lane_xor_bits<16>(x);
    case 32: return lane_xor_bits<32>(x);
    default: return uint32_t(__shfl_xor(int(x), m, kWave));
  }
}

// Sum of an int over the wave, every lane receiving it.
__device__ inline int wave_sum(int v) {
  v += int(lane_xor_bits<32>(uint32_t(v)));
  v += int(lane_xor_bits<16>(uint32_t(v)));
  v += int(lane_xor_bits<8>(uint32_t(v)));
  v += int(lane_xor_bits<4>(uint32_t(v)));
  v += int(lane_xor_bits<2>(uint32_t(v)));
  v += int(lane_xor_bits<1>(uint32_t(v)));
  return v;
}

__device__ inline int lane_xor(int v, int m) { return int(lane_xor_bits(uint32_t(v), m)); }
__device__ inline uint32_t lane_xor(uint32_t v, int m) { return lane_xor_bits(v, m); }
__device__ inline float lane_xor(float v, int m) { return __uint_as_float(lane_xor_bits(__float_as_uint(v), m)); }
__device__ inline double lane_xor(double v, int m) {
  const uint64_t b = uint64_t(__double_as_longlong(v));
  const uint64_t lo = lane_xor_bits(uint32_t(b), m), hi = lane_xor_bits(uint32_t(b >> 32), m);
  return __longlong_as_double((long long)((hi << 32) | lo));
}

__device__ inline double shfl_xor_d(double v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

}  // namespace tv
