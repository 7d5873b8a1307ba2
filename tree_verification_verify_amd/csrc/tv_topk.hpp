// Per-thread top-K lists and a wave-level K-th largest, shared by the
// kernels that select the K best entries of a vocabulary row.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

#include "tv_device.hpp"

namespace tv {

// The K-th largest (K <= 64) of one value per lane, by a bitonic sort across
// the wave (descending, partners exchanged by VALU cross-lane moves; every
// lane must be active), read from lane K-1.
__device__ inline float wave_kth_largest(float v, int K) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int size = 2; size <= kWave; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const float o = lane_xor(v, stride);
      const bool desc = (lane & size) == 0;  // this block of `size` lanes sorts descending
      const bool low = (lane & stride) == 0;
      v = (low == desc) ? fmaxf(v, o) : fminf(v, o);
    }
  }
  return __shfl(v, K - 1, kWave);
}

// Per-thread list of the K best (value, id) seen, best first.
template <int K>
struct TopList {
  float v[K];
  int i[K];
  __device__ void init() {
#pragma unroll
    for (int j = 0; j < K; ++j) {
      v[j] = -INFINITY;
      i[j] = 0x7fffffff;
    }
  }
  // Elements arrive in ascending id, so strict comparisons keep a tie's
  // earlier (lower) id ahead.
  __device__ void insert(float x, int id) {
    if (!(x > v[K - 1])) return;
#pragma unroll
    for (int j = K - 1; j > 0; --j) {
      const bool up = x > v[j - 1];
      const bool here = !up && x > v[j];
      v[j] = up ? v[j - 1] : (here ? x : v[j]);
      i[j] = up ? i[j - 1] : (here ? id : i[j]);
    }
    if (x > v[0]) {
      v[0] = x;
      i[0] = id;
    }
  }
  __device__ void pop() {
#pragma unroll
    for (int j = 0; j + 1 < K; ++j) {
      v[j] = v[j + 1];
      i[j] = i[j + 1];
    }
    v[K - 1] = -INFINITY;
    i[K - 1] = 0x7fffffff;
  }
};

}  // namespace tv
