// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers:
// as easy as 1, 2, 3", SC 2011): ten rounds of two 32x32->64-bit multiplies
// with the published multipliers and Weyl key increments. Counter c, key
// (k0, k1); four 32-bit output words.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tv {

__device__ inline uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    if (i) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = uint64_t(0xD2511F53u) * c.x;
    const uint64_t p1 = uint64_t(0xCD9E8D57u) * c.z;
    c = make_uint4(uint32_t(p1 >> 32) ^ c.y ^ k0, uint32_t(p1), uint32_t(p0 >> 32) ^ c.w ^ k1,
                   uint32_t(p0));
  }
  return c;
}

}  // namespace tv
