// Drawing each expanded node's children without replacement: Gumbel-top-k.
//
// The survey page's Timeline section has Recursive Speculative Decoding draw
// tree siblings without replacement via Gumbel-Top-k; TreeSpark (§1, §3.3)
// draws siblings without replacement from the draft distribution q_T, in a
// draw order the verifier replays. For a row with draft logits d, temperature
// T and k children: the children are the k tokens of largest
// d[y]/T - ln(-ln u(y)) (T > 0) or d[y] (T = 0), in descending score, lower
// token id first on ties.
//
// u(y) comes from Philox4x32-10 (Salmon, Moraes, Dror and Shaw, SC 2011:
// ten rounds of two 32x32->64 multiplies with the published multipliers and
// Weyl key increments), counter (y/4, row, stream, 0), key (seed lo, seed hi),
// output word y%4: u = ((word >> 8) + 1/2) / 2^24, strictly inside (0, 1).
//
// One workgroup of 512 threads per row streams the row once (float4 loads,
// two ahead of the one being scored; one Philox call per float4). Each thread
// keeps its K best (score, id) in registers, sorted (K = the next power of
// two >= k). Per float4 one score bound for its four tokens (-ln u >= 1 - u
// gives g <= -ln(1 - u); the largest logit with the smallest 1 - u, one fast
// hardware log plus a margin) is tested against the wave's threshold
// (below): a wave executes per-token work when any
// lane needs it, so it is entered only for the few float4 that can enter a
// list; there each token is scored exactly (log1p for u near 1, where ln u
// loses its relative precision) and inserted. The threads' lists are merged
// by k rounds of a block argmax.
#include "tv_device.hpp"
#include "tv_internal.hpp"
#include "tv_philox.hpp"

namespace tv {

namespace {

constexpr int kSibThreads = 512;  // 8 waves: about five waves per SIMD over the rows
constexpr int kMaxChildren = 16;

struct SibParams {
  const float* logits;
  const int32_t* counts;
  const float* temperature;
  int32_t* tokens;
  uint32_t* status;
  int rows, vocab;
  uint32_t stream, key0, key1;
};

// (a, ia) ranks before (b, ib): larger score, then lower id.
__device__ inline bool before(float a, int ia, float b, int ib) {
  return a > b || (a == b && ia < ib);
}

template <int K>
__device__ inline void insert(float (&sc)[K], int (&ix)[K], float s, int y) {
  if (!before(s, y, sc[K - 1], ix[K - 1])) return;
  sc[K - 1] = s;
  ix[K - 1] = y;
#pragma unroll
  for (int j = K - 1; j > 0; --j) {
    if (before(sc[j], ix[j], sc[j - 1], ix[j - 1])) {
      const float ts = sc[j];
      sc[j] = sc[j - 1];
      sc[j - 1] = ts;
      const int ti = ix[j];
      ix[j] = ix[j - 1];
      ix[j - 1] = ti;
    }
  }
}

// The row of workgroup r with k children, each thread keeping its K >= k
// best. A token is skipped unless (an upper bound of) its score reaches the
// wave threshold: the largest K-th best over the wave's lanes, refreshed
// every 8 steps. One lane alone holds K >= k tokens at or above that value,
// so no skipped token can be among the row's k best; the threshold keeps the
// rare insertions (and the exact noise) rare for the wave, not only per lane.
template <int K>
__device__ void draw_row(const SibParams& p, int r, int k, float T, int32_t* out) {
  __shared__ float s_sc[2][kSibThreads / 64];
  __shared__ int s_ix[2][kSibThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool noisy = T > 0.f;
  const float invT = noisy ? 1.f / T : 0.f;
  const float* row = p.logits + size_t(r) * p.vocab;
  const int V = p.vocab;

  float sc[K];
  int ix[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    sc[j] = -INFINITY;
    ix[j] = 0x7fffffff;
  }
  float theta = -INFINITY;  // wave threshold
  bool bad = false;
  // Two valid thresholds, the larger kept: the largest K-th best over the
  // lanes (one lane holds K >= k tokens at or above it), and the k-th largest
  // of the lanes' best scores (k distinct lanes each hold a token at or above
  // it), found by k rounds of a wave argmax over (best, lane).
  auto refresh = [&]() __attribute__((always_inline)) {
    float t = sc[K - 1];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) t = fmaxf(t, __shfl_xor(t, o, 64));
    const float mine = sc[0];
    bool taken = false;
    float kth = -INFINITY;
    for (int i = 0; i < k; ++i) {
      float bs = taken ? -INFINITY : mine;
      int bl = taken ? 64 : lane;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float os = __shfl_xor(bs, o, 64);
        const int ol = __shfl_xor(bl, o, 64);
        if (os > bs || (os == bs && ol < bl)) {
          bs = os;
          bl = ol;
        }
      }
      taken = taken || bl == lane;
      kth = bs;
    }
    theta = fmaxf(t, kth);
  };

  // Score of token y from its logit and Philox word; bounds first.
  auto consider = [&](float d, uint32_t w, int y) __attribute__((always_inline)) {
    if (!(d == d) || d == INFINITY || d == -INFINITY) {  // NaN / Inf logits
      bad = true;
      return;
    }
    if (!noisy) {
      if (d >= theta) insert(sc, ix, d, y);
      return;
    }
    const float base = d * invT;
    const float x = (float(16777216u - (w >> 8)) - 0.5f) * (1.f / 16777216.f);  // 1 - u
    // g <= -ln(1 - u): fast log with a generous margin
    const float bound = base - __logf(x) + 1e-3f;
    if (bound < theta || !before(bound, y, sc[K - 1], ix[K - 1])) return;
    const float u = (float(w >> 8) + 0.5f) * (1.f / 16777216.f);
    const float e = u > 0.5f ? -log1pf(-x) : -logf(u);  // -ln u, accurate near u = 1
    insert(sc, ix, base - logf(e), y);
  };

  const bool vec = (V & 3) == 0 && (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
  int step = 0;
  if (vec) {
    const int n4 = V >> 2;
    const float4* row4 = reinterpret_cast<const float4*>(row);
    // the next two float4 of this thread load while the current one is scored
    const float4 zero4 = make_float4(0.f, 0.f, 0.f, 0.f);
    float4 d1 = tid < n4 ? row4[tid] : zero4;
    float4 d2 = tid + kSibThreads < n4 ? row4[tid + kSibThreads] : zero4;
    for (int c4 = tid; c4 < n4; c4 += kSibThreads) {
      const float4 d = d1;
      d1 = d2;
      d2 = c4 + 2 * kSibThreads < n4 ? row4[c4 + 2 * kSibThreads] : zero4;
      // Finite check for the four logits at once, then one test of the
      // largest score bound against the threshold: the per-token work below
      // runs only for the few float4 that can enter a list.
      bad |= !(fabsf(d.x) <= 3.4e38f) | !(fabsf(d.y) <= 3.4e38f) | !(fabsf(d.z) <= 3.4e38f) |
             !(fabsf(d.w) <= 3.4e38f);
      if (!noisy) {
        if (fmaxf(fmaxf(d.x, d.y), fmaxf(d.z, d.w)) >= theta) {
          consider(d.x, 0u, 4 * c4);
          consider(d.y, 0u, 4 * c4 + 1);
          consider(d.z, 0u, 4 * c4 + 2);
          consider(d.w, 0u, 4 * c4 + 3);
        }
      } else {
        const uint4 w = philox4x32_10(make_uint4(uint32_t(c4), uint32_t(r), p.stream, 0u), p.key0, p.key1);
        // One bound for the four tokens: the largest logit with the largest
        // noise bound (the smallest 1 - u: the largest 24-bit word), so one
        // logarithm instead of four; the per-token bounds follow if it passes.
        const uint32_t wm = max(max(w.x, w.y), max(w.z, w.w)) >> 8;
        const float xm = (float(16777216u - wm) - 0.5f) * (1.f / 16777216.f);  // smallest 1 - u
        const float bmax = fmaxf(fmaxf(d.x, d.y), fmaxf(d.z, d.w)) * invT - __logf(xm) + 1e-3f;
        if (bmax >= theta) {
          consider(d.x, w.x, 4 * c4);
          consider(d.y, w.y, 4 * c4 + 1);
          consider(d.z, w.z, 4 * c4 + 2);
          consider(d.w, w.w, 4 * c4 + 3);
        }
      }
      if ((++step & 7) == 0) refresh();
    }
  } else {
    for (int y = tid; y < V; y += kSibThreads) {
      uint32_t wy = 0;
      if (noisy) {
        const uint4 w = philox4x32_10(make_uint4(uint32_t(y >> 2), uint32_t(r), p.stream, 0u),
                                      p.key0, p.key1);
        const int q = y & 3;
        wy = q == 0 ? w.x : q == 1 ? w.y : q == 2 ? w.z : w.w;
      }
      consider(row[y], wy, y);
      if ((++step & 31) == 0) refresh();
    }
  }
  if (bad) raise_status(p.status, TV_DEV_LOGITS);

  // k rounds of a block argmax over the threads' list heads; the winner's
  // list shifts by one.
  for (int i = 0; i < k; ++i) {
    float bs = sc[0];
    int bi = ix[0];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float os = __shfl_xor(bs, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (before(os, oi, bs, bi)) {
        bs = os;
        bi = oi;
      }
    }
    const int buf = i & 1;
    if (lane == 0) {
      s_sc[buf][wave] = bs;
      s_ix[buf][wave] = bi;
    }
    __syncthreads();
    bs = s_sc[buf][0];
    bi = s_ix[buf][0];
#pragma unroll
    for (int w2 = 1; w2 < kSibThreads / 64; ++w2)
      if (before(s_sc[buf][w2], s_ix[buf][w2], bs, bi)) {
        bs = s_sc[buf][w2];
        bi = s_ix[buf][w2];
      }
    if (tid == 0) out[i] = bi < V ? bi : -1;
    if (ix[0] == bi) {  // ids are distinct: exactly one thread holds the winner
#pragma unroll
      for (int j = 0; j < K - 1; ++j) {
        sc[j] = sc[j + 1];
        ix[j] = ix[j + 1];
      }
      sc[K - 1] = -INFINITY;
      ix[K - 1] = 0x7fffffff;
    }
  }
  if (tid >= k && tid < kMaxChildren) out[tid] = -1;
}

// Two launches share the rows: the narrow kernel checks every row, writes
// the -1 padding of empty and rejected rows and draws rows with k <= 8; the
// wide one draws rows with 8 < k <= 16 (their 16-entry lists would set the
// register budget, and so the occupancy, of every row).
template <bool kWide>
__global__ __launch_bounds__(kSibThreads) void draw_siblings_kernel(SibParams p) {
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  int32_t* out = p.tokens + size_t(r) * kMaxChildren;
  const int k = p.counts[r];
  const float T = p.temperature[r];
  const bool ok = k >= 0 && k <= kMaxChildren && T >= 0.f && T != INFINITY;
  if (kWide) {
    if (ok && k > 8) draw_row<16>(p, r, k, T, out);
    return;
  }
  if (!ok) {
    if (tid == 0) raise_status(p.status, (k < 0 || k > kMaxChildren) ? TV_DEV_SHAPE : TV_DEV_LOGITS);
    if (tid < kMaxChildren) out[tid] = -1;
    return;
  }
  if (k == 0) {
    if (tid < kMaxChildren) out[tid] = -1;
    return;
  }
  // per-thread list length: the next power of two >= k
  if (k <= 1)
    draw_row<1>(p, r, k, T, out);
  else if (k <= 2)
    draw_row<2>(p, r, k, T, out);
  else if (k <= 4)
    draw_row<4>(p, r, k, T, out);
  else if (k <= 8)
    draw_row<8>(p, r, k, T, out);
}

}  // namespace

hipError_t launch_draw_siblings(int32_t rows, int32_t vocab, const float* draft_logits,
                                const int32_t* counts, const float* temperature, uint32_t stream_id,
                                uint64_t seed, int32_t* tokens, uint32_t* status,
                                hipStream_t stream) {
  SibParams p{};
  p.logits = draft_logits;
  p.counts = counts;
  p.temperature = temperature;
  p.tokens = tokens;
  p.status = status;
  p.rows = rows;
  p.vocab = vocab;
  p.stream = stream_id;
  p.key0 = uint32_t(seed);
  p.key1 = uint32_t(seed >> 32);
  hipLaunchKernelGGL(draw_siblings_kernel<false>, dim3(unsigned(rows)), dim3(kSibThreads), 0, stream, p);
  hipLaunchKernelGGL(draw_siblings_kernel<true>, dim3(unsigned(rows)), dim3(kSibThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace tv
