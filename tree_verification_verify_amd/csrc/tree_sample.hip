// Multi-step speculative sampling over a draft tree (the verification walk).
//
// Rules: greedy exact match at T = 0 and recursive rejection sampling without
// replacement at T > 0 (survey page, Taxonomy rules (a) and (c); SpecInfer's
// residual-renormalising walk in its Timeline section), with the sibling
// proposals rebuilt from the shared draft logits and the sibling draw order
// (TreeSpark §1, §3.3 and Proposition 1), and one correction or bonus token
// at the stop node (TreeSpark §3.2 step 3).
//
// Design (gfx950):
//  * One team of W workgroups per request, all on one XCD (so team traffic
//    stays in that XCD's L2); the team splits the vocabulary into W slices,
//    so every vocab-wide reduction is W-way parallel. Members publish
//    partials and meet at a device-scope counter (bounded spin; the launch
//    is cooperative when W > 1, so every member is resident). Partials are
//    combined by every member in the same fixed order, so all members take
//    bit-identical decisions without a broadcast.
//  * No residual vector is stored. After rejecting siblings x_1..x_j the
//    residual is max(p - a q, 0) / B with scalars a_{j+1} = a_j + B_j / S_j,
//    B_{j+1} = sum_y max(p(y) - a_{j+1} q(y), 0), S_j = 1 - sum_{i<j} q(x_i)
//    (a rejected token's residual is already 0, so removing it from the
//    proposal is implicit). Each rejection costs one vocab-wide pass over
//    the two logit rows. The per-slice sums of that pass (or of p, at a leaf)
//    locate the slice of the correction/bonus draw, so the draw rescans one
//    slice only.
//  * Arithmetic is fp64 (logits widened exactly). exp uses Tang's table
//    method (2^(j/64) table in LDS, degree-5 polynomial, ~1 ulp), about half
//    the instructions of the library routine. Decisions therefore agree with
//    an fp64 reference except within ~1e-12 of a threshold.
//  * Sweeps keep 8 independent 16-byte loads per thread in flight.
//  * T = 0 requests: the team splits the rows; argmax (lowest index on ties)
//    of every row, then the exact-match flags; no draft logits are read.
#include <math.h>

#include "tv_device.hpp"
#include "tv_internal.hpp"

namespace tv {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxTeam = 16;             // members per team (one XCD holds a team)
constexpr int kUnroll = 4;               // float4 loads per row per step of a two-row sweep
constexpr uint32_t kSpinLimit = 1u << 25;

struct SampleParams {
  const float* t;
  const float* d;
  const int32_t* tokens;
  const int32_t* node_indptr;
  const int32_t* parent;
  const float* temperature;
  const float* uniforms;
  int8_t* flag;
  int32_t* next_token;
  uint32_t* status;
  uint32_t* team_ctr;
  double* part;
  int B, V, W, max_nodes, part_stride;
};

// ---------------------------------------------------------------------------
// exp(a) for a <= 0 in fp64: a = (64 k + j) ln2/64 + r, |r| <= ln2/128,
// e^a = 2^k * 2^(j/64) * P(r) with P the degree-5 Taylor polynomial
// (remainder below 2^-53 on that interval). tbl[j] = 2^(j/64).
constexpr double kInvLn2x64 = 92.33248261689366;
constexpr double kLn2by64Hi = 0.01083042469326756;  // low mantissa bits zero: n*hi exact
constexpr double kLn2by64Lo = 2.9815858269852933e-12;

__device__ inline double exp_nonpos(double a, const double* tbl) {
  a = fmax(a, -746.0);  // -inf and anything below underflow to 0 through ldexp
  const double n = rint(a * kInvLn2x64);
  const double r = fma(-n, kLn2by64Lo, fma(-n, kLn2by64Hi, a));
  double p = fma(r, 1.0 / 120.0, 1.0 / 24.0);
  p = fma(p, r, 1.0 / 6.0);
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  const int ni = int(n);
  return ldexp(tbl[ni & 63] * p, ni >> 6);
}

// ---------------------------------------------------------------------------
// Team synchronisation.

struct Team {
  uint32_t* ctr;
  uint32_t target;
  int W;
  int member;
  int phase;
  double* part;   // this team's partial area: [2 parities][W][part_stride]
  int stride;
  uint32_t* status;
};

__device__ inline double* member_slot(Team& tm, int member) {
  return tm.part + (size_t(tm.phase & 1) * tm.W + member) * tm.stride;
}

// Partials travel through device-coherent (agent-scope) atomic stores and
// loads, which bypass the non-coherent caches; so the barrier needs no L2
// write-back or invalidate, only ordering: a member's partial stores
// complete before its counter increment (release at workgroup scope is a
// wait for them), and no partial is read before the counter says all
// members have arrived.
__device__ inline void put_partial(double* slot, int k, double v) {
  __hip_atomic_store(slot + k, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline double get_partial(const double* slot, int k) {
  return __hip_atomic_load(const_cast<double*>(slot) + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// All K partials of every member for the current phase, loaded in parallel
// (one device-coherent load per thread) into LDS s_part[w * K + k].
__device__ void gather_partials(Team& tm, int K, double* s_part) {
  for (int i = threadIdx.x; i < tm.W * K; i += blockDim.x) {
    const int w = i / K;
    s_part[i] = get_partial(tm.part + (size_t(tm.phase & 1) * tm.W + w) * tm.stride, i - w * K);
  }
  __syncthreads();
}

// All members have published their partial for the current phase.
__device__ void team_sync(Team& tm) {
  __syncthreads();
  if (tm.W > 1) {
    tm.target += uint32_t(tm.W);
    if (threadIdx.x == 0) {
      __hip_atomic_fetch_add(tm.ctr, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      uint32_t spins = 0;
      while (__hip_atomic_load(tm.ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < tm.target) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > kSpinLimit) {
          raise_status(tm.status, TV_DEV_TIMEOUT);
          break;
        }
      }
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
    __syncthreads();
  }
}

// Leave the counter at zero: the last member to leave resets it. No member
// waits after this point, so the reset cannot strand anyone.
__device__ void team_exit(Team& tm) {
  __syncthreads();
  if (tm.W > 1 && threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(tm.ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == tm.target + uint32_t(tm.W) - 1u)
      __hip_atomic_store(tm.ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------------------
// Block reductions (fixed order: wave shuffles, then waves in index order).

__device__ inline double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += shfl_xor_d(v, off);
  return __shfl(v, 0, kWave);
}

__device__ inline double block_sum(double v, double* sh) {
  v = wave_sum(v);
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & 63) == 0) sh[wave] = v;
  __syncthreads();
  double tot = 0.0;
  for (int w = 0; w < kWaves; ++w) tot += sh[w];
  __syncthreads();
  return tot;
}

// Block-wide (max, sum of exp(x - max)) of per-thread pairs: the maximum is
// reduced first (shuffles only), then every sum is rescaled to it with one
// exp and the sums are added in a fixed order.
__device__ inline void block_ms(double& m, double& s, double* sh, const double* tbl) {
  double M = m;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmax(M, shfl_xor_d(M, off));
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & 63) == 0) sh[wave] = M;
  __syncthreads();
  M = sh[0];
  for (int w = 1; w < kWaves; ++w) M = fmax(M, sh[w]);
  __syncthreads();
  double v = (M == -INFINITY || m == -INFINITY) ? 0.0 : s * exp_nonpos(m - M, tbl);
  v = block_sum(v, sh);
  m = M;
  s = v;
}

// argmax with the lowest index on ties.
__device__ inline void am_combine(float& v, int& i, float v2, int i2) {
  const bool take = v2 > v || (v2 == v && i2 < i);
  v = take ? v2 : v;
  i = take ? i2 : i;
}

// ---------------------------------------------------------------------------
// Vocabulary sweeps over [lo, hi) of one or two rows. Each step issues
// kUnroll 16-byte loads per row per thread before using any of them; then
// f(t, d, y, valid) sees every element once (d = 0 when only one row is
// read). Indices past hi are clamped to a valid address and passed with
// valid = false, so the loop body never branches. lo is a multiple of 4 in
// the vectorised form (rows are 16-byte aligned when V % 4 == 0).
template <bool TWO, class F>
__device__ inline void sweep(const float* tr, const float* dr, int lo, int hi, bool vec4, F&& f) {
  constexpr int kUnroll = TWO ? 4 : 8;  // 8 independent 16-byte loads per thread either way
  if (vec4) {
    const float4* t4 = reinterpret_cast<const float4*>(tr + lo);
    const float4* d4 = reinterpret_cast<const float4*>(dr + lo);
    const int n4 = (hi - lo) >> 2;
    for (int base = threadIdx.x; base < n4; base += kUnroll * kThreads) {
      float4 tv[kUnroll], dv[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int i = min(base + u * kThreads, n4 - 1);
        tv[u] = t4[i];
        if (TWO) dv[u] = d4[i];
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int i = base + u * kThreads;
        const bool ok = i < n4;
        const int y = lo + 4 * i;
        f(tv[u].x, TWO ? dv[u].x : 0.f, y, ok);
        f(tv[u].y, TWO ? dv[u].y : 0.f, y + 1, ok);
        f(tv[u].z, TWO ? dv[u].z : 0.f, y + 2, ok);
        f(tv[u].w, TWO ? dv[u].w : 0.f, y + 3, ok);
      }
    }
  } else {
    for (int base = lo + threadIdx.x; base < hi; base += kUnroll * kThreads) {
      float tv[kUnroll], dv[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int y = min(base + u * kThreads, hi - 1);
        tv[u] = tr[y];
        if (TWO) dv[u] = dr[y];
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int y = base + u * kThreads;
        f(tv[u], TWO ? dv[u] : 0.f, y, y < hi);
      }
    }
  }
}

// Per-thread (max, sum of exp(x/T - max)) of both rows over [lo, hi): every
// step loads 4 float4 per row, raises the running maxima once from the
// step's own maxima (one rescale), then adds the step's terms. Tail
// elements are masked to -inf, so nothing branches per element.
__device__ inline void slice_stats(const float* tr, const float* dr, int lo, int hi, bool vec4,
                                   double invT, const double* tbl, double& mt, double& st,
                                   double& md, double& sd, bool& bad) {
  constexpr int U = 4;
  auto step = [&](float (&a)[4 * U], float (&b)[4 * U]) {
    float smt = -INFINITY, smd = -INFINITY;
#pragma unroll
    for (int k = 0; k < 4 * U; ++k) {
      smt = fmaxf(smt, a[k]);
      smd = fmaxf(smd, b[k]);
    }
    const double nmt = fmax(mt, double(smt) * invT), nmd = fmax(md, double(smd) * invT);
    st = mt == -INFINITY ? 0.0 : st * exp_nonpos(mt - nmt, tbl);
    sd = md == -INFINITY ? 0.0 : sd * exp_nonpos(md - nmd, tbl);
    mt = nmt;
    md = nmd;
#pragma unroll
    for (int k = 0; k < 4 * U; ++k) {
      st += exp_nonpos(fma(double(a[k]), invT, -mt), tbl);
      sd += exp_nonpos(fma(double(b[k]), invT, -md), tbl);
    }
  };
  if (vec4) {
    const float4* t4 = reinterpret_cast<const float4*>(tr + lo);
    const float4* d4 = reinterpret_cast<const float4*>(dr + lo);
    const int n4 = (hi - lo) >> 2;
    for (int base = threadIdx.x; base < n4; base += U * kThreads) {
      float4 tv[U], dv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = min(base + u * kThreads, n4 - 1);
        tv[u] = t4[i];
        dv[u] = d4[i];
      }
      float a[4 * U], b[4 * U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool ok = base + u * kThreads < n4;
        const float ta[4] = {tv[u].x, tv[u].y, tv[u].z, tv[u].w};
        const float da[4] = {dv[u].x, dv[u].y, dv[u].z, dv[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bad |= ok && (!isfinite(ta[e]) || !isfinite(da[e]));
          a[4 * u + e] = ok ? ta[e] : -INFINITY;
          b[4 * u + e] = ok ? da[e] : -INFINITY;
        }
      }
      step(a, b);
    }
  } else {
    for (int base = lo + threadIdx.x; base < hi; base += 4 * U * kThreads) {
      float a[4 * U], b[4 * U];
#pragma unroll
      for (int k = 0; k < 4 * U; ++k) {
        const int y = base + k * kThreads;
        const int yc = min(y, hi - 1);
        const float t = tr[yc], d = dr[yc];
        const bool ok = y < hi;
        bad |= ok && (!isfinite(t) || !isfinite(d));
        a[k] = ok ? t : -INFINITY;
        b[k] = ok ? d : -INFINITY;
      }
      step(a, b);
    }
  }
}

// Residual weight max(p(y) - a q(y), 0) with p(y) = exp(t/T - Mt)/Zt and
// q(y) = exp(d/T - Md)/Zd (plain p(y) when a == 0; the draft row is then
// not needed).
struct Resid {
  double invT, Mt, invZt, Md, invZd, a;
  __device__ inline double p(float t, const double* tbl) const {
    return exp_nonpos(fma(double(t), invT, -Mt), tbl) * invZt;
  }
  __device__ inline double q(float d, const double* tbl) const {
    return exp_nonpos(fma(double(d), invT, -Md), tbl) * invZd;
  }
  __device__ inline double w(float t, float d, const double* tbl) const {
    const double r = p(t, tbl) - a * q(d, tbl);  // a == 0: plain p (d is not needed)
    return r > 0.0 ? r : 0.0;
  }
};

// Smallest y in [lo, hi) where the running sum of weights passes thr
// (ascending token id), searched by the whole block. Each wave owns a
// contiguous quarter of [lo, hi) and sums it in blocks of 64 x 8 tokens
// (8 loads per lane in flight); the quarter holding thr is then scanned
// block by block with an in-order prefix over the block's tokens. Falls
// back to the last token with positive weight. Result in *s_y.
__device__ void slice_search(const float* tr, const float* dr, int lo, int hi, const Resid& R,
                             double thr, const double* tbl, double* sh, int* s_y) {
  constexpr int K = 8;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x / kWave;
  const int n = hi - lo;
  int per = (n + kWaves - 1) / kWaves;
  per = (per + 64 * K - 1) / (64 * K) * (64 * K);
  const int cb = min(hi, lo + wave * per), ce = min(hi, cb + per);
  // weights of block [base, base + 64K): element k of lane l is y = base + 64k + l
  auto block_w = [&](int base, double* w) {
    float tv[K], dv[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int y = min(base + 64 * k + lane, hi - 1);
      tv[k] = tr[y];
      dv[k] = dr[y];
    }
#pragma unroll
    for (int k = 0; k < K; ++k) w[k] = base + 64 * k + lane < ce ? R.w(tv[k], dv[k], tbl) : 0.0;
  };
  double run = 0.0;
  for (int base = cb; base < ce; base += 64 * K) {
    double w[K];
    block_w(base, w);
    double ls = 0.0;
#pragma unroll
    for (int k = 0; k < K; ++k) ls += w[k];
    run += wave_sum(ls);
  }
  if (lane == 0) sh[wave] = run;
  __syncthreads();
  int fw = -1, last_w = -1;
  double pre = 0.0, fpre = 0.0, last_pre = 0.0;
  for (int w = 0; w < kWaves; ++w) {
    const double cw = sh[w];
    if (cw > 0.0) {
      last_w = w;
      last_pre = pre;
    }
    if (fw < 0 && pre <= thr && thr < pre + cw) {
      fw = w;
      fpre = pre;
    }
    pre += cw;
  }
  const bool past_end = fw < 0;  // rounding put thr past the end
  if (past_end) {
    fw = last_w;
    fpre = last_pre;
  }
  __syncthreads();
  if (wave == fw) {
    const double local = thr - fpre;
    double acc = 0.0;
    int found = -1, last_pos = -1;
    for (int base = cb; base < ce && found < 0; base += 64 * K) {
      double w[K];
      block_w(base, w);
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const unsigned long long posmask = __ballot(w[k] > 0.0);
        if (posmask) last_pos = base + 64 * k + 63 - __clzll(posmask);
        double incl = w[k];
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const double o = __shfl_up(incl, off, kWave);
          if (lane >= off) incl += o;
        }
        const unsigned long long hit = __ballot(!past_end && acc + incl > local && w[k] > 0.0);
        if (found < 0 && hit) found = base + 64 * k + __ffsll(static_cast<long long>(hit)) - 1;
        acc += __shfl(incl, 63, kWave);
      }
    }
    if (found < 0) found = last_pos;
    if (lane == 0) *s_y = found < 0 ? lo : found;
  }
  if (fw < 0 && threadIdx.x == 0) *s_y = lo;
  __syncthreads();
}

// Next child of v after row `after` (children in ascending row = draw
// order), found by wave 0 with a ballot; -1 when none. Broadcast via LDS.
__device__ int next_child(const int* par, int N, int v, int after, int* s_c) {
  if (threadIdx.x < kWave) {
    int found = -1;
    for (int base = after + 1; base < N && found < 0; base += kWave) {
      const int i = base + threadIdx.x;
      const unsigned long long m = __ballot(i < N && par[i] == v);
      if (m) found = base + __ffsll(static_cast<long long>(m)) - 1;
    }
    if (threadIdx.x == 0) *s_c = found;
  }
  __syncthreads();
  const int c = *s_c;
  __syncthreads();
  return c;
}

__global__ __launch_bounds__(kThreads) void sample_kernel(SampleParams p) {
  __shared__ double tbl[64];
  __shared__ double sh[2 * kWaves];
  __shared__ double s_slice[kMaxTeam];
  __shared__ double s_part[4 * kMaxTeam];
  __shared__ float shv[kWaves];
  __shared__ int shi[kWaves];
  __shared__ int s_int;

  // Team placement: block b runs on XCD b % 8; the W members of a team are
  // consecutive slots of one XCD.
  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  const int r = (slot / p.W) * 8 + xcd;
  const int member = slot - (slot / p.W) * p.W;
  if (r >= p.B) return;  // padding block: belongs to no team

  for (int j = threadIdx.x; j < 64; j += kThreads) tbl[j] = exp2(double(j) / 64.0);

  Team tm;
  tm.ctr = p.team_ctr + r;
  tm.target = 0;
  tm.W = p.W;
  tm.member = member;
  tm.phase = 0;
  tm.part = p.part + size_t(r) * 2 * p.W * p.part_stride;
  tm.stride = p.part_stride;
  tm.status = p.status;

  const int nbeg = p.node_indptr[r];
  const int N = p.node_indptr[r + 1] - nbeg;
  const int V = p.V;
  const float T = p.temperature[r];
  if (N <= 0 || N > p.max_nodes) {
    if (N != 0 && threadIdx.x == 0 && member == 0) raise_status(p.status, TV_DEV_SHAPE);
    return;  // uniform for the whole team: nobody waits on anybody
  }
  const int* par = p.parent + nbeg;
  const int* tok = p.tokens + nbeg;
  const bool vec4 = (V & 3) == 0;
  __syncthreads();  // table ready

  if (!(T >= 0.f) || (T > 0.f && p.d == nullptr)) {
    if (member == 0) {
      if (threadIdx.x == 0) raise_status(p.status, TV_DEV_LOGITS);
      for (int i = threadIdx.x; i < N; i += kThreads) {
        p.flag[nbeg + i] = i == 0 ? 1 : 0;
        p.next_token[nbeg + i] = -1;
      }
    }
    return;
  }

  if (T == 0.f) {
    // Greedy exact match: argmax of every row, then the match flags.
    for (int i = member; i < N; i += p.W) {
      const float* row = p.t + size_t(nbeg + i) * V;
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      bool bad = false;
      sweep<false>(row, row, 0, V, vec4, [&](float t, float, int y, bool ok) {
        bad |= ok && !isfinite(t);
        const bool take = ok && t > bv;  // ascending y per thread: ties keep the first
        bv = take ? t : bv;
        bi = take ? y : bi;
      });
      if (bad) raise_status(p.status, TV_DEV_LOGITS);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const float v2 = __shfl_xor(bv, off, kWave);
        const int i2 = __shfl_xor(bi, off, kWave);
        am_combine(bv, bi, v2, i2);
      }
      const int wave = threadIdx.x / kWave;
      if ((threadIdx.x & 63) == 0) {
        shv[wave] = bv;
        shi[wave] = bi;
      }
      __syncthreads();
      if (threadIdx.x == 0) {
        float v = -INFINITY;
        int idx = 0x7fffffff;
        for (int w = 0; w < kWaves; ++w) am_combine(v, idx, shv[w], shi[w]);
        // device-coherent store: other members read it after the barrier
        __hip_atomic_store(p.next_token + nbeg + i, idx == 0x7fffffff ? 0 : idx, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
    }
    team_sync(tm);
    for (int i = member * kThreads + threadIdx.x; i < N; i += p.W * kThreads) {
      int8_t f = 0;
      if (i == 0) {
        f = 1;
      } else {
        const int pi = par[i];
        if (pi < 0 || pi >= i) {
          raise_status(p.status, TV_DEV_TREE);
        } else {
          const int ntp = __hip_atomic_load(p.next_token + nbeg + pi, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
          f = (tok[i] == ntp) ? 1 : 0;
        }
      }
      p.flag[nbeg + i] = f;
    }
    team_exit(tm);
    return;
  }

  // Sampled walk (T > 0).
  if (member == 0) {
    for (int i = threadIdx.x; i < N; i += kThreads) {
      p.flag[nbeg + i] = i == 0 ? 1 : 0;
      p.next_token[nbeg + i] = -1;
    }
  }
  const double invT = 1.0 / double(T);
  int slice = (V + p.W - 1) / p.W;
  slice = (slice + 3) / 4 * 4;
  const int lo = min(V, member * slice);
  const int hi = min(V, lo + slice);

  int v = 0;
  for (int depth_guard = 0; depth_guard <= N; ++depth_guard) {
    const float* trow = p.t + size_t(nbeg + v) * V;
    const float* drow = p.d + size_t(nbeg + v) * V;
    // Stats pass: (max, sum exp) of t/T and d/T over the member's slice.
    double mt = -INFINITY, st = 0.0, md = -INFINITY, sd = 0.0;
    bool bad = false;
    slice_stats(trow, drow, lo, hi, vec4, invT, tbl, mt, st, md, sd, bad);
    if (bad) raise_status(p.status, TV_DEV_LOGITS);
    block_ms(mt, st, sh, tbl);
    block_ms(md, sd, sh, tbl);
    if (threadIdx.x == 0) {
      double* ms = member_slot(tm, member);
      put_partial(ms, 0, mt);
      put_partial(ms, 1, st);
      put_partial(ms, 2, md);
      put_partial(ms, 3, sd);
    }
    team_sync(tm);
    gather_partials(tm, 4, s_part);
    double Mt = -INFINITY, Zt = 0.0, Md = -INFINITY, Zd = 0.0;
    for (int w = 0; w < p.W; ++w) {
      Mt = fmax(Mt, s_part[4 * w]);
      Md = fmax(Md, s_part[4 * w + 2]);
    }
    for (int w = 0; w < p.W; ++w) {  // fixed member order
      if (s_part[4 * w] != -INFINITY) Zt += s_part[4 * w + 1] * exp_nonpos(s_part[4 * w] - Mt, tbl);
      if (s_part[4 * w + 2] != -INFINITY) Zd += s_part[4 * w + 3] * exp_nonpos(s_part[4 * w + 2] - Md, tbl);
    }
    // Slice sums of p (for a draw at a leaf): s_w exp(m_w - Mt) / Zt.
    if (threadIdx.x < p.W) {
      const double m0 = s_part[4 * threadIdx.x], s0 = s_part[4 * threadIdx.x + 1];
      s_slice[threadIdx.x] = m0 == -INFINITY ? 0.0 : s0 * exp_nonpos(m0 - Mt, tbl) / Zt;
    }
    tm.phase++;
    __syncthreads();

    Resid R{invT, Mt, 1.0 / Zt, Md, 1.0 / Zd, 0.0};
    double B = 1.0, S = 1.0;
    int accepted = -1;
    for (int c = next_child(par, N, v, v, &s_int); c >= 0; c = next_child(par, N, v, c, &s_int)) {
      int x = tok[c];
      if (x < 0 || x >= V) {
        if (threadIdx.x == 0 && member == 0) raise_status(p.status, TV_DEV_SHAPE);
        x = 0;
      }
      const double px = R.p(trow[x], tbl);
      const double qx = R.q(drow[x], tbl);
      double pj = px - R.a * qx;
      pj = (pj > 0.0 ? pj : 0.0) / B;
      const double qj = qx / S;
      const double ratio = qj > 0.0 ? pj / qj : (pj > 0.0 ? INFINITY : 0.0);
      const double u = double(p.uniforms[2 * size_t(nbeg + c)]);
      if (u < ratio) {
        accepted = c;
        if (member == 0 && threadIdx.x == 0) p.flag[nbeg + c] = 1;
        break;
      }
      // Rejected: one residual pass at a' = a + B/S.
      Resid Rn = R;
      Rn.a = R.a + B / S;
      double part = 0.0;
      sweep<true>(trow, drow, lo, hi, vec4, [&](float t, float d, int, bool ok) {
        const double w = Rn.w(t, d, tbl);
        part += ok ? w : 0.0;
      });
      part = block_sum(part, sh);
      if (threadIdx.x == 0) put_partial(member_slot(tm, member), 0, part);
      team_sync(tm);
      gather_partials(tm, 1, s_part);
      double F = 0.0;
      for (int w = 0; w < p.W; ++w) F += s_part[w];
      if (F > 0.0) {
        R.a = Rn.a;
        B = F;
        if (threadIdx.x < p.W) s_slice[threadIdx.x] = s_part[threadIdx.x];
      }
      tm.phase++;
      S -= qx;
      __syncthreads();
    }
    if (accepted >= 0) {
      v = accepted;
      continue;
    }

    // Stop at v: inverse-CDF draw from the residual (p itself when a == 0).
    // The slice sums of the last pass locate the slice; its owner scans it.
    const double u = double(p.uniforms[2 * size_t(nbeg + v) + 1]);
    double total = 0.0;
    for (int w = 0; w < p.W; ++w) total += s_slice[w];
    const double thr = u * total;
    int finder = -1, last_w = -1;
    double pre = 0.0, base_w = 0.0, last_pre = 0.0;
    for (int w = 0; w < p.W; ++w) {
      const double sw = s_slice[w];
      if (sw > 0.0) {
        last_w = w;
        last_pre = pre;
      }
      if (finder < 0 && pre <= thr && thr < pre + sw) {
        finder = w;
        base_w = pre;
      }
      pre += sw;
    }
    if (finder < 0) {
      finder = last_w;
      base_w = last_pre;
    }
    if (finder == member) {
      slice_search(trow, drow, lo, hi, R, thr - base_w, tbl, sh, &s_int);
      if (threadIdx.x == 0) p.next_token[nbeg + v] = s_int;
    }
    break;
  }
  team_exit(tm);
}

}  // namespace

bool plan_sample(const tv_sample_desc& d, SamplePlan* out) {
  if (d.batch < 1 || d.vocab < 1 || d.max_nodes < 1 || d.max_nodes > 65536 || d.max_depth < 0)
    return false;
  SamplePlan pl{};
  pl.threads = kThreads;
  pl.part_stride = 4;
  size_t off = kHeaderBytes;
  pl.off_team_ctr = off;
  off = align256(off + size_t(d.batch) * sizeof(uint32_t));
  pl.off_part = off;
  off = align256(off + size_t(d.batch) * 2 * kMaxTeam * pl.part_stride * sizeof(double));
  pl.total_bytes = off;
  *out = pl;
  return true;
}

namespace {
int g_coop_blocks_per_cu = -1;
int g_num_cus = -1;
}  // namespace

hipError_t launch_sample(const tv_sample_desc& d, const SamplePlan& pl, const SampleArgs& a,
                         hipStream_t stream) {
  if (g_num_cus < 0) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return e;
    int per = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, reinterpret_cast<const void*>(sample_kernel),
                                                     kThreads, 0);
    if (e != hipSuccess) return e;
    g_coop_blocks_per_cu = per;
    g_num_cus = prop.multiProcessorCount;
  }
  // Team size: as many workgroups per request as stay resident (the
  // launch is cooperative), at most kMaxTeam; a team lives on one XCD.
  const long resident = long(g_coop_blocks_per_cu) * g_num_cus;
  int W = int(resident / ((d.batch + 7) / 8 * 8));
  if (W > kMaxTeam) W = kMaxTeam;
  if (W < 1) W = 1;
  auto grid_for = [&](int w) { return long((d.batch + 7) / 8) * 8 * w; };
  while (W > 1 && grid_for(W) > resident) --W;
  SampleParams p{};
  p.t = a.target;
  p.d = a.draft;
  p.tokens = a.tokens;
  p.node_indptr = a.node_indptr;
  p.parent = a.parent;
  p.temperature = a.temperature;
  p.uniforms = a.uniforms;
  p.flag = a.flag;
  p.next_token = a.next_token;
  char* ws = static_cast<char*>(a.workspace);
  p.status = reinterpret_cast<uint32_t*>(ws);
  p.team_ctr = reinterpret_cast<uint32_t*>(ws + pl.off_team_ctr);
  p.part = reinterpret_cast<double*>(ws + pl.off_part);
  p.B = d.batch;
  p.V = d.vocab;
  p.W = W;
  p.max_nodes = d.max_nodes;
  p.part_stride = pl.part_stride;
  const dim3 grid(unsigned(grid_for(W))), block(kThreads);
  if (W == 1) {
    hipLaunchKernelGGL(sample_kernel, grid, block, 0, stream, p);
    return hipGetLastError();
  }
  void* args[] = {&p};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(sample_kernel), grid, block,
                                    args, 0, stream);
}

}  // namespace tv
