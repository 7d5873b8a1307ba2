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
//  * One team of W workgroups per request; the team splits the vocabulary,
//    so every vocab-wide reduction is W-way parallel. Teams synchronise with a
//    device-scope counter (bounded spin; the launch is cooperative whenever
//    W > 1, so every member is resident). Partials are combined by every
//    member in the same fixed order, so all members take bit-identical
//    decisions without a broadcast step.
//  * No residual vector is ever stored. After rejecting siblings x_1..x_j the
//    residual is max(p - a q, 0) / B with scalars a_{j+1} = a_j + B_j / S_j,
//    B_{j+1} = sum_y max(p(y) - a_{j+1} q(y), 0), S_j = 1 - sum_{i<j} q(x_i)
//    (the drawn tokens' residual is already 0, so removing them from the
//    proposal is implicit). Each rejection therefore costs exactly one
//    vocab-wide pass over the two logit rows and a handful of scalars.
//  * Arithmetic is fp64 (logits widened exactly): exp, sums, ratios and the
//    inverse-CDF prefix sums, so decisions agree with an fp64 reference except
//    within ~1e-12 of a threshold.
//  * T = 0 requests: argmax (lowest index on ties) of every row, then the
//    exact-match flags for every node; no draft logits are read.
#include <math.h>

#include "tv_device.hpp"
#include "tv_internal.hpp"

namespace tv {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxChildren = 4096;
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

// All members have published their partial for the current phase.
__device__ void team_sync(Team& tm) {
  __syncthreads();
  if (tm.W > 1) {
    tm.target += uint32_t(tm.W);
    if (threadIdx.x == 0) {
      __threadfence();
      atomicAdd(tm.ctr, 1u);
      uint32_t spins = 0;
      while (__hip_atomic_load(tm.ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < tm.target) {
        __builtin_amdgcn_s_sleep(2);
        if (++spins > kSpinLimit) {
          raise_status(tm.status, TV_DEV_TIMEOUT);
          break;
        }
      }
    }
    __syncthreads();
    __threadfence();
  }
}

// Leave the counter at zero: the last member to leave resets it. No member
// waits after this point, so the reset cannot strand anyone.
__device__ void team_exit(Team& tm) {
  __syncthreads();
  if (tm.W > 1 && threadIdx.x == 0) {
    __threadfence();
    const uint32_t old = atomicAdd(tm.ctr, 1u);
    if (old == tm.target + uint32_t(tm.W) - 1u) atomicExch(tm.ctr, 0u);
  }
}

// Wave sum; every lane returns lane 0's value (bit-identical across lanes).
__device__ inline double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += shfl_xor_d(v, off);
  return __shfl(v, 0, kWave);
}

// Block sum in a fixed order (wave sums, then waves in index order).
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

// (max, sum of exp(x - max)) pairs.
__device__ inline void ms_combine(double& m, double& s, double m2, double s2) {
  if (m2 > m) {
    s = s * exp(m - m2) + s2;
    m = m2;
  } else if (m2 != -INFINITY) {
    s += s2 * exp(m2 - m);
  }
}

__device__ inline void wave_ms(double& m, double& s) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const double m2 = shfl_xor_d(m, off), s2 = shfl_xor_d(s, off);
    ms_combine(m, s, m2, s2);
  }
  m = __shfl(m, 0, kWave);
  s = __shfl(s, 0, kWave);
}

__device__ inline void block_ms(double& m, double& s, double* sh) {
  wave_ms(m, s);
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & 63) == 0) {
    sh[2 * wave] = m;
    sh[2 * wave + 1] = s;
  }
  __syncthreads();
  m = -INFINITY;
  s = 0.0;
  for (int w = 0; w < kWaves; ++w) ms_combine(m, s, sh[2 * w], sh[2 * w + 1]);
  __syncthreads();
}

// Online (max, sum) update with one element x.
__device__ inline void ms_push(double& m, double& s, double x) {
  if (x > m) {
    s = s * exp(m - x) + 1.0;
    m = x;
  } else {
    s += exp(x - m);
  }
}

// argmax with the lowest index on ties.
__device__ inline void am_combine(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

__device__ int block_argmax(const float* row, int V, uint32_t* status, float* shv, int* shi) {
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  bool bad = false;
  if ((V & 3) == 0) {
    const float4* r4 = reinterpret_cast<const float4*>(row);
    for (int i = threadIdx.x; i < V / 4; i += kThreads) {
      const float4 a = r4[i];
      bad |= !isfinite(a.x) || !isfinite(a.y) || !isfinite(a.z) || !isfinite(a.w);
      am_combine(bv, bi, a.x, 4 * i);
      am_combine(bv, bi, a.y, 4 * i + 1);
      am_combine(bv, bi, a.z, 4 * i + 2);
      am_combine(bv, bi, a.w, 4 * i + 3);
    }
  } else {
    for (int i = threadIdx.x; i < V; i += kThreads) {
      const float a = row[i];
      bad |= !isfinite(a);
      am_combine(bv, bi, a, i);
    }
  }
  if (bad) raise_status(status, TV_DEV_LOGITS);
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
  float v = -INFINITY;
  int idx = 0x7fffffff;
  for (int w = 0; w < kWaves; ++w) am_combine(v, idx, shv[w], shi[w]);
  __syncthreads();
  return idx == 0x7fffffff ? 0 : idx;
}

// Per-node softmax statistics of one row slice: max and sum of exp of x/T.
struct RowStats {
  double m, z;
};

__device__ void slice_stats(const float* row, int lo, int hi, double invT, bool vec4,
                            double& m, double& s, bool& bad) {
  if (vec4) {
    for (int i = lo + 4 * threadIdx.x; i < hi; i += 4 * kThreads) {
      const float4 a = *reinterpret_cast<const float4*>(row + i);
      bad |= !isfinite(a.x) || !isfinite(a.y) || !isfinite(a.z) || !isfinite(a.w);
      const double x0 = double(a.x) * invT, x1 = double(a.y) * invT;
      const double x2 = double(a.z) * invT, x3 = double(a.w) * invT;
      const double lm = fmax(fmax(x0, x1), fmax(x2, x3));
      if (lm > m) {
        s *= exp(m - lm);
        m = lm;
      }
      s += exp(x0 - m) + exp(x1 - m) + exp(x2 - m) + exp(x3 - m);
    }
  } else {
    for (int i = lo + threadIdx.x; i < hi; i += kThreads) {
      const float a = row[i];
      bad |= !isfinite(a);
      ms_push(m, s, double(a) * invT);
    }
  }
}

// Residual weight of token y: max(p(y) - a q(y), 0) with
// p(y) = exp(t_y/T - Mt)/Zt, q(y) = exp(d_y/T - Md)/Zd. With a == 0 the draft
// row is not read.
struct Resid {
  const float* trow;
  const float* drow;
  double invT, Mt, invZt, Md, invZd, a;
  __device__ inline double p(int y) const { return exp(fma(double(trow[y]), invT, -Mt)) * invZt; }
  __device__ inline double q(int y) const { return exp(fma(double(drow[y]), invT, -Md)) * invZd; }
  __device__ inline double w(int y) const {
    const double pv = p(y);
    if (a == 0.0) return pv;
    const double r = pv - a * q(y);
    return r > 0.0 ? r : 0.0;
  }
};

__device__ double slice_resid_sum(const Resid& R, int lo, int hi, bool vec4) {
  double acc = 0.0;
  if (vec4) {
    for (int i = lo + 4 * threadIdx.x; i < hi; i += 4 * kThreads) {
      const float4 tv = *reinterpret_cast<const float4*>(R.trow + i);
      const float4 dv = *reinterpret_cast<const float4*>(R.drow + i);
      const float tt[4] = {tv.x, tv.y, tv.z, tv.w};
      const float dd[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double pv = exp(fma(double(tt[e]), R.invT, -R.Mt)) * R.invZt;
        const double qv = exp(fma(double(dd[e]), R.invT, -R.Md)) * R.invZd;
        const double r = pv - R.a * qv;
        acc += r > 0.0 ? r : 0.0;
      }
    }
  } else {
    for (int i = lo + threadIdx.x; i < hi; i += kThreads) acc += R.w(i);
  }
  return acc;
}

__device__ inline int wave_chunk_begin(int lo, int hi, int wv) {
  const int n = hi - lo;
  int per = (n + kWaves - 1) / kWaves;
  per = (per + 63) / 64 * 64;
  return min(hi, lo + wv * per);
}

// Sum of residual weights over this wave's contiguous chunk, in 64-token
// steps (the same step structure the search below replays).
__device__ double wave_chunk_sum(const Resid& R, int cb, int ce) {
  const int lane = threadIdx.x & 63;
  double run = 0.0;
  for (int base = cb; base < ce; base += 64) {
    const int y = base + lane;
    const double w = (y < ce) ? R.w(y) : 0.0;
    run += wave_sum(w);
  }
  return run;
}

// Smallest token in [cb, ce) where the running sum exceeds thr (token ids
// ascending). Falls back to the last token with positive weight.
__device__ int wave_chunk_search(const Resid& R, int cb, int ce, double thr) {
  const int lane = threadIdx.x & 63;
  double run = 0.0;
  int last_pos = -1;
  for (int base = cb; base < ce; base += 64) {
    const int y = base + lane;
    const double w = (y < ce) ? R.w(y) : 0.0;
    const double step = wave_sum(w);
    const unsigned long long posmask = __ballot(w > 0.0);
    if (posmask) last_pos = base + 63 - __clzll(posmask);
    if (run + step > thr) {
      double incl = w;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const double o = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += o;
      }
      const unsigned long long hit = __ballot(run + incl > thr && w > 0.0);
      if (hit) return base + __ffsll(static_cast<long long>(hit)) - 1;
      return last_pos;
    }
    run += step;
  }
  return last_pos;
}

__global__ __launch_bounds__(kThreads) void sample_kernel(SampleParams p) {
  __shared__ double sh[2 * kWaves];
  __shared__ double sh_chunk[kWaves];
  __shared__ float shv[kWaves];
  __shared__ int shi[kWaves];
  __shared__ int s_children[kMaxChildren];
  __shared__ int s_nchild;

  const int r = blockIdx.x / p.W;
  const int member = blockIdx.x - r * p.W;
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
  const bool shape_ok = N > 0 && N <= p.max_nodes && N <= kMaxChildren;
  if (!shape_ok) {
    if (N != 0 && threadIdx.x == 0 && member == 0) raise_status(p.status, TV_DEV_SHAPE);
    return;  // uniform for the whole team: nobody waits on anybody
  }
  const int* par = p.parent + nbeg;
  const int* tok = p.tokens + nbeg;

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
      const int y = block_argmax(p.t + size_t(nbeg + i) * V, V, p.status, shv, shi);
      if (threadIdx.x == 0) p.next_token[nbeg + i] = y;
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
          f = (tok[i] == p.next_token[nbeg + pi]) ? 1 : 0;
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
  const bool vec4 = (V & 3) == 0;
  const int wv = threadIdx.x / kWave;
  const int cb = wave_chunk_begin(lo, hi, wv);
  const int ce = wave_chunk_begin(lo, hi, wv + 1);

  int v = 0;
  for (int depth_guard = 0; depth_guard <= N; ++depth_guard) {
    const float* trow = p.t + size_t(nbeg + v) * V;
    const float* drow = p.d + size_t(nbeg + v) * V;
    // Stats pass: (max, sum exp) of t/T and d/T over the team's slices.
    double mt = -INFINITY, st = 0.0, md = -INFINITY, sd = 0.0;
    bool bad = false;
    slice_stats(trow, lo, hi, invT, vec4, mt, st, bad);
    slice_stats(drow, lo, hi, invT, vec4, md, sd, bad);
    if (bad) raise_status(p.status, TV_DEV_LOGITS);
    block_ms(mt, st, sh);
    block_ms(md, sd, sh);
    if (threadIdx.x == 0) {
      double* slot = member_slot(tm, member);
      slot[0] = mt;
      slot[1] = st;
      slot[2] = md;
      slot[3] = sd;
    }
    team_sync(tm);
    double Mt = -INFINITY, Zt = 0.0, Md = -INFINITY, Zd = 0.0;
    for (int w = 0; w < p.W; ++w) {
      const double* slot = member_slot(tm, w);
      ms_combine(Mt, Zt, slot[0], slot[1]);
      ms_combine(Md, Zd, slot[2], slot[3]);
    }
    tm.phase++;

    // Children of v in draw order.
    if (threadIdx.x < kWave) {
      int cnt = 0;
      for (int base = v + 1; base < N; base += kWave) {
        const int i = base + threadIdx.x;
        const bool is_child = i < N && par[i] == v;
        const unsigned long long m = __ballot(is_child);
        if (is_child) s_children[cnt + __popcll(m & ((1ull << threadIdx.x) - 1ull))] = i;
        cnt += __popcll(m);
      }
      if (threadIdx.x == 0) s_nchild = cnt;
    }
    __syncthreads();
    const int nchild = s_nchild;

    Resid R{trow, drow, invT, Mt, 1.0 / Zt, Md, 1.0 / Zd, 0.0};
    double B = 1.0, S = 1.0;
    int accepted = -1;
    for (int j = 0; j < nchild; ++j) {
      const int c = s_children[j];
      int x = tok[c];
      if (x < 0 || x >= V) {
        if (threadIdx.x == 0 && member == 0) raise_status(p.status, TV_DEV_SHAPE);
        x = 0;
      }
      const double px = R.p(x);
      const double qx = R.q(x);
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
      double part = slice_resid_sum(Rn, lo, hi, vec4);
      part = block_sum(part, sh);
      if (threadIdx.x == 0) member_slot(tm, member)[0] = part;
      team_sync(tm);
      double F = 0.0;
      for (int w = 0; w < p.W; ++w) F += member_slot(tm, w)[0];
      tm.phase++;
      if (F > 0.0) {
        R.a = Rn.a;
        B = F;
      }
      S -= qx;
    }
    if (accepted >= 0) {
      v = accepted;
      continue;
    }

    // Stop at v: inverse-CDF draw from the residual (p itself when a == 0).
    const double wsum = wave_chunk_sum(R, cb, ce);
    if ((threadIdx.x & 63) == 0) sh_chunk[wv] = wsum;
    __syncthreads();
    double mine = 0.0;
    for (int w = 0; w < kWaves; ++w) mine += sh_chunk[w];
    if (threadIdx.x == 0) member_slot(tm, member)[0] = mine;
    team_sync(tm);
    double total = 0.0;
    int finder = -1;
    double base_w = 0.0;
    const double u = double(p.uniforms[2 * size_t(nbeg + v) + 1]);
    {
      double run = 0.0;
      for (int w = 0; w < p.W; ++w) run += member_slot(tm, w)[0];
      total = run;
      const double thr = u * total;
      double pre = 0.0;
      int last_pos = -1;
      double last_pre = 0.0;
      for (int w = 0; w < p.W; ++w) {
        const double sw = member_slot(tm, w)[0];
        if (sw > 0.0) {
          last_pos = w;
          last_pre = pre;
        }
        if (finder < 0 && pre <= thr && thr < pre + sw) {
          finder = w;
          base_w = pre;
        }
        pre += sw;
      }
      if (finder < 0) {
        finder = last_pos;
        base_w = last_pre;
      }
    }
    tm.phase++;
    if (finder == member) {
      const double local = u * total - base_w;
      int fw = -1;
      double pre = 0.0, fpre = 0.0;
      int last_w = -1;
      double last_pre = 0.0;
      for (int w = 0; w < kWaves; ++w) {
        const double cw = sh_chunk[w];
        if (cw > 0.0) {
          last_w = w;
          last_pre = pre;
        }
        if (fw < 0 && pre <= local && local < pre + cw) {
          fw = w;
          fpre = pre;
        }
        pre += cw;
      }
      if (fw < 0) {
        fw = last_w;
        fpre = last_pre;
      }
      if (wv == fw) {
        int y = wave_chunk_search(R, cb, ce, local - fpre);
        if (y < 0) y = 0;
        if ((threadIdx.x & 63) == 0) p.next_token[nbeg + v] = y;
      }
    }
    break;
  }
  team_exit(tm);
}

}  // namespace

bool plan_sample(const tv_sample_desc& d, SamplePlan* out) {
  if (d.batch < 1 || d.vocab < 1 || d.max_nodes < 1 || d.max_nodes > kMaxChildren ||
      d.max_depth < 0)
    return false;
  SamplePlan pl{};
  pl.threads = kThreads;
  pl.part_stride = 4;
  size_t off = kHeaderBytes;
  pl.off_team_ctr = off;
  off = align256(off + size_t(d.batch) * sizeof(uint32_t));
  pl.off_part = off;
  // Up to 16 members per team, two parities.
  off = align256(off + size_t(d.batch) * 2 * 16 * pl.part_stride * sizeof(double));
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
  // Team size: roughly one workgroup per CU across the batch, at most 16.
  const long resident = long(g_coop_blocks_per_cu) * g_num_cus;
  int W = int(g_num_cus / d.batch);
  if (W > 16) W = 16;
  if (W < 1) W = 1;
  while (W > 1 && long(W) * d.batch > resident) --W;
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
  const dim3 grid(unsigned(d.batch * W)), block(kThreads);
  if (W == 1) {
    hipLaunchKernelGGL(sample_kernel, grid, block, 0, stream, p);
    return hipGetLastError();
  }
  void* args[] = {&p};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(sample_kernel), grid, block,
                                    args, 0, stream);
}

}  // namespace tv
