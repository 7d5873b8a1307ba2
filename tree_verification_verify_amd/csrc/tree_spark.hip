// TreeSpark's best-first draft-tree construction with the calibrated theta
// stop (TreeSpark: Markov-conditioned draft trees, §3.1-§3.5).
//
// The drafter gives, per request, base logits U_1..U_b (one row per depth)
// and shares a rank-r Markov head B(x, v) = <W1[x], W2[v]> (§3.1). A node at
// depth d carrying token x has children drawn from q0 = softmax(U_{d+1} +
// B(x, .)) (§3.2 step 1). A max-heap of child slots is keyed by calibrated
// path survival: the sum of log p_hat along the root path with
// p_hat = sigma(a logit(q0) + b) on the unscaled q0 (§1, §3.4). A node's slot
// is its next child: the most probable unused token at T = 0, the next
// without-replacement draw from q_T at T > 0, where the slot is keyed by the
// admissible pre-draw bound S(v) p_hat(max unused q0) (§3.2). Materialising a
// node opens its first-child slot and its parent's next-sibling slot (up to
// K siblings); expansion stops when the best key falls below log theta or
// the tree holds N drafted nodes (§3.5).
//
// GPU design: one persistent kernel runs every round, phases separated by
// grid barriers (bounded waits). The launch is a plain one of as many
// workgroups as the device keeps resident at once (a cooperative launch
// costs more to start): on a device running nothing else they are all
// resident together; workgroups held back past the wait limit by other work
// make the call report TV_DEV_TIMEOUT instead of waiting on.
//  A select   one workgroup per request merges the statistics of the nodes
//             expanded last round, then pops slots while the best exact key
//             exceeds every pending node's bound (a node not yet expanded can
//             only open slots keyed at or below its own survival), so the
//             pops are exactly those of the one-at-a-time heap. It then lists
//             the nodes that need their conditional (at most kRows per round).
//             The request's state is kept as arrays (one entry per node), so
//             lanes reading their own node hit distinct LDS banks.
//  B logits   the listed nodes' W1 rows are staged in LDS 64 at a time (rows
//             padded so an operand read is conflict-free); every wave takes
//             16-token tiles of W2 as the A operand of
//             v_mfma_f32_16x16x32_bf16 against the four 16-row tiles of the
//             group, adds U and writes l = U + B for every listed row: W2 is
//             read once per row group. The next tile's W2 rows and U values
//             are loaded while the current tile is used, unconditionally (a
//             wave's last prefetch repeats the final tile), so the wait
//             before each product covers only its own tile's loads.
//  C stats    (row, segment) items stream l once, eight 16-byte loads per
//             thread in flight: fp32 online log-sum-exp, the row's K+1 best
//             logits, and at T > 0 its K best Gumbel scores l/T - ln(-ln u)
//             (u from Philox4x32-10 at counter (y/4, request * (N+1) + node,
//             stream, 0)), kept in per-thread lists behind a wave threshold
//             (each value's insert runs only where some lane's own value
//             passes), merged per wave by cross-lane reductions and across
//             waves in LDS.
// The select and logits phases are functions of their own (each gets the
// whole register file; inlined into one kernel they spilled into the logits
// loop), reading the parameters in place in the kernel-argument segment.
// Wave reductions and sorts exchange lanes by DPP and the row-swap permutes
// rather than LDS permutes.
// Grid barriers poll with relaxed loads and take one acquire fence after: an
// acquire load invalidates the XCD's L2 on every poll, which would evict the
// lines the working waves of that XCD are using. Rounds end when no request
// lists a node.
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "tv_device.hpp"
#include "tv_internal.hpp"
#include "tv_philox.hpp"
#include "tv_topk.hpp"

namespace tv {

namespace {

constexpr int kSpThreads = 256;
constexpr int kSpWaves = kSpThreads / kWave;
constexpr int kNodes = kSparkMaxNodes + 1;    // root + drafted nodes
constexpr int kList = kSparkMaxSiblings + 1;  // K + 1 entries per list
constexpr int kRows = kSparkRowsPerRound;
constexpr int kMaxSeg = kSparkMaxSeg;
constexpr int kMaxRank = 256;
constexpr int kGroupRows = 64;                // W1 rows staged per group
constexpr int kW1Stride = kMaxRank + 8;       // bf16 per staged row (528 B: 16-byte shift per row)
constexpr int kStatBatch = 8;                 // float4 loads per thread in flight (stats)

// A request's tree, one entry per node (workspace and LDS).
struct ReqState {
  double logS[kNodes];       // log path survival
  double lse[kNodes];        // log-sum-exp of the node's child logits
  int tok[kNodes], par[kNodes], dep[kNodes], nch[kNodes];
  int state[kNodes];         // 0 not expanded, 1 listed for expansion, 2 expanded
  int top_id[kNodes][kList]; // K+1 largest child logits, best first
  float top_l[kNodes][kList];
  int drw_id[kNodes][kList]; // T > 0: the K first without-replacement draws
  float drw_l[kNodes][kList];
  double lph_top[kNodes][kList];      // log p_hat of each top logit's q0
  double lph_drw[kNodes][kList];      // T > 0: log p_hat of each draw's q0
  uint8_t unused_e[kNodes][kList];    // T > 0: first top entry not among the first j draws
};
static_assert(sizeof(ReqState) % 16 == 0, "state is copied in 16-byte units");

// Statistics of one (row, segment).
struct Part {
  float m;
  float pad;
  double s;                  // sum exp(l - m)
  float tv[kList];           // best logits
  int ti[kList];
  float gv[kList];           // best Gumbel scores
  int gi[kList];
};

struct ReqHead {
  int done, count, pad[6];
};

struct SparkParams {
  const float* U;          // [B][depths][V]
  const uint16_t* w1;      // [V][r] bf16
  const uint16_t* w2;      // [V][r] bf16
  const int32_t* anchor;
  const float* temperature;
  const float* theta;
  int32_t* out_parent;     // [B][N+1]
  int32_t* out_token;
  int32_t* out_count;
  float* out_logs;         // optional
  uint32_t* status;
  uint32_t* bar;           // [0] arrivals, [1] generation
  ReqHead* head;           // [B]
  ReqState* state;         // [B]
  int4* rows;              // [2][B][kRows]: listed node, its token, its depth
  int* cnt;                // [2][B]
  float* ell;              // [B * kRows][V]
  Part* part;              // [B * kRows][kMaxSeg]
  int B, V, r, depths, N, K, nwg;
  float a, b;
  uint32_t stream, key0, key1;
  uint64_t wait_ticks;      // limit of the grid barrier's waits
};

// The kernel's parameters read in place (kernel-argument segment, constant
// address space): the phases take a pointer to them, made wave-uniform, so
// their fields are read with scalar loads rather than from a private copy.
typedef const __attribute__((address_space(4))) SparkParams KParams;

__device__ inline KParams* uniform_params(KParams* q) {
  const uint64_t v = reinterpret_cast<uint64_t>(q);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v)), hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  return reinterpret_cast<KParams*>((uint64_t(hi) << 32) | lo);
}

// Phase-local LDS: the select phase's request state, or the logits phase's
// staged W1 rows, or the statistics merge lists.
constexpr size_t kSelectBytes = sizeof(ReqState);
constexpr size_t kW1Bytes = size_t(kGroupRows) * kW1Stride * 2;
constexpr size_t kMergeBytes = size_t(kSpWaves) * kList * 8 * 2;
constexpr size_t kPhaseMax =
    kSelectBytes > kW1Bytes ? (kSelectBytes > kMergeBytes ? kSelectBytes : kMergeBytes)
                            : (kW1Bytes > kMergeBytes ? kW1Bytes : kMergeBytes);
// whole 1 KB blocks: the state is loaded a wave-wide 1 KB block at a time
constexpr size_t kPhaseBytes = (kPhaseMax + 1023) / 1024 * 1024;

// ---------------------------------------------------------------------------
// Grid barrier, in two levels along the XCDs (block b runs on XCD b % 8,
// and an XCD's L2 is coherent for its own CUs but not with the other XCDs'):
// a workgroup arrives on its XCD's counter; the XCD's last arrival writes
// back that L2 (one release per XCD) and arrives on the grid counter; the
// grid's last arrival bumps the grid generation, which every XCD's last
// arrival waits for (polled at system scope, past its own L2), then
// invalidates that L2 (one acquire) and bumps the XCD generation that the
// XCD's other workgroups wait for. Waits are bounded by time; after a
// timeout the workgroup is dead and every later barrier returns false.
// Words: grid counter 0, grid generation 1; XCD x's counter at 64 + 64x and
// generation at 96 + 64x (separate 256-byte lines). One arrival costs ~6 us
// at 512 workgroups against ~17 us for one grid-wide counter with an
// acquire-release arrival per workgroup.
constexpr int kBarWords = 64 + 8 * 64;

template <typename During>
__device__ bool grid_sync(KParams& p, uint32_t& gen, int* s_dead, During&& during) {
  __syncthreads();
  during();  // work whose memory latency may overlap the wait (no LDS, no barrier)
  if (threadIdx.x == 0 && !*s_dead) {
    const int x = blockIdx.x & 7;
    const uint32_t members = uint32_t((p.nwg - x + 7) / 8);  // workgroups on XCD x
    uint32_t* xc = p.bar + 64 + 64 * x;
    uint32_t* xg = p.bar + 96 + 64 * x;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    bool dead = false;
    const uint32_t old = __hip_atomic_fetch_add(xc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == members - 1u) {
      __hip_atomic_store(xc, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      const uint32_t groups = uint32_t(p.nwg < 8 ? p.nwg : 8);
      const uint32_t o2 = __hip_atomic_fetch_add(p.bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (o2 == groups - 1u) {
        __hip_atomic_store(p.bar, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(p.bar + 1, gen + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      } else {
        while (__hip_atomic_load(p.bar + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) == gen) {
          if (__builtin_amdgcn_s_memrealtime() - t0 > p.wait_ticks) {
            dead = true;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      __hip_atomic_store(xg, gen + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      while (__hip_atomic_load(xg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gen) {
        if (__builtin_amdgcn_s_memrealtime() - t0 > p.wait_ticks) {
          dead = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    if (dead) {
      raise_status(p.status, TV_DEV_TIMEOUT);
      *s_dead = 1;
    }
  }
  gen += 1u;
  __syncthreads();
  return !*reinterpret_cast<volatile int*>(s_dead);
}

__device__ bool grid_sync(KParams& p, uint32_t& gen, int* s_dead) {
  return grid_sync(p, gen, s_dead, [] {});
}

// ---------------------------------------------------------------------------
// Calibration and keys (fp64).

// log sigma(a logit(q) + b), in the stable form log sigma(z) = -softplus(-z).
__device__ inline double log_p_hat(double q, double a, double b) {
  if (!(q > 0.0)) return -INFINITY;
  if (q >= 1.0) return 0.0;
  const double z = a * (log(q) - log1p(-q)) + b;
  return z < 0.0 ? z - log1p(exp(z)) : -log1p(exp(-z));
}

__device__ inline bool rank_before(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// Wave argmax over (value, id) candidates, larger value then lower id; every
// lane returns the winner.
__device__ inline void wave_best(float& v, int& id) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = lane_xor(v, o);
    const int oi = lane_xor(id, o);
    if (rank_before(ov, oi, v, id)) {
      v = ov;
      id = oi;
    }
  }
}

// n rounds of a wave argmax over the first nc of kC candidates per lane
// (nc the same in every lane); the k-th winner goes to (dv[k], di[k])
// through lane 0.
template <int kC>
__device__ inline void wave_top(float (&cv)[kC], int (&ci)[kC], int nc, int n, float* dv, int* di) {
  const int lane = threadIdx.x & (kWave - 1);
  for (int k = 0; k < n; ++k) {
    float bv = cv[0];
    int bi = ci[0];
#pragma unroll
    for (int u = 1; u < kC; ++u)
      if (u < nc && rank_before(cv[u], ci[u], bv, bi)) {
        bv = cv[u];
        bi = ci[u];
      }
    wave_best(bv, bi);
#pragma unroll
    for (int u = 0; u < kC; ++u)
      if (u < nc && ci[u] == bi) {
        cv[u] = -INFINITY;
        ci[u] = 0x7fffffff;
      }
    if (lane == 0) {
      dv[k] = bv;
      di[k] = bi;
    }
  }
}

// A request's head (done, drafted nodes) into s_pf[0..1], its temperature
// and theta (bits) into s_pf[3..4] and, unless done, its state into LDS;
// s_pf[2] = 1 marks them loaded.
__device__ inline void load_request(KParams& p, int r, ReqState& st, int* s_pf) {
  constexpr int kWords = int(sizeof(ReqState) / 16);
  if (threadIdx.x == 0) {
    s_pf[0] = p.head[r].done;
    s_pf[1] = p.head[r].count;
    s_pf[3] = __float_as_int(p.temperature[r]);
    s_pf[4] = __float_as_int(p.theta[r]);
  }
  __syncthreads();
  if (!s_pf[0]) {
    const uint4* src = reinterpret_cast<const uint4*>(p.state + r);
    uint4* dst = reinterpret_cast<uint4*>(&st);
    for (int i = threadIdx.x; i < kWords; i += kSpThreads) dst[i] = src[i];
  }
  if (threadIdx.x == 0) s_pf[2] = 1;
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Phase A: one request.

__device__ __attribute__((noinline)) void select_request(KParams* pin, int r, int round, ReqState& st,
                                                        int* s_misc, int* s_pf) {
  KParams& p = *uniform_params(pin);
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int N = p.N, K = p.K;
  const int cur = round & 1, prev = cur ^ 1;
  const bool pre = round > 0 && s_pf[2];  // loaded at the end of the last round
  const float T = pre ? __int_as_float(s_pf[3]) : p.temperature[r];
  const bool sampled = T > 0.f;
  const float th = pre ? __int_as_float(s_pf[4]) : p.theta[r];
  const double logth = th > 0.f ? log(double(th)) : -INFINITY;
  ReqHead* hd = p.head + r;
  int4* my_rows = p.rows + (size_t(cur) * p.B + r) * kRows;
  constexpr int kWords = int(sizeof(ReqState) / 16);

  if (round == 0) {
    for (int i = tid; i <= N; i += kSpThreads) {
      p.out_parent[size_t(r) * (N + 1) + i] = -1;
      p.out_token[size_t(r) * (N + 1) + i] = -1;
      if (p.out_logs) p.out_logs[size_t(r) * (N + 1) + i] = i == 0 ? 0.f : -INFINITY;
    }
    if (tid == 0) {
      int a = p.anchor[r];
      if (a < 0 || a >= p.V) {
        raise_status(p.status, TV_DEV_SHAPE);
        a = 0;
      }
      if (!(T >= 0.f) || !(th >= 0.f)) raise_status(p.status, TV_DEV_LOGITS);  // read as 0
      st.tok[0] = a;
      st.par[0] = -1;
      st.dep[0] = 0;
      st.nch[0] = 0;
      st.state[0] = 0;
      st.logS[0] = 0.0;
      st.lse[0] = 0.0;
      s_misc[0] = 0;  // done
      s_misc[1] = 0;  // drafted nodes
    }
  } else {
    // the request's state, unless the workgroup loaded it at the end of the
    // last round (its only request)
    if (!s_pf[2]) load_request(p, r, st, s_pf);
    if (tid == 0) {
      s_misc[0] = s_pf[0];
      s_misc[1] = s_pf[1];
    }
  }
  __syncthreads();
  if (tid == 0) s_pf[2] = 0;
  if (s_misc[0]) {
    if (tid == 0) p.cnt[size_t(cur) * p.B + r] = 0;
    return;
  }
  const int count0 = s_misc[1];

  const double ca = p.a, cb = p.b;
  // --- merge last round's statistics of this request's listed nodes, one
  // node per wave (each touches only its own node's entries)
  if (round > 0) {
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    {
      int nprev = 0, pre = 0;
      for (int q = lane; q < p.B; q += kWave) {
        const int c = p.cnt[size_t(prev) * p.B + q];
        nprev += c;
        pre += q < r ? c : 0;
      }
      nprev = wave_sum(nprev);
      pre = wave_sum(pre);
      const int S = spark_segments(nprev, p.nwg);
      const int mine = p.cnt[size_t(prev) * p.B + r];
      for (int j = wave; j < mine; j += kSpWaves) {
        const int i = p.rows[(size_t(prev) * p.B + r) * kRows + j].x;
        const size_t g = size_t(pre + j);
        const Part* pp = p.part + g * kMaxSeg;
        // log-sum-exp of the segments
        double M = lane < S ? double(pp[lane].m) : -INFINITY;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) M = fmax(M, lane_xor(M, o));
        double t = lane < S && pp[lane].m != -INFINITY ? pp[lane].s * exp(double(pp[lane].m) - M) : 0.0;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) t += lane_xor(t, o);
        // the K+1 best logits and (T > 0) the K best scores over the
        // segments: candidates c = seg * n + e (n = K+1, resp. K), packed so
        // only the first ceil(S n / 64) slots of a lane are used
        constexpr int kC = (kMaxSeg * kList + kWave - 1) / kWave;
        const int nl = K + 1;
        const int ncl = (S * nl + kWave - 1) / kWave, ncg = (S * K + kWave - 1) / kWave;
        float cv[kC], gv[kC];
        int ci[kC], gi[kC];
#pragma unroll
        for (int u = 0; u < kC; ++u) {
          const int c = lane + u * kWave;
          const int sg = c / nl, e = c - sg * nl;
          const bool ok = u < ncl && sg < S;
          cv[u] = ok ? pp[sg].tv[e] : -INFINITY;
          ci[u] = ok ? pp[sg].ti[e] : 0x7fffffff;
          const int sgg = c / K, eg = c - sgg * K;
          const bool okg = sampled && u < ncg && sgg < S;
          gv[u] = okg ? pp[sgg].gv[eg] : -INFINITY;
          gi[u] = okg ? pp[sgg].gi[eg] : 0x7fffffff;
        }
        wave_top(cv, ci, ncl, nl, st.top_l[i], st.top_id[i]);
        if (sampled) wave_top(gv, gi, ncg, K, st.drw_l[i], st.drw_id[i]);
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        // fewer than K+1 candidates only with non-finite logits (already
        // reported): keep every id a valid row of W1; the drawn tokens'
        // logits are read back from the row, all at once
        if (lane < nl) {
          const int y = st.top_id[i][lane];
          if (y < 0 || y >= p.V) {
            raise_status(p.status, TV_DEV_LOGITS);
            st.top_id[i][lane] = 0;
          }
        }
        if (sampled && lane < K) {
          int y = st.drw_id[i][lane];
          if (y < 0 || y >= p.V) y = 0;
          st.drw_id[i][lane] = y;
          st.drw_l[i][lane] = p.ell[g * size_t(p.V) + y];
        }
        const double lse_i = M + log(t);
        if (lane == 0) {
          st.lse[i] = lse_i;
          st.state[i] = 2;
          if (!(t > 0.0) || !isfinite(lse_i)) raise_status(p.status, TV_DEV_LOGITS);
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        // tables for the pops: log p_hat of each top logit's and each
        // draw's q0 (the child's factor of its path survival), and at T > 0
        // the first top entry whose token is not among the first j draws
        // (the node's largest unused q0 after j children), j = 0..K
        if (lane < nl) st.lph_top[i][lane] = log_p_hat(exp(double(st.top_l[i][lane]) - lse_i), ca, cb);
        if (sampled) {
          if (lane < K) st.lph_drw[i][lane] = log_p_hat(exp(double(st.drw_l[i][lane]) - lse_i), ca, cb);
          int fd = K;  // the first draw of top entry `lane`'s token, K if none
          if (lane < nl) {
            const int y = st.top_id[i][lane];
            for (int j = 0; j < K; ++j)
              if (fd == K && st.drw_id[i][j] == y) fd = j;
          }
          for (int j = 0; j <= K; ++j) {
            const uint64_t m = __builtin_amdgcn_ballot_w64(lane < nl && fd >= j);
            if (lane == j) st.unused_e[i][j] = uint8_t(m ? min(__builtin_ctzll(m), kList - 1) : kList - 1);
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
      }
    }
  }
  __syncthreads();

  if (tid < kWave) {
    // --- pops. Each lane caches the slot key and the pending bound of its
    // nodes (lane and lane + 64); a pop changes only the popped node's key
    // (one more child) and adds one pending node, so only those two are
    // recomputed.
    int count = count0;
    int done = 0;
    static_assert(kNodes <= 2 * kWave, "two nodes per lane");
    double key[2], pend[2];
    bool keyed[2], pending[2];
    auto refresh = [&](int k) __attribute__((always_inline)) {
      const int i = lane + k * kWave;
      keyed[k] = pending[k] = false;
      key[k] = pend[k] = -INFINITY;
      if (i > count || st.dep[i] >= p.depths) return;
      if (st.state[i] == 2) {
        const int nch = st.nch[i];
        if (nch < K) {
          keyed[k] = true;
          key[k] = st.logS[i] + st.lph_top[i][sampled ? int(st.unused_e[i][nch]) : nch];
        }
      } else if (st.logS[i] >= logth) {
        pending[k] = true;
        pend[k] = st.logS[i];
      }
    };
    refresh(0);
    refresh(1);
    while (true) {
      if (count >= N) {
        done = 1;
        break;
      }
      // best slot (larger key, then lower node index), pending bound and count
      double bk = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int k = 0; k < 2; ++k)
        if (keyed[k] && (key[k] > bk || (key[k] == bk && lane + k * kWave < bi))) {
          bk = key[k];
          bi = lane + k * kWave;
        }
      double pb = fmax(pend[0], pend[1]);
      int npend = (pending[0] ? 1 : 0) + (pending[1] ? 1 : 0);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const double ok = lane_xor(bk, o);
        const int oi = lane_xor(bi, o);
        if (ok > bk || (ok == bk && oi < bi)) {
          bk = ok;
          bi = oi;
        }
        pb = fmax(pb, lane_xor(pb, o));
        npend += lane_xor(npend, o);
      }
      if (npend > 0 && (bi == 0x7fffffff || pb >= bk)) break;  // expand first
      if (bi == 0x7fffffff || bk < logth) {
        done = 1;
        break;
      }
      if (npend >= kRows) break;
      // pop the slot of node v (the node outputs are written after the loop)
      const int v = __builtin_amdgcn_readfirstlane(bi);
      const int j = st.nch[v];
      const int x = sampled ? st.drw_id[v][j] : st.top_id[v][j];
      const double lS = st.logS[v] + (sampled ? st.lph_drw[v][j] : st.lph_top[v][j]);
      const int c = count + 1;
      const int dv = st.dep[v];
      __builtin_amdgcn_wave_barrier();
      if (lane == 0) {
        st.tok[c] = x;
        st.par[c] = v;
        st.dep[c] = dv + 1;
        st.nch[c] = 0;
        st.state[c] = 0;
        st.logS[c] = lS;
        st.lse[c] = 0.0;
        st.nch[v] = j + 1;
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // LDS, within this wave
      __builtin_amdgcn_wave_barrier();
      count = c;
      if (lane == (v & (kWave - 1))) refresh(v / kWave);
      if (lane == (c & (kWave - 1))) refresh(c / kWave);
    }
    // the nodes materialised this round
    for (int c = count0 + 1 + lane; c <= count; c += kWave) {
      const size_t o = size_t(r) * (N + 1) + c;
      p.out_parent[o] = st.par[c];
      p.out_token[o] = st.tok[c];
      if (p.out_logs) p.out_logs[o] = float(st.logS[c]);
    }
    // --- list the nodes to expand (not when done)
    int listed = 0;
    if (!done) {
      for (int base = 0; base <= count; base += kWave) {
        const int i = base + lane;
        const bool want = i <= count && st.state[i] == 0 && st.dep[i] < p.depths && st.logS[i] >= logth;
        const uint64_t m = __ballot(want);
        const int pos = listed + int(__builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32),
                                                                __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u)));
        if (want && pos < kRows) {
          my_rows[pos] = make_int4(i, st.tok[i], st.dep[i], 0);  // what the logits phase needs
          st.state[i] = 1;
        }
        listed += __popcll(m);
      }
      listed = min(listed, kRows);
    }
    if (lane == 0) {
      s_misc[0] = done;
      s_misc[1] = count;
      s_misc[2] = listed;
    }
  }
  __syncthreads();
  // request state back to the workspace
  {
    const uint4* src = reinterpret_cast<const uint4*>(&st);
    uint4* dst = reinterpret_cast<uint4*>(p.state + r);
    for (int i = tid; i < kWords; i += kSpThreads) dst[i] = src[i];
  }
  if (tid == 0) {
    hd->done = s_misc[0];
    hd->count = s_misc[1];
    p.cnt[size_t(cur) * p.B + r] = s_misc[2];
    if (s_misc[0]) p.out_count[r] = s_misc[1] + 1;
  }
}

// ---------------------------------------------------------------------------
// Phase B: logits of the listed rows.

// Global-memory views (loads issued as global, not flat, accesses).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) u32x4 g_u32x4;
typedef const __attribute__((address_space(1))) f32x4 g_f32x4;
typedef const __attribute__((address_space(1))) float g_float;
typedef __attribute__((address_space(1))) f32x4 g_out_f32x4;

// A pointer that is the same in every lane, in scalar registers.
template <typename T>
__device__ inline T* uniform_ptr(T* q) {
  const uint64_t v = reinterpret_cast<uint64_t>(q);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v)), hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  return reinterpret_cast<T*>((uint64_t(hi) << 32) | lo);
}

// KKc > 0: the rank is 32 KKc (W2 loads and products unconditional);
// KKc = 0: any rank that is a multiple of 32 up to kMaxRank. kFull: V is a
// multiple of 16, so every 16-token tile is whole and 16-byte aligned.
template <int KKc, bool kFull>
__device__ __attribute__((noinline)) void logits_phase(KParams* pin, int n_act, const int* s_rx, const long long* s_ru,
                             uint16_t* s_w1) {
  KParams& p = *uniform_params(pin);
  // the parameters this phase uses, read once into wave-uniform registers
  // (reads through p inside the loop would be reloads past every store)
  const int V = __builtin_amdgcn_readfirstlane(p.V), rank = __builtin_amdgcn_readfirstlane(p.r);
  const int nwg = __builtin_amdgcn_readfirstlane(p.nwg);
  const uint16_t* w1 = uniform_ptr(p.w1);
  const float* U = uniform_ptr(p.U);
  float* ell = uniform_ptr(p.ell);
  const char* w2 = reinterpret_cast<const char*>(uniform_ptr(p.w2));
  const int tid = threadIdx.x, lane = tid & (kWave - 1), l16 = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  n_act = __builtin_amdgcn_readfirstlane(n_act);
  constexpr int kK = KKc ? KKc : kMaxRank / 32;
  const int KK = KKc ? KKc : rank / 32;
  const int nt = (V + 15) / 16;
  const int gw = blockIdx.x * kSpWaves + wave;
  const int nwave = nwg * kSpWaves;
  const bool vec = (V & 3) == 0;
  const uint32_t w2_row = uint32_t(rank) * 2u;  // bytes per W2 row (V r 2 < 4 GB)
  for (int g0 = 0; g0 < n_act; g0 += kGroupRows) {
    const int gn = min(kGroupRows, n_act - g0);
    // stage the group's W1 rows (zero past the group)
    __syncthreads();
    const int chunks = rank / 8;  // 16-byte pieces per row
    for (int c = tid; c < kGroupRows * chunks; c += kSpThreads) {
      const int row = c / chunks, piece = c - row * chunks;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row < gn) v = *reinterpret_cast<const uint4*>(w1 + size_t(s_rx[g0 + row]) * rank + piece * 8);
      *reinterpret_cast<uint4*>(s_w1 + row * kW1Stride + piece * 8) = v;
    }
    __syncthreads();
    const int nrt = (gn + 15) / 16;
    // this lane's U row in each row tile (rows past the group repeat the
    // group's last row; their results are not stored)
    const float* urow[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) urow[rt] = U + s_ru[g0 + min(rt * 16 + l16, gn - 1)];
    // one tile's operands: W2 rows (A operand) and U of the row tiles
    auto load_tile = [&](int tile, bf16x8 (&A)[kK], float4 (&uu)[4]) __attribute__((always_inline)) {
      const uint32_t tok = uint32_t(min(tile * 16 + l16, V - 1));
      const char* src = w2 + (tok * w2_row + uint32_t(16 * lg));
#pragma unroll
      for (int kk = 0; kk < kK; ++kk)
        if (KKc || kk < KK) A[kk] = __builtin_bit_cast(bf16x8, *(g_u32x4*)(src + kk * 64));
      const int y0 = tile * 16 + 4 * lg;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        if (kFull) {  // every row tile (absent ones repeat a loaded row: cache hits)
          const f32x4 v = *(g_f32x4*)(urow[rt] + y0);
          uu[rt] = make_float4(v[0], v[1], v[2], v[3]);
        } else {
          if (rt >= nrt) break;
          const g_float* u = (g_float*)urow[rt];
          uu[rt].x = y0 < V ? u[y0] : 0.f;
          uu[rt].y = y0 + 1 < V ? u[y0 + 1] : 0.f;
          uu[rt].z = y0 + 2 < V ? u[y0 + 2] : 0.f;
          uu[rt].w = y0 + 3 < V ? u[y0 + 3] : 0.f;
        }
      }
    };
    auto use_tile = [&](int tile, const bf16x8 (&A)[kK], const float4 (&uu)[4]) __attribute__((always_inline)) {
      const int y0 = tile * 16 + 4 * lg;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        if (rt >= nrt) break;
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        const uint16_t* brow = s_w1 + (rt * 16 + l16) * kW1Stride + 8 * lg;
#pragma unroll
        for (int kk = 0; kk < kK; ++kk)
          if (KKc || kk < KK)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[kk], *reinterpret_cast<const bf16x8*>(brow + kk * 32),
                                                          acc, 0, 0, 0);
        // lane holds row g, tokens y0 .. y0 + 3
        const int g = g0 + rt * 16 + l16;
        if (g < g0 + gn) {
          float* out = ell + size_t(g) * V;
          const float4 o = make_float4(acc[0] + uu[rt].x, acc[1] + uu[rt].y, acc[2] + uu[rt].z,
                                       acc[3] + uu[rt].w);
          if (kFull) {
            *(g_out_f32x4*)(out + y0) = f32x4{o.x, o.y, o.z, o.w};
          } else if (vec && y0 + 3 < V) {
            *reinterpret_cast<float4*>(out + y0) = o;
          } else {
            if (y0 < V) out[y0] = o.x;
            if (y0 + 1 < V) out[y0 + 1] = o.y;
            if (y0 + 2 < V) out[y0 + 2] = o.z;
            if (y0 + 3 < V) out[y0 + 3] = o.w;
          }
        }
      }
    };
    // two tiles' operands in registers: the next tile in flight while one
    // is used. The loads are unconditional (a wave's last prefetch reloads
    // the final tile, which every wave reads: cache hits) so that the wait
    // before each product covers only the loads of the tile it uses.
    bf16x8 A0[kK], A1[kK];
    float4 U0[4], U1[4];
    if (gw < nt) load_tile(gw, A0, U0);
    for (int t = gw; t < nt; t += 2 * nwave) {
      load_tile(min(t + nwave, nt - 1), A1, U1);
      use_tile(t, A0, U0);
      if (t + nwave >= nt) break;
      load_tile(min(t + 2 * nwave, nt - 1), A0, U0);
      use_tile(t + nwave, A1, U1);
    }
  }
}

// ---------------------------------------------------------------------------
// Phase C: statistics of one (row, segment).

template <int L>
__device__ void stats_item(KParams& p, int g, int seg, int S, int req, int node, float T,
                           float* s_v, int* s_i, double* s_d, float* m_v, int* m_i) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int K = p.K, nl = K + 1;
  const bool noisy = T > 0.f;
  const float invT = noisy ? 1.f / T : 0.f;
  const float* row = p.ell + size_t(g) * p.V;
  const int ng = (p.V + 3) / 4;
  const int q0 = int(long(ng) * seg / S), q1 = int(long(ng) * (seg + 1) / S);
  const uint32_t node_row = uint32_t(req) * uint32_t(p.N + 1) + uint32_t(node);
  const bool vec = (p.V & 3) == 0;
  constexpr float kLog2e = 1.4426950408889634f;

  TopList<L> A, G;
  A.init();
  G.init();
  float m = -INFINITY, s = 0.f, thA = -INFINITY, thG = -INFINITY;
  bool bad = false;
  int step = 0;
  // Every thread runs the same batches (the thresholds are wave-wide
  // shuffles); a thread past the segment's end carries -inf values.
  const int steps = (q1 - q0 + kSpThreads - 1) / kSpThreads;
  for (int b0 = 0; b0 < steps; b0 += kStatBatch) {
    float4 buf[kStatBatch];
#pragma unroll
    for (int u = 0; u < kStatBatch; ++u) {
      const int q = q0 + (b0 + u) * kSpThreads + tid;
      const int y = 4 * q;
      buf[u] = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      if (b0 + u < steps && q < q1) {
        if (vec) {
          buf[u] = *reinterpret_cast<const float4*>(row + y);
        } else {
          buf[u].x = row[y];
          buf[u].y = y + 1 < p.V ? row[y + 1] : -INFINITY;
          buf[u].z = y + 2 < p.V ? row[y + 2] : -INFINITY;
          buf[u].w = y + 3 < p.V ? row[y + 3] : -INFINITY;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kStatBatch; ++u) {
      if (b0 + u >= steps) break;
      const int q = q0 + (b0 + u) * kSpThreads + tid;
      const bool in = q < q1;
      const int y = 4 * q;
      const float v[4] = {buf[u].x, buf[u].y, buf[u].z, buf[u].w};
      const float mx = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
      if (in) {
#pragma unroll
        for (int e = 0; e < 4; ++e) bad |= y + e < p.V && !(v[e] - v[e] == 0.f);
        if (mx > m) {
          s *= __builtin_amdgcn_exp2f((m - mx) * kLog2e);
          m = mx;
        }
        s += __builtin_amdgcn_exp2f((v[0] - m) * kLog2e) + __builtin_amdgcn_exp2f((v[1] - m) * kLog2e) +
             __builtin_amdgcn_exp2f((v[2] - m) * kLog2e) + __builtin_amdgcn_exp2f((v[3] - m) * kLog2e);
      }
      // each value's insert runs only where some lane's own value qualifies
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (in && v[e] >= thA && v[e] > A.v[L - 1]) A.insert(v[e], y + e);
      if (noisy) {
        const uint4 w4 = philox4x32_10(make_uint4(uint32_t(q), node_row, p.stream, 0u), p.key0, p.key1);
        const uint32_t w[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = (float(16777216u - (w[e] >> 8)) - 0.5f) * (1.f / 16777216.f);  // 1 - u
          const float bound = v[e] * invT - __logf(x) + 1e-3f;                             // g <= -ln(1 - u)
          if (in && v[e] != -INFINITY && bound >= thG && bound > G.v[L - 1]) {
            const float uu = (float(w[e] >> 8) + 0.5f) * (1.f / 16777216.f);
            const float en = uu > 0.5f ? -log1pf(-x) : -logf(uu);  // -ln u, accurate near u = 1
            G.insert(v[e] * invT - logf(en), y + e);
          }
        }
      }
      ++step;
      if (step == 2 || step == 4 || (step & 7) == 0) {  // early refreshes: the lists fill fast
        thA = wave_kth_largest(A.v[0], nl);
        if (noisy) thG = wave_kth_largest(G.v[0], K);
      }
    }
  }
  if (bad) raise_status(p.status, TV_DEV_LOGITS);

  Part* out = p.part + size_t(g) * kMaxSeg + seg;
  // log-sum-exp partial: block maximum, then the rescaled sums in fp64
  float M = m;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, lane_xor(M, o));
  if (lane == 0) s_v[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(s_v[0], s_v[1]), fmaxf(s_v[2], s_v[3]));
  double sd = m == -INFINITY ? 0.0 : double(s) * exp(double(m) - double(M));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sd += lane_xor(sd, o);
  if (lane == 0) s_d[wave] = sd;
  // the lists: each wave's n best by cross-lane reductions, then one wave
  // over the waves'
  for (int k = 0; k < nl; ++k) {
    float bv = A.v[0];
    int bi = A.i[0];
    wave_best(bv, bi);
    if (A.i[0] == bi && bi != 0x7fffffff) A.pop();
    if (lane == 0) {
      m_v[wave * kList + k] = bv;
      m_i[wave * kList + k] = bi;
    }
  }
  if (noisy)
    for (int k = 0; k < K; ++k) {
      float hv = G.v[0];
      int hi = G.i[0];
      wave_best(hv, hi);
      if (G.i[0] == hi && hi != 0x7fffffff) G.pop();
      if (lane == 0) {
        m_v[(kSpWaves + wave) * kList + k] = hv;
        m_i[(kSpWaves + wave) * kList + k] = hi;
      }
    }
  __syncthreads();
  if (tid < kWave) {
    constexpr int kC = (kSpWaves * kList + kWave - 1) / kWave;
    float cv[kC], gv[kC];
    int ci[kC], gi[kC];
#pragma unroll
    for (int u = 0; u < kC; ++u) {
      const int c = lane + u * kWave, w = c / kList, e = c - w * kList;
      const bool ok = w < kSpWaves && e < nl;
      cv[u] = ok ? m_v[w * kList + e] : -INFINITY;
      ci[u] = ok ? m_i[w * kList + e] : 0x7fffffff;
      const bool okg = noisy && w < kSpWaves && e < K;
      gv[u] = okg ? m_v[(kSpWaves + w) * kList + e] : -INFINITY;
      gi[u] = okg ? m_i[(kSpWaves + w) * kList + e] : 0x7fffffff;
    }
    wave_top(cv, ci, kC, nl, out->tv, out->ti);
    if (noisy) wave_top(gv, gi, kC, K, out->gv, out->gi);
    if (lane == 0) {
      out->m = M;
      out->s = (s_d[0] + s_d[1]) + (s_d[2] + s_d[3]);
    }
  }
  __syncthreads();
}

template <int L>
__global__ __launch_bounds__(kSpThreads, 2) void spark_kernel(SparkParams params) {
  KParams* pk = (KParams*)__builtin_amdgcn_kernarg_segment_ptr();  // the first argument is at offset 0
  KParams& p = *pk;
  __shared__ __align__(16) unsigned char s_phase[kPhaseBytes];
  __shared__ int s_rx[kSparkMaxRows];
  __shared__ long long s_ru[kSparkMaxRows];
  __shared__ int s_rq[kSparkMaxRows], s_rn[kSparkMaxRows];
  __shared__ float s_v[kSpWaves];
  __shared__ int s_i[kSpWaves];
  __shared__ double s_d[kSpWaves];
  __shared__ int s_misc[4];
  __shared__ int s_pf[5];  // prefetched request: done, count, loaded flag, temperature, theta
  __shared__ int s_dead;
  if (threadIdx.x == 0) {
    s_dead = 0;
    s_pf[2] = 0;
  }
  __syncthreads();
  ReqState& st = *reinterpret_cast<ReqState*>(s_phase);
  uint16_t* s_w1 = reinterpret_cast<uint16_t*>(s_phase);
  float* m_v = reinterpret_cast<float*>(s_phase);
  int* m_i = reinterpret_cast<int*>(s_phase + size_t(2) * kSpWaves * kList * sizeof(float));
  uint32_t gen = __hip_atomic_load(p.bar + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint32_t expanded = 0;
  // state prefetch (a workgroup whose only request is blockIdx.x)
  constexpr int kStateBlocks = int((sizeof(ReqState) + 1023) / 1024);
  static_assert(size_t(kStateBlocks) * 1024 <= kPhaseBytes, "the state's blocks fit the phase area");
  const bool pf_on = p.B <= p.nwg && int(blockIdx.x) < p.B;
  int4 pf_head = make_int4(0, 0, 0, 0);
  for (int round = 0; round <= p.N + 2; ++round) {
    for (int r = blockIdx.x; r < p.B; r += p.nwg) {
      select_request(pk, r, round, st, s_misc, s_pf);
      __syncthreads();
    }
    if (!grid_sync(p, gen, &s_dead)) return;
    // the rows listed this round, in request order
    const int cur = round & 1;
    if (threadIdx.x < kWave) {
      int listed = 0;
      for (int q0 = 0; q0 < p.B; q0 += kWave) {
        const int q = q0 + int(threadIdx.x);
        const int c = q < p.B ? p.cnt[size_t(cur) * p.B + q] : 0;
        // the request's row descriptors, loaded together with its count
        // (every slot is in the workspace; slots past the count unused)
        int4 dsc[kRows];
        const int4* qd = p.rows + (size_t(cur) * p.B + (q < p.B ? q : 0)) * kRows;
#pragma unroll
        for (int j = 0; j < kRows; ++j) dsc[j] = qd[j];
        int inc = c;  // inclusive prefix over the wave
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
          const int t = __shfl_up(inc, o, kWave);
          if (int(threadIdx.x) >= o) inc += t;
        }
        const int start = listed + inc - c;
#pragma unroll
        for (int j = 0; j < kRows; ++j) {
          if (j < c) {
            s_rx[start + j] = dsc[j].y;
            s_ru[start + j] = ((long long)q * p.depths + dsc[j].z) * p.V;
            s_rq[start + j] = q;
            s_rn[start + j] = dsc[j].x;
          }
        }
        listed += __shfl(inc, kWave - 1, kWave);
      }
      if (threadIdx.x == 0) s_misc[3] = listed;
    }
    __syncthreads();
    const int n_act = s_misc[3];
    if (n_act == 0) {  // every request is done (the same for every workgroup)
      if (blockIdx.x == 0 && threadIdx.x == 0) {  // diagnostics: rounds run, rows expanded
        p.status[2] = uint32_t(round);
        p.status[3] = expanded;
      }
      return;
    }
    expanded += uint32_t(n_act);
    if (p.r == 256 && p.V % 16 == 0)
      logits_phase<8, true>(pk, n_act, s_rx, s_ru, s_w1);
    else
      logits_phase<0, false>(pk, n_act, s_rx, s_ru, s_w1);
    if (!grid_sync(p, gen, &s_dead)) return;
    const int S = spark_segments(n_act, p.nwg);
    for (int it = blockIdx.x; it < n_act * S; it += p.nwg) {
      const int g = it / S, seg = it - g * S;
      stats_item<L>(p, g, seg, S, s_rq[g], s_rn[g], p.temperature[s_rq[g]], s_v, s_i, s_d, m_v, m_i);
    }
    // a workgroup with one request loads its state for the next round
    // during the barrier, straight into LDS (16-byte buffer-to-LDS loads,
    // 1 KB per wave instruction; the phase area is free by then) from waves
    // 1-3: wave 0 arrives on the barrier, and its release fence would wait
    // for its own loads
    const bool live = grid_sync(p, gen, &s_dead, [&] {
      if (pf_on && threadIdx.x >= kWave) {
        const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave) - 1;
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(p.state + blockIdx.x, 0, int(sizeof(ReqState)), 0x00020000);
        const int lane = threadIdx.x & (kWave - 1);
        for (int c = w; c < kStateBlocks; c += kSpWaves - 1)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(s_phase + c * 1024),
                                                   16, c * 1024 + lane * 16, 0, 0, 0);
        if (threadIdx.x == kWave)
          pf_head = make_int4(p.head[blockIdx.x].done, p.head[blockIdx.x].count,
                              __float_as_int(p.temperature[blockIdx.x]), __float_as_int(p.theta[blockIdx.x]));
      }
    });
    if (!live) return;
    if (pf_on) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // LDS reads are not ordered after these loads
      if (threadIdx.x == kWave) {
        s_pf[0] = pf_head.x;
        s_pf[1] = pf_head.y;
        s_pf[2] = 1;
        s_pf[3] = pf_head.z;
        s_pf[4] = pf_head.w;
      }
      __syncthreads();
    }
  }
}

// Per-device resident workgroups of each kernel instantiation.
constexpr int kMaxDevices = 64;
std::atomic<int> g_nwg9[kMaxDevices], g_nwg17[kMaxDevices];

template <int L>
hipError_t resident_workgroups(int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::atomic<int>* cache = L == 9 ? g_nwg9 : g_nwg17;
  if (dev >= 0 && dev < kMaxDevices) {
    const int v = cache[dev].load(std::memory_order_acquire);
    if (v > 0) {
      *out = v;
      return hipSuccess;
    }
  }
  int cus = 0, per = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, reinterpret_cast<const void*>(spark_kernel<L>),
                                                   kSpThreads, 0);
  if (e != hipSuccess) return e;
  if (per < 1 || cus < 1) return hipErrorInvalidDevice;
  const int v = per * cus;
  if (dev >= 0 && dev < kMaxDevices) cache[dev].store(v, std::memory_order_release);
  *out = v;
  return hipSuccess;
}

template <int L>
hipError_t launch(SparkParams& p, hipStream_t stream) {
  int nwg = 0;
  hipError_t e = resident_workgroups<L>(&nwg);
  if (e != hipSuccess) return e;
  p.nwg = nwg;
  hipLaunchKernelGGL(spark_kernel<L>, dim3(unsigned(nwg)), dim3(kSpThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

size_t spark_workspace_bytes(const tv_spark_desc& d) {
  size_t off = kHeaderBytes;                      // status word
  off += align256(size_t(kBarWords) * sizeof(uint32_t));  // grid barrier words
  off += align256(size_t(d.batch) * sizeof(ReqHead));
  off += align256(size_t(d.batch) * sizeof(ReqState));
  off += align256(size_t(2) * d.batch * kRows * sizeof(int4));
  off += align256(size_t(2) * d.batch * sizeof(int));
  off += align256(size_t(d.batch) * kRows * kMaxSeg * sizeof(Part));
  off += align256(size_t(d.batch) * kRows * size_t(d.vocab) * sizeof(float));
  return off;
}

hipError_t launch_spark(const tv_spark_desc& d, const SparkArgs& a, hipStream_t stream) {
  SparkParams p{};
  char* ws = static_cast<char*>(a.workspace);
  size_t off = 0;
  p.status = reinterpret_cast<uint32_t*>(ws);
  off += kHeaderBytes;
  p.bar = reinterpret_cast<uint32_t*>(ws + off);
  off += align256(size_t(kBarWords) * sizeof(uint32_t));
  p.head = reinterpret_cast<ReqHead*>(ws + off);
  off += align256(size_t(d.batch) * sizeof(ReqHead));
  p.state = reinterpret_cast<ReqState*>(ws + off);
  off += align256(size_t(d.batch) * sizeof(ReqState));
  p.rows = reinterpret_cast<int4*>(ws + off);
  off += align256(size_t(2) * d.batch * kRows * sizeof(int4));
  p.cnt = reinterpret_cast<int*>(ws + off);
  off += align256(size_t(2) * d.batch * sizeof(int));
  p.part = reinterpret_cast<Part*>(ws + off);
  off += align256(size_t(d.batch) * kRows * kMaxSeg * sizeof(Part));
  p.ell = reinterpret_cast<float*>(ws + off);
  p.U = a.base_logits;
  p.w1 = static_cast<const uint16_t*>(a.w1);
  p.w2 = static_cast<const uint16_t*>(a.w2);
  p.anchor = a.anchor;
  p.temperature = a.temperature;
  p.theta = a.theta;
  p.out_parent = a.out_parent;
  p.out_token = a.out_token;
  p.out_count = a.out_count;
  p.out_logs = a.out_logsurv;
  p.B = d.batch;
  p.V = d.vocab;
  p.r = d.rank;
  p.depths = d.depths;
  p.N = d.max_nodes;
  p.K = d.max_siblings;
  p.a = d.calib_a;
  p.b = d.calib_b;
  p.stream = a.stream_id;
  p.key0 = uint32_t(a.seed);
  p.key1 = uint32_t(a.seed >> 32);
  p.wait_ticks = wait_ticks();
  if (d.max_siblings + 1 <= 9) return launch<9>(p, stream);
  return launch<17>(p, stream);
}

}  // namespace tv
