// Dynamic draft-tree construction by expansion and rerank (EAGLE-2).
//
// Survey page, Timeline: EAGLE-2 grows the draft tree by expanding the top-k
// nodes by path-product value and reranking to keep the top-m nodes; the
// value is the cumulative draft probability along the root path (survey
// page, Taxonomy, construction policy axis). Values here are logs: a node's
// value is the sum of log q along its root path, q = softmax(draft row).
//
// One expansion round (tree_expand_step) = expand_kernel + select_kernel:
//  * expand_kernel: one workgroup per frontier row. One pass over the row's
//    logits keeps, per thread, its K best logits (ascending-index scan, so a
//    tie keeps the lower id ahead) and an online log-sum-exp (fp32 running
//    max and sum of the hardware exp2, within 1 ulp on normal results; the
//    block combines them in fp64). k rounds of a block
//    argmax over the threads' list heads then give the row's top-k in
//    descending logit, lowest id first on ties; child value = frontier value
//    + (logit - lse). Children are stored at candidate ids cand_offset +
//    slot * k + rank (generation order).
//  * select_kernel: one workgroup per request ranks the round's k_in * k new
//    candidates (value descending, id ascending) and writes the k best ids,
//    best first: the next frontier.
// tree_rerank = rerank_kernel: one 1024-thread workgroup per request ranks
// all candidates (float4 reads of the values in LDS), keeps ranks < m, and
// places the kept ones in ascending id (block prefix count of kept flags):
// root at 0, then the tree in topological order with request-local parents.
//
// The row pass is bound by HBM (4 bytes per logit); the selections touch a
// few KB per request.
#include <math.h>

#include <algorithm>

#include "tv_device.hpp"
#include "tv_internal.hpp"
#include "tv_topk.hpp"

namespace tv {

namespace {

constexpr int kConThreads = 256;
constexpr int kConWaves = kConThreads / kWave;
constexpr int kRrThreads = 1024;  // rerank_kernel
constexpr int kRrWaves = kRrThreads / kWave;
constexpr float kLog2e = 1.4426950408889634f;
constexpr long kSplitRows = 512;  // rounds with fewer rows split them (workspace permitting)

// (value, id) order of every selection: larger value first, lower id on ties.
// Values pass through key() first: NaN (from non-finite logits, already
// reported) orders as -inf, so the order stays total and ranks unique.
__device__ inline float key(float v) { return v != v ? -INFINITY : v; }
__device__ inline bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

struct ExpandParams {
  const float* logits;      // [batch][k_in][V]
  const int32_t* frontier;  // [batch][k_in] candidate ids, -1 = root; NULL: every slot is the root
  float* value;             // [batch][cap]
  int32_t* token;           // [batch][cap]
  int32_t* parent;          // [batch][cap]
  uint32_t* status;
  int V, k_in, k, cap, offset;
  // Split rounds (S > 1): workgroup (row, seg) covers float4s (or logits)
  // [seg * n / S, (seg + 1) * n / S) of the row and writes its k best
  // (logit, id) and its log-sum-exp partial (max, rescaled sum) here.
  int S;
  float* part_v;    // [rows][S][k]
  int32_t* part_i;  // [rows][S][k]
  float* part_m;    // [rows][S]
  double* part_s;   // [rows][S]
};

template <int K>
__global__ __launch_bounds__(kConThreads) void expand_kernel(ExpandParams p) {
  __shared__ float s_v[kConWaves];
  __shared__ int s_i[kConWaves];
  __shared__ float s_m[kConWaves];
  __shared__ double s_s[kConWaves];
  const int row = blockIdx.x / p.S;  // request * k_in + slot
  const int seg = blockIdx.x - row * p.S;
  const int b = row / p.k_in, slot = row - b * p.k_in;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const float* x = p.logits + size_t(row) * p.V;

  TopList<K> L;
  L.init();
  float m = -INFINITY, s = 0.f;
  bool bad = false;
  auto take = [&](float a, int id) __attribute__((always_inline)) {
    bad |= !(a - a == 0.f);  // NaN or +-Inf
    L.insert(a, id);
  };
  const bool vec = (p.V & 3) == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0;
  if (vec) {
    // kBatch float4 loads per thread in flight before any is consumed; each
    // thread still visits its elements in ascending index.
    const float4* x4 = reinterpret_cast<const float4*>(x);
    const int n4 = int((long(seg + 1) * (p.V >> 2)) / p.S);  // this segment's end
    const int lo4 = int((long(seg) * (p.V >> 2)) / p.S);
    // theta: the k-th largest of the wave's lane maxima. Those k lanes hold
    // k distinct elements >= theta, so an element below theta is not among
    // the row's k best (the lists keep K >= k entries; only k are used). A
    // float4 enters the list update only when some lane of the wave has an
    // element that passes both its own K-th best and theta (one wave-level
    // test per float4); theta is refreshed every other batch.
    float theta = -INFINITY;
    // Non-finite logits show in the sums: a NaN or a +Inf (Inf - Inf) makes
    // the running sum NaN; -Inf shows in the running minimum.
    float lo = INFINITY;
    auto use = [&](const float4 a, int e) __attribute__((always_inline)) {
      const float mx = fmaxf(fmaxf(a.x, a.y), fmaxf(a.z, a.w));
      lo = fminf(lo, fminf(fminf(a.x, a.y), fminf(a.z, a.w)));
      if (mx > m) {
        s *= __builtin_amdgcn_exp2f((m - mx) * kLog2e);
        m = mx;
      }
      s += __builtin_amdgcn_exp2f((a.x - m) * kLog2e) + __builtin_amdgcn_exp2f((a.y - m) * kLog2e) +
           __builtin_amdgcn_exp2f((a.z - m) * kLog2e) + __builtin_amdgcn_exp2f((a.w - m) * kLog2e);
      if (__builtin_amdgcn_ballot_w64((mx >= theta) & (mx > L.v[K - 1])) != 0) {
        // Only elements at or above theta can be among the row's k best.
        if (a.x >= theta) L.insert(a.x, 4 * e);
        if (a.y >= theta) L.insert(a.y, 4 * e + 1);
        if (a.z >= theta) L.insert(a.z, 4 * e + 2);
        if (a.w >= theta) L.insert(a.w, 4 * e + 3);
      }
    };
    // The batch loop's exit test is taken on the wave's last lane, so every
    // lane of a wave runs the same batches (the sort needs all 64 lanes);
    // the remainder runs lane by lane without refreshing theta.
    constexpr int kBatch = 8;
    const int to_last = (kWave - 1) - lane;
    int e = lo4 + tid, nb = 0;
    for (; e + to_last + (kBatch - 1) * kConThreads < n4; e += kBatch * kConThreads) {
      float4 a[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) a[u] = x4[e + u * kConThreads];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) use(a[u], e + u * kConThreads);
      if ((++nb & 1) == 1) theta = wave_kth_largest(L.v[0], p.k);  // every other batch
    }
    for (; e < n4; e += kConThreads) use(x4[e], e);
    bad |= !(s - s == 0.f) | (lo == -INFINITY);
  } else {
    const int hi = int((long(seg + 1) * p.V) / p.S);
    for (int e = int((long(seg) * p.V) / p.S) + tid; e < hi; e += kConThreads) {
      const float a = x[e];
      if (a > m) {
        s *= __builtin_amdgcn_exp2f((m - a) * kLog2e);
        m = a;
      }
      s += __builtin_amdgcn_exp2f((a - m) * kLog2e);
      take(a, e);
    }
  }
  if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0) raise_status(p.status, TV_DEV_LOGITS);

  // Block log-sum-exp: max in fp32, the rescaled sums in fp64.
  float mw = m;
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) mw = fmaxf(mw, shfl_xor(mw, o));
  if (lane == 0) s_m[wave] = mw;
  __syncthreads();
  float M = s_m[0];
#pragma unroll
  for (int w = 1; w < kConWaves; ++w) M = fmaxf(M, s_m[w]);
  double sd = m == -INFINITY ? 0.0 : double(s) * exp(double(m) - double(M));
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) sd += shfl_xor_d(sd, o);
  if (lane == 0) s_s[wave] = sd;
  __syncthreads();
  double sum = 0.0;
#pragma unroll
  for (int w = 0; w < kConWaves; ++w) sum += s_s[w];
  const double lse = double(M) + log(sum);

  // Frontier value (root: 0); a frontier id outside the earlier candidates
  // is reported and taken as the root. (Split rounds: the merge does this.)
  int f = p.frontier ? p.frontier[size_t(b) * p.k_in + slot] : -1;
  if (f < -1 || f >= p.offset) {
    if (tid == 0 && p.S == 1) raise_status(p.status, TV_DEV_TREE);
    f = -1;
  }
  const size_t cb = size_t(b) * p.cap;
  const double base = f < 0 || p.S > 1 ? 0.0 : double(p.value[cb + f]);
  const size_t ps = size_t(row) * p.S + seg;  // this segment's partial slot
  if (p.S > 1 && tid == 0) {
    p.part_m[ps] = M;
    p.part_s[ps] = sum;
  }

  // k rounds of block argmax over the list heads.
  for (int r = 0; r < p.k; ++r) {
    float bv = L.v[0];
    int bi = L.i[0];
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
      const float ov = shfl_xor(bv, o);
      const int oi = shfl_xor(bi, o);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane == 0) {
      s_v[wave] = bv;
      s_i[wave] = bi;
    }
    __syncthreads();
    float wv = s_v[0];
    int wi = s_i[0];
#pragma unroll
    for (int w = 1; w < kConWaves; ++w)
      if (better(s_v[w], s_i[w], wv, wi)) {
        wv = s_v[w];
        wi = s_i[w];
      }
    __syncthreads();  // every thread has read this round's winners
    if (L.i[0] == wi) L.pop();  // ids are unique across threads
    if (tid == 0 && p.S > 1) {
      p.part_v[ps * p.k + r] = wv;
      p.part_i[ps * p.k + r] = wi;
    } else if (tid == 0) {
      const size_t c = cb + size_t(p.offset) + size_t(slot) * p.k + r;
      const bool ok = wi < p.V;
      p.token[c] = ok ? wi : -1;
      p.value[c] = ok ? float(base + (double(wv) - lse)) : -INFINITY;
      p.parent[c] = f;
    }
  }
}

struct SelectParams {
  float* value;           // [batch][cap]
  int32_t* token;         // [batch][cap]
  int32_t* parent;        // [batch][cap]
  const int32_t* frontier;
  int32_t* next;          // [batch][k]
  uint32_t* status;
  int cap, offset, n, k;  // candidates offset .. offset + n - 1 (n = k_in * k)
  int k_in, V, S;         // S > 1: first merge the segments' partials
  const float* part_v;
  const int32_t* part_i;
  const float* part_m;
  const double* part_s;
};

__global__ __launch_bounds__(kConThreads) void select_kernel(SelectParams p) {
  __shared__ float s_v[kConThreads];
  __shared__ float s_pv[kConThreads * kMaxSplit];
  __shared__ int s_pi[kConThreads * kMaxSplit];
  __shared__ double s_lse[kMaxExpand], s_base[kMaxExpand];
  __shared__ int s_f[kMaxExpand];
  __shared__ float s_pm[kMaxExpand * kMaxSplit];
  __shared__ double s_ps[kMaxExpand * kMaxSplit];
  const int b = blockIdx.x, t = threadIdx.x;
  const size_t cb = size_t(b) * p.cap;
  if (p.S > 1) {
    // Merge: slot j's S * k partial entries -> its k children, and the
    // segments' log-sum-exp partials -> the row's lse (fp64).
    const int per_row = p.S * p.k, total = p.k_in * per_row;
    s_v[t] = -INFINITY;  // (a row without k finite logits leaves slots unwritten)
    const size_t row0 = size_t(b) * p.k_in;
    // Every partial is staged into LDS by its own thread (one round of
    // loads), next to the frontier nodes' ids and values.
    for (int q = t; q < total; q += kConThreads) {
      s_pv[q] = p.part_v[row0 * per_row + q];
      s_pi[q] = p.part_i[row0 * per_row + q];
    }
    if (t < p.k_in * p.S) {
      s_pm[t] = p.part_m[row0 * p.S + t];
      s_ps[t] = p.part_s[row0 * p.S + t];
    }
    if (t < p.k_in) {
      int f = p.frontier ? p.frontier[row0 + t] : -1;
      if (f < -1 || f >= p.offset) {
        raise_status(p.status, TV_DEV_TREE);
        f = -1;
      }
      s_base[t] = f < 0 ? 0.0 : double(p.value[cb + f]);
      s_f[t] = f;
    }
    __syncthreads();
    if (t < p.k_in) {
      float M = -INFINITY;
      for (int g = 0; g < p.S; ++g) M = fmaxf(M, s_pm[t * p.S + g]);
      double sum = 0.0;
      for (int g = 0; g < p.S; ++g) {
        const double sg = s_ps[t * p.S + g];
        if (sg > 0.0) sum += sg * exp(double(s_pm[t * p.S + g]) - double(M));
      }
      s_lse[t] = double(M) + log(sum);
    }
    __syncthreads();
    for (int q = t; q < total; q += kConThreads) {
      const int j = q / per_row, e0 = j * per_row;
      const float vq = s_pv[q];
      const int iq = s_pi[q];
      int rank = 0;
      for (int e = 0; e < per_row; ++e) rank += better(s_pv[e0 + e], s_pi[e0 + e], vq, iq);
      if (rank < p.k) {
        const int c = j * p.k + rank;
        const bool ok = iq < p.V;
        const float val = ok ? float(s_base[j] + (double(vq) - s_lse[j])) : -INFINITY;
        p.token[cb + p.offset + c] = ok ? iq : -1;
        p.value[cb + p.offset + c] = val;
        p.parent[cb + p.offset + c] = s_f[j];
        s_v[c] = val;  // the selection below reads the values from LDS
      }
    }
    __syncthreads();
  } else {
    s_v[t] = t < p.n ? p.value[cb + p.offset + t] : -INFINITY;
    __syncthreads();
  }
  const float mine = t < p.n ? key(s_v[t]) : -INFINITY;
  if (t < p.n) {
    int rank = 0;
    for (int j = 0; j < p.n; ++j) rank += better(key(s_v[j]), j, mine, t);
    if (rank < p.k) p.next[size_t(b) * p.k + rank] = p.offset + t;
  }
}

struct RerankParams {
  const float* value;     // [batch][cap]
  const int32_t* token;   // [batch][cap]
  const int32_t* parent;  // [batch][cap]
  int32_t* out_parent;    // [batch][m + 1]
  int32_t* out_token;     // [batch][m + 1]
  int32_t* out_count;     // [batch]
  uint32_t* status;
  int cap, n, m;
};

__global__ __launch_bounds__(kRrThreads) void rerank_kernel(RerankParams p) {
  __shared__ __align__(16) float s_v[kMaxRerank];
  __shared__ int s_pos[kMaxRerank];
  __shared__ int s_wsum[kRrWaves];
  const int b = blockIdx.x, t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  const size_t cb = size_t(b) * p.cap;
  const int n4 = (p.n + 3) >> 2;  // values padded with -inf to whole float4s
  for (int i = t; i < 4 * n4; i += kRrThreads) s_v[i] = i < p.n ? key(p.value[cb + i]) : -INFINITY;
  __syncthreads();
  // Thread t owns ids [t * per, t * per + per), per <= 4. A padded id j >= n
  // is never better than a real one (its value is -inf and its id larger).
  const int per = (p.n + kRrThreads - 1) / kRrThreads;
  const int lo = min(p.n, t * per), hi = min(p.n, lo + per);
  uint32_t kept = 0;  // bit j: id lo + j is kept
  const float4* v4 = reinterpret_cast<const float4*>(s_v);
  for (int i = lo; i < hi; ++i) {
    const float vi = s_v[i];
    int rank = 0;
    for (int j4 = 0; j4 < n4; ++j4) {
      const float4 w = v4[j4];
      const int j = 4 * j4;
      rank += better(w.x, j, vi, i) + better(w.y, j + 1, vi, i) + better(w.z, j + 2, vi, i) +
              better(w.w, j + 3, vi, i);
    }
    if (rank < p.m) kept |= 1u << (i - lo);
  }
  // Block exclusive prefix of the kept counts (thread order = id order).
  const int mine = __builtin_popcount(kept);
  int incl = mine;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int u = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += u;
  }
  if (lane == kWave - 1) s_wsum[wave] = incl;
  __syncthreads();
  int before = incl - mine, total = 0;
  for (int w = 0; w < kRrWaves; ++w) {
    const int c = s_wsum[w];
    before += w < wave ? c : 0;
    total += c;
  }
  int pos = 1 + before;
  for (int i = lo; i < hi; ++i) s_pos[i] = (kept >> (i - lo)) & 1 ? pos++ : 0;
  __syncthreads();
  const int W = p.m + 1;
  int32_t* op = p.out_parent + size_t(b) * W;
  int32_t* ot = p.out_token + size_t(b) * W;
  for (int i = lo; i < hi; ++i) {
    const int q = s_pos[i];
    if (!q || q > p.m) continue;  // ranks are unique, so at most m are kept
    int par = p.parent[cb + i];
    int pp;
    if (par < 0) {
      pp = 0;
    } else if (par < i && s_pos[par] > 0) {
      pp = s_pos[par];
    } else {  // a kept node whose parent is not kept (or not earlier): not a tree
      raise_status(p.status, TV_DEV_TREE);
      pp = 0;
    }
    op[q] = pp;
    ot[q] = p.token[cb + i];
  }
  for (int q = 1 + total + t; q < W; q += kRrThreads) {
    op[q] = -1;
    ot[q] = -1;
  }
  if (t == 0) {
    op[0] = -1;
    ot[0] = -1;
    p.out_count[b] = 1 + total;
  }
}

}  // namespace

size_t expand_workspace_bytes(int32_t batch, int32_t k_in, int32_t k) {
  const size_t slots = size_t(batch) * k_in * kMaxSplit;
  return kHeaderBytes + align256(slots * k * 4) * 2 + align256(slots * 4) + align256(slots * 8);
}

hipError_t launch_expand_step(int32_t batch, int32_t vocab, int32_t k_in, int32_t k,
                              const float* logits, const int32_t* frontier, int32_t cap,
                              int32_t offset, float* value, int32_t* token, int32_t* parent,
                              int32_t* next, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  uint32_t* status = static_cast<uint32_t*>(workspace);
  // Rounds with fewer rows than kSplitRows split each row over up to
  // kMaxSplit workgroups when the workspace holds the partials.
  const long rows = long(batch) * k_in;
  int S = 1;
  if (workspace && workspace_bytes >= expand_workspace_bytes(batch, k_in, k) && rows < kSplitRows)
    S = int(std::min<long>(kMaxSplit, std::max<long>(1, kSplitRows / rows)));
  ExpandParams e{logits, frontier, value, token, parent, status, vocab, k_in, k, cap, offset,
                 S, nullptr, nullptr, nullptr, nullptr};
  if (S > 1) {
    const size_t slots = size_t(batch) * k_in * kMaxSplit;
    char* w = static_cast<char*>(workspace) + kHeaderBytes;
    e.part_v = reinterpret_cast<float*>(w);
    w += align256(slots * k * 4);
    e.part_i = reinterpret_cast<int32_t*>(w);
    w += align256(slots * k * 4);
    e.part_m = reinterpret_cast<float*>(w);
    w += align256(slots * 4);
    e.part_s = reinterpret_cast<double*>(w);
  }
  const dim3 grid(static_cast<unsigned>(rows * S));
  if (k <= 4)
    hipLaunchKernelGGL(expand_kernel<4>, grid, dim3(kConThreads), 0, stream, e);
  else if (k <= 8)
    hipLaunchKernelGGL(expand_kernel<8>, grid, dim3(kConThreads), 0, stream, e);
  else if (k <= 12)
    hipLaunchKernelGGL(expand_kernel<12>, grid, dim3(kConThreads), 0, stream, e);
  else
    hipLaunchKernelGGL(expand_kernel<16>, grid, dim3(kConThreads), 0, stream, e);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  SelectParams sp{value, token, parent, frontier, next, status, cap, offset, k_in * k, k,
                  k_in, vocab, S, e.part_v, e.part_i, e.part_m, e.part_s};
  hipLaunchKernelGGL(select_kernel, dim3(unsigned(batch)), dim3(kConThreads), 0, stream, sp);
  return hipGetLastError();
}

hipError_t launch_rerank(int32_t batch, int32_t num_cand, int32_t cap, int32_t m,
                         const float* value, const int32_t* token, const int32_t* parent,
                         int32_t* out_parent, int32_t* out_token, int32_t* out_count,
                         uint32_t* status, hipStream_t stream) {
  RerankParams r{value, token, parent, out_parent, out_token, out_count, status, cap, num_cand, m};
  hipLaunchKernelGGL(rerank_kernel, dim3(unsigned(batch)), dim3(kRrThreads), 0, stream, r);
  return hipGetLastError();
}

}  // namespace tv
