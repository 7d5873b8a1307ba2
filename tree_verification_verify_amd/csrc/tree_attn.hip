// Tree-masked attention over a paged prefix KV cache (one layer).
//
// What it computes follows SpecInfer's tree-based parallel decoding as the
// survey page's Timeline section describes it (tree tokens stored in the KV
// cache in topological order, each token attending to its ancestors only) and
// TreeSpark §3.2 step 3 / §4 (one target pass, per-step ancestor bitmask).
//
// bf16 path (gfx950, the production path):
//  * Rows are (tree node x grouped q head); a row block is 128 rows of one
//    (request r, kv head g), so one K/V tile staged in LDS serves every node
//    of the block and all G = Hq/Hkv heads that share the kv head.
//  * Work is the flat list of 64-key tiles of every (r, g, row block) pair.
//    A fixed grid of persistent workgroups (one of 8 waves per CU) splits
//    that list into contiguous shares of equal cost (stream-K, with tiles of
//    wide row blocks and each pair's set-up weighted), so uneven prefixes
//    balance. A pair wholly inside one share is finished in registers and
//    written out; a pair cut by share boundaries leaves fp32 partials
//    (offset, l, acc), which a second, small kernel merges in share order
//    (deterministic; the kernel boundary makes the partials visible, so the
//    streaming kernel needs no fences, counters or waiting). Shares are laid
//    out XCD by XCD, so the row blocks of one kv head share an XCD's L2.
//  * One 16-row tile per wave. S^T = K Q^T and O^T += V^T P^T on
//    v_mfma_f32_16x16x32_bf16; both keep a row on lane%16, so the online
//    softmax rescale is lane-local and P never leaves registers.
//  * V pages are stored transposed ([D][16] per page and head). K and V^T
//    stages go from HBM straight into a ring of LDS slots (1 KB per wave
//    load instruction), three stages ahead of the one being computed; the
//    slots are XOR-swizzled so operand reads are free of bank conflicts, and
//    the QK operand rows are permuted so each PV operand is one 16-byte read.
//  * The ancestor mask is a per-node bitset built in LDS while a segment's
//    first stages load, and consulted only in tiles reaching the tree keys.
// fp32 path (small validation shapes): a VALU kernel, one workgroup per
// (request, kv head, row block, key split), with the same partial format.
#include <type_traits>

#include "tv_device.hpp"
#include "tv_internal.hpp"

namespace tv {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kRowsPB = 128;     // rows per row block (bf16 path)
constexpr int kStage = 64;       // keys per stage / tile (bf16 path)
constexpr int kMaxWG = 256;      // persistent workgroups: one per CU on 256 CUs
constexpr int kMinTilesPerWG = 2;
constexpr size_t kLdsBytes = 160 * 1024;  // LDS per workgroup (gfx950)

struct AttnParams {
  const void* q;
  const void* k_pages;
  const void* v_pages;
  const int32_t* page_indptr;
  const int32_t* page_indices;
  const int32_t* prefix_len;
  const int32_t* node_indptr;
  const int32_t* parent;
  void* out;
  float* part_o;
  float* part_ml;
  uint32_t* counters;
  int4* merge_desc;  // [nwg][3]: cut pair finished by each share (bf16 path)
  uint32_t* status;
  int B, Hq, Hkv, G, num_pages, max_nodes, max_kv_len, words;
  int rb_max, c_max, chunk_len, grid_real, nwg, lg_nwg;
  float scale_log2;
};

__device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Row i's element offset in q / out: row = node * G + grouped head.
__device__ inline size_t qo_offset(const AttnParams& p, int nbeg, int g, int row, int D) {
  const int node = row / p.G;
  const int gh = row - node * p.G;
  return (size_t(nbeg + node) * p.Hq + size_t(g) * p.G + gh) * D;
}

// Ancestor-or-self bitsets of nodes first_node .. first_node+nn-1 in LDS
// (nn rows of `words`, zero-filled), walking the request's parent links
// already staged in LDS (`par`). Caller synchronises before and after.
__device__ inline void link_anc(const AttnParams& p, int first_node, int nn, int words,
                                uint32_t* anc, const int* par) {
  for (int t = threadIdx.x; t < nn; t += blockDim.x) {
    uint32_t* row = anc + t * words;
    int j = first_node + t;
    while (true) {
      row[j >> 5] |= 1u << (j & 31);
      const int pj = par[j];
      if (j == 0) {
        if (pj != -1) raise_status(p.status, TV_DEV_TREE);
        break;
      }
      if (pj < 0 || pj >= j) {
        raise_status(p.status, TV_DEV_TREE);
        break;
      }
      j = pj;
    }
  }
}

// As link_anc, staging the request's N parents and clearing the bitsets
// first. Caller synchronises before and after.
__device__ inline void build_anc(const AttnParams& p, int nbeg, int N, int first_node, int nn,
                                 int words, uint32_t* anc, int* par) {
  for (int i = threadIdx.x; i < nn * words; i += blockDim.x) anc[i] = 0u;
  for (int i = threadIdx.x; i < N; i += blockDim.x) par[i] = p.parent[nbeg + i];
  __syncthreads();
  link_anc(p, first_node, nn, words, anc, par);
}

// Keep bf16 elements [0, n) of an 8-element chunk, zero the rest (no branches).
__device__ inline uint4 keep_first(uint4 v, int n) {
  auto word = [n](uint32_t w, int i) {
    const int k = n - 2 * i;  // elements of word i to keep: <=0, 1, or >=2
    return k >= 2 ? w : (k == 1 ? (w & 0xffffu) : 0u);
  };
  return make_uint4(word(v.x, 0), word(v.y, 1), word(v.z, 2), word(v.w, 3));
}

// ---------------------------------------------------------------------------
// Stream-K bookkeeping of the bf16 path.

// Work is measured in cost units. A 64-key tile costs kCostSmall units when
// its row block has at most four 16-row tiles and kCostBig when it has more
// (one row tile per wave, twice the MFMA and softmax work of a split wave),
// and each (request, kv head, row block) pair adds kCostPair units for the
// set-up and hand-off of a segment. Shares are equal in units, so a
// workgroup that crosses many short pairs, or streams many wide row blocks,
// gets fewer tiles.
constexpr int kCostSmall = 8;
constexpr int kCostBig = 10;
constexpr int kCostPair = 64;

__device__ inline int tile_cost(int rows) { return rows > 64 ? kCostBig : kCostSmall; }

// Units of one kv head of a request with R rows and nt tiles per pair.
__device__ inline int head_units(int R, int nt) {
  const int full = R / kRowsPB, rem = R - full * kRowsPB;
  return full * (kCostPair + nt * kCostBig) + (rem > 0 ? kCostPair + nt * tile_cost(rem) : 0);
}

// Units of request r (all kv heads and row blocks); 0 for an empty or
// rejected request (rejections are reported once, by `report`).
__device__ inline int request_units(const AttnParams& p, int r, bool report) {
  const int nbeg = p.node_indptr[r];
  const int N = p.node_indptr[r + 1] - nbeg;
  const int P = p.prefix_len[r];
  if (N <= 0) return 0;
  if (N > p.max_nodes || P < 0 || P > p.max_kv_len - N) {
    if (report) raise_status(p.status, TV_DEV_SHAPE);
    return 0;
  }
  const int L = P + N;
  const int npg = p.page_indptr[r + 1] - p.page_indptr[r];
  if (npg < 0 || npg < ceil_div(L, kPage)) {
    if (report) raise_status(p.status, TV_DEV_PAGES);
    return 0;
  }
  return p.Hkv * head_units(N * p.G, ceil_div(L, kStage));
}

// The pair of request r (first unit `base`, R rows, nt tiles per pair) that
// holds unit x: kv head g, row block rb, first tile unit t0 (after the
// pair's header), units per tile c.
struct PairAt {
  int g, rb, t0, c;
};
__device__ inline PairAt pair_at(int base, int x, int R, int nt) {
  const int per_g = head_units(R, nt);
  PairAt q;
  q.g = (x - base) / per_g;
  const int rem = x - base - q.g * per_g;
  const int full = R / kRowsPB;
  const int fu = kCostPair + nt * kCostBig;  // units of a full row block
  q.rb = min(rem / fu, full);
  q.t0 = base + q.g * per_g + q.rb * fu + kCostPair;
  q.c = q.rb < full ? kCostBig : tile_cost(R - full * kRowsPB);
  return q;
}

// Share [a_w, b_w) of the T units given to logical workgroup w of n = 2^lg.
__device__ inline int share_begin(int T, int w, int lg) {
  return int((uint64_t(T) * uint32_t(w)) >> lg);
}

// Logical workgroup whose share contains unit x (x < T): the largest w with
// share_begin(w) <= x.
__device__ inline int share_of(int T, int x, int lg) {
  const int n = 1 << lg;
  int w = int(float(x) * float(n) / float(T));
  w = min(max(w, 0), n - 1);
  while (w > 0 && share_begin(T, w, lg) > x) --w;
  while (w + 1 < n && share_begin(T, w + 1, lg) <= x) ++w;
  return w;
}

// Tiles [lo, hi) of a pair (first tile unit t0, c units per tile, nt tiles)
// whose first unit lies in the share [sa, sb): a tile belongs to the share
// holding its first unit.
__device__ inline int tiles_before(int x, int t0, int c, int nt) {
  return x <= t0 ? 0 : min(nt, (x - t0 + c - 1) / c);
}

// Partial slot of logical workgroup w for its part of a cut pair: a share
// holds at most two cut pairs, one continued from earlier shares (its part
// starts past tile 0; slot 2w) and one continued by later shares (slot 2w+1).
__device__ inline size_t cut_slot(int w, int lo) {
  return lo > 0 ? size_t(2 * w) : size_t(2 * w + 1);
}

// Block-wide unit offsets of every request: off[r] = first unit of request
// r in the flat (request, kv head, row block, tile) order, off[B] = T.
// Rejected requests (reported once when `report`) contribute no units.
// s_scan holds one int per wave of the block.
__device__ inline int scan_units(const AttnParams& p, int* off, int* s_scan, bool report) {
  const int nt = blockDim.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = ceil_div(p.B, nt);
  const int r0 = min(p.B, tid * per), r1 = min(p.B, r0 + per);
  int mine = 0;
  for (int r = r0; r < r1; ++r) {
    const int t = request_units(p, r, report);
    off[r] = t;
    mine += t;
  }
  int inc = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += t;
  }
  if (lane == 63) s_scan[wave] = inc;
  __syncthreads();
  int base = 0, total = 0;
  for (int w = 0; w < (nt >> 6); ++w) {
    base += (w < wave) ? s_scan[w] : 0;
    total += s_scan[w];
  }
  int run = base + inc - mine;
  for (int r = r0; r < r1; ++r) {
    const int t = off[r];
    off[r] = run;
    run += t;
  }
  if (tid == 0) off[p.B] = total;
  __syncthreads();
  return off[p.B];
}

// Last r with off[r] <= x (x < off[B]).
__device__ inline int request_of(const int* off, int B, int x) {
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= x) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Merge descriptor of share w (logical workgroup lw of the streaming pass):
// when the share's first pair was cut by earlier shares and ends in this
// share, it records that pair (first share w0, nbeg, kv head, first row |
// rows, first tile unit t0, units per tile, tiles | T); otherwise w0 = -1.
// Every share writes its entry on every launch, so no entry outlives the
// launch that wrote it.
__device__ inline void write_merge_desc(const AttnParams& p, const int* off, int T, int a, int b,
                                        int lw) {
  int4 d0 = make_int4(-1, 0, 0, 0), d1 = make_int4(0, 0, 0, 0);
  if (a < b) {
    const int r = request_of(off, p.B, a);
    const int nbeg = p.node_indptr[r];
    const int N = p.node_indptr[r + 1] - nbeg;
    const int L = p.prefix_len[r] + N;
    const int R = N * p.G;
    const int nt = ceil_div(L, kStage);
    const PairAt q = pair_at(off[r], a, R, nt);
    const int tlo = tiles_before(a, q.t0, q.c, nt);
    const int thi = tiles_before(b, q.t0, q.c, nt);
    if (tlo > 0 && tlo < thi && thi == nt) {
      d0 = make_int4(share_of(T, q.t0, p.lg_nwg), nbeg, q.g, q.rb * kRowsPB);
      d1 = make_int4(min(kRowsPB, R - q.rb * kRowsPB), q.t0, q.c, nt);
    }
  }
  p.merge_desc[3 * lw] = d0;
  p.merge_desc[3 * lw + 1] = d1;
  p.merge_desc[3 * lw + 2] = make_int4(T, 0, 0, 0);
}

// Merge kernel: workgroup (w, rt) merges rows 16rt .. 16rt+15 of the cut
// pair whose last tile lies in share w (its merge descriptor), combining the
// (offset, l, acc) partials of every share holding part of the pair in share
// order (deterministic), with a running offset so all loads of a group of
// shares are in flight together. 16 threads per row, D/16 floats each.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnParams p) {
  constexpr int F = D / 64;  // float4 per thread
  constexpr int U = 8;       // shares loaded together
  __shared__ int s_slot[kMaxWG];  // partial slot of share w0 + i, -1 when it holds no tile
  const int w = blockIdx.x >> 3;
  const int rt = blockIdx.x & 7;
  const int4 d0 = p.merge_desc[3 * w];
  if (d0.x < 0) return;
  const int4 d1 = p.merge_desc[3 * w + 1];
  const int T = p.merge_desc[3 * w + 2].x;
  const int rows_here = d1.x;
  if (rt * 16 >= rows_here) return;
  const int row = rt * 16 + (threadIdx.x >> 4);
  const int seg = threadIdx.x & 15;
  const bool live = row < rows_here;
  const int w0 = d0.x, t0 = d1.y, c = d1.z, nt = d1.w;
  const int nsh = w - w0 + 1;  // shares w0 .. w
  // Partial slot of share w0 + i, or -1 when that share holds no tile of
  // the pair. Up to four shares (the common case) take one round with the
  // slots formed in registers; more take rounds of U with the slots formed
  // once in LDS.
  auto slot_of = [&](int i) {
    const int v = w0 + i;
    const int lo = tiles_before(share_begin(T, v, p.lg_nwg), t0, c, nt);
    const int hi = tiles_before(share_begin(T, v + 1, p.lg_nwg), t0, c, nt);
    return hi > lo ? int(cut_slot(v, lo)) : -1;
  };
  const bool table = nsh > 4;
  if (table) {
    for (int i = threadIdx.x; i < nsh; i += blockDim.x) s_slot[i] = slot_of(i);
    __syncthreads();
  }

  float M = -INFINITY, Ls = 0.f;
  float4 acc[F];
#pragma unroll
  for (int f = 0; f < F; ++f) acc[f] = make_float4(0.f, 0.f, 0.f, 0.f);
  auto round = [&](int i0, auto u_c) __attribute__((always_inline)) {
    constexpr int NU = decltype(u_c)::value;
    float m[NU], l[NU];
    float4 o[NU][F];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int i = i0 + u;
      const int slot = i < nsh ? (table ? s_slot[i] : slot_of(i)) : -1;
      m[u] = -INFINITY;
      l[u] = 0.f;
#pragma unroll
      for (int f = 0; f < F; ++f) o[u][f] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (slot >= 0 && live) {
        const size_t base = size_t(slot) * kRowsPB + row;
        m[u] = p.part_ml[base * 2];
        l[u] = p.part_ml[base * 2 + 1];
#pragma unroll
        for (int f = 0; f < F; ++f)
          o[u][f] = *reinterpret_cast<const float4*>(p.part_o + base * D + (seg * F + f) * 4);
      }
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      if (m[u] > M) {
        const float sc = M == -INFINITY ? 0.f : exp2f(M - m[u]);
        Ls *= sc;
#pragma unroll
        for (int f = 0; f < F; ++f) {
          acc[f].x *= sc;
          acc[f].y *= sc;
          acc[f].z *= sc;
          acc[f].w *= sc;
        }
        M = m[u];
      }
      const float wt = m[u] == -INFINITY ? 0.f : exp2f(m[u] - M);
      Ls += wt * l[u];
#pragma unroll
      for (int f = 0; f < F; ++f) {
        acc[f].x += wt * o[u][f].x;
        acc[f].y += wt * o[u][f].y;
        acc[f].z += wt * o[u][f].z;
        acc[f].w += wt * o[u][f].w;
      }
    }
  };
  if (!table)
    round(0, std::integral_constant<int, 4>{});
  else
    for (int i0 = 0; i0 < nsh; i0 += U) round(i0, std::integral_constant<int, U>{});
  if (!live) return;
  const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
  uint16_t* dst = static_cast<uint16_t*>(p.out) + qo_offset(p, d0.y, d0.z, d0.w + row, D) + seg * F * 4;
#pragma unroll
  for (int f = 0; f < F; ++f) {
    uint2 pk;
    pk.x = pack_bf16x2(acc[f].x * inv, acc[f].y * inv);
    pk.y = pack_bf16x2(acc[f].z * inv, acc[f].w * inv);
    *reinterpret_cast<uint2*>(dst + f * 4) = pk;
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel: one workgroup of 8 waves per CU, persistent over tiles.

constexpr int kWavesS = 8;                // waves per workgroup
constexpr int kThreadsS = 64 * kWavesS;   // threads per workgroup

// LDS layout of a stage slot, unpadded, swizzled at 16-byte granularity:
//  * K [64 keys][D]: row r keeps its chunk c at c ^ swz_k(r);
//  * V^T page-major [4 pages][D][16 keys]: the two 8-key halves h of row d
//    sit at 16-byte unit 2d + (h ^ swz_v(d)) of the page block.
// The 16 lanes that read together in an MFMA operand load (K: rows differing
// in bits 0, 1, 3 and 4; V^T: 16 consecutive rows, one half each) then hit
// 16 distinct 16-byte bank groups (and 8 distinct ones per 8 lanes).
template <int D>
__device__ inline int swz_k(int r) {
  return D == 128 ? ((r & 3) | ((r >> 1) & 12)) : ((r & 3) | ((r >> 1) & 4));
}
__device__ inline int swz_v(int d) { return ((d >> 2) ^ (d >> 3)) & 1; }

// NaN-propagating max (gfx950 v_maximum3_f32; no operand canonicalisation).
__device__ inline float fmax_(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Row max over a lane's group of four lanes (lanes l, l^16, l^32, l^48),
// with gfx950's cross-row swaps (no LDS round trip).
__device__ inline float max_across_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmax_(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmax_(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Wait until at most N vector-memory operations of this wave are pending
// (s_waitcnt vmcnt(N); the other counters are left alone).
template <int N>
__device__ inline void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// 16 bytes per lane from global memory straight into LDS: lane i of the
// wave writes lds_base + 16*i (lds_base must be wave-uniform). Written as
// inline asm so the compiler keeps no account of these loads: every wait
// for them is explicit (wait_vm before a stage barrier), and the compiler
// adds no conservative full waits of its own in front of LDS reads.
__device__ inline void load_lds16(const void* src, void* lds_base) {
  const uint32_t base = uint32_t(reinterpret_cast<uintptr_t>(lds_base));
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(base) : "memory");
}
// As load_lds16 with 4 bytes per lane (lane i writes lds_base + 4*i).
__device__ inline void load_lds4(const void* src, void* lds_base) {
  const uint32_t base = uint32_t(reinterpret_cast<uintptr_t>(lds_base));
  asm volatile("global_load_lds_dword %0, off" ::"v"(src), "{m0}"(base) : "memory");
}

// Workgroup barrier without a memory fence (no wait for pending global
// loads or stores); this wave's LDS operations complete first. The empty
// asm statements keep the compiler from moving memory operations across it.
__device__ inline void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int I, int N, class F>
__device__ __attribute__((always_inline)) inline void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Stage ring: NS slots of 64 keys, each K [64][D] then V^T [D][64] (bf16).
// Loads go straight from HBM to LDS (global_load_lds_dwordx4), NS-1 stages
// ahead of the one being computed; each slot is its own LDS object so the
// compiler knows which pending loads a read depends on.
// page_idx, node_ip, prefix and page_ip alias p.page_indices,
// p.node_indptr, p.prefix_len and p.page_indptr, declared __restrict__ so
// their (wave-uniform) loads go through the scalar cache.
template <int D, int NS>
__global__ __launch_bounds__(kThreadsS, 1) void attn_stream_kernel(AttnParams p,
                                                                   const int32_t* __restrict__ page_idx,
                                                                   const int32_t* __restrict__ node_ip,
                                                                   const int32_t* __restrict__ prefix,
                                                                   const int32_t* __restrict__ page_ip) {
  constexpr int KK = D / 32;          // 32-wide k-steps of the QK product
  constexpr int DT = D / 16;          // 16-wide d tiles of the PV product
  constexpr int NI = D / 32;          // 1 KB loads per wave per stage (K and V^T)
  constexpr int KI = NI / 2;          // of which K
  constexpr int KROWS = 512 / D;      // K rows per 1 KB load
  constexpr int SLOT = 2 * kStage * D;

  __shared__ __attribute__((aligned(16))) uint16_t s0[SLOT];
  __shared__ __attribute__((aligned(16))) uint16_t s1[SLOT];
  __shared__ __attribute__((aligned(16))) uint16_t s2[NS > 2 ? SLOT : 8];
  __shared__ __attribute__((aligned(16))) uint16_t s3[NS > 3 ? SLOT : 8];
  __shared__ float s_xol[4 * 16 * 2];
  __shared__ int s_scan[kWavesS];
  extern __shared__ int dyn_lds[];
  int* off = dyn_lds;                                                 // [B + 1]
  int* par = dyn_lds + p.B + 1;                                       // [max_nodes, to 64]
  uint32_t* anc = reinterpret_cast<uint32_t*>(par + ((p.max_nodes + 63) & ~63));  // [nn][words]

  auto slot = [&](auto j_c) __attribute__((always_inline)) -> uint16_t* {
    constexpr int J = decltype(j_c)::value % NS;
    if constexpr (J == 0) return s0;
    else if constexpr (J == 1) return s1;
    else if constexpr (J == 2) return s2;
    else return s3;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int l16 = lane & 15;
  const int lg = lane >> 4;
  const int lw = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);

  const int T = scan_units(p, off, s_scan, lw == 0);
  const int a = share_begin(T, lw, p.lg_nwg);
  const int b = share_begin(T, lw + 1, p.lg_nwg);
  if (tid == 0) write_merge_desc(p, off, T, a, b, lw);
  if (a >= b) return;

  int r = request_of(off, p.B, a);  // request holding unit a

  const uint16_t* qb = static_cast<const uint16_t*>(p.q);
  const uint16_t* kp = static_cast<const uint16_t*>(p.k_pages);
  const uint16_t* vp = static_cast<const uint16_t*>(p.v_pages);
  const size_t head_block = size_t(kPage) * D;  // elements per (page, head)

  // Operand addresses (elements) inside one slot. In the QK product block h
  // of 32-key half kt2 feeds lane row l16 with stage key kt2*32 + 4h + krow,
  // krow = 8*(l16/4) + l16%4, so the S^T accumulator of lane group lg holds
  // keys kt2*32 + 8lg + 4h + e (e < 4): eight consecutive keys, which are
  // exactly the keys the PV operand of lane group lg takes from one 16-byte
  // V^T chunk.
  const int krow = 8 * (l16 >> 2) + (l16 & 3);
  int kaddr[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) kaddr[kk] = krow * D + (((kk * 4 + lg) ^ swz_k<D>(krow)) * 8);
  // V^T operand of lane group lg in half kt2: keys 8lg..8lg+7 of the half,
  // i.e. page 2*kt2 + lg/2, 8-key half lg&1, row d = 16*dt + l16 (the
  // swizzle depends on d's bits 2 and 3 only, so on l16).
  const int vaddr = kStage * D + (lg >> 1) * (D * kPage) + 16 * l16 + 8 * ((lg & 1) ^ swz_v(l16));

  // Stage loads of this wave, each 1 KB and inside one (page, head) block:
  // K rows 8*wave .. 8*wave+7 (page wave/2 of the stage), and V^T rows
  // 32*(q % (D/32)) .. +31 of page q / (D/32), q = KI*wave + j. Lane offsets
  // inside a block are fixed; only the page ids change.
  constexpr int VPI = D / 32;  // 1 KB loads per V^T page block
  int k_off[KI], v_off[KI];
#pragma unroll
  for (int j = 0; j < KI; ++j) {
    const int kr = 8 * wave + j * KROWS + lane / (D / 8);
    k_off[j] = (kr & 15) * D + (((lane % (D / 8)) ^ swz_k<D>(kr)) * 8);
    const int q = KI * wave + j;
    const int d = 32 * (q % VPI) + (lane >> 1);
    v_off[j] = d * kPage + 8 * ((lane & 1) ^ swz_v(d));
  }

  int c = a;  // unit cursor
  while (c < b) {
    while (off[r + 1] <= c) ++r;
    r = __builtin_amdgcn_readfirstlane(r);
    const int nbeg = node_ip[r];
    const int N = node_ip[r + 1] - nbeg;
    const int P = prefix[r];
    const int L = P + N;
    const int R = N * p.G;
    const int nt = ceil_div(L, kStage);
    const PairAt q = pair_at(__builtin_amdgcn_readfirstlane(off[r]), c, R, nt);
    c = q.t0 + nt * q.c;  // next pair
    // This share's tiles of the pair.
    const int tlo = tiles_before(a, q.t0, q.c, nt);
    const int thi = tiles_before(b, q.t0, q.c, nt);
    if (tlo >= thi) continue;
    const int g = q.g;
    const bool whole = tlo == 0 && thi == nt;
    const int row0 = q.rb * kRowsPB;
    const int rows_here = min(kRowsPB, R - row0);
    const int pbase = page_ip[r];
    const int pend = page_ip[r + 1] - 1;  // last listed page (>= pbase)
    const int words = ceil_div(N, 32);
    const int first_node = row0 / p.G;
    const int nn_blk = (row0 + rows_here - 1) / p.G - first_node + 1;

    stage_barrier();  // every wave is done with the LDS of the previous segment

    // Wave roles. Row tile t holds block rows 16t..16t+15. With five or
    // more row tiles each wave takes one and every key of a stage (NH = 2
    // halves); with four or fewer, waves w and w+4 take row tile w and the
    // 32-key halves 0 and 1 of each stage (NH = 1), merged through LDS at
    // the end of the segment.
    const int nrt = ceil_div(rows_here, 16);
    const bool ksplit = nrt <= 4;
    const int rt0 = ksplit ? (wave & 3) : wave;
    const int rt = rt0 < nrt ? rt0 : -1;
    const int half = ksplit ? (wave >> 2) : 0;
    bool active = rt >= 0;
    const int row = rt * 16 + l16;  // block-local row of this lane

    // Q and the parent links come through LDS by the same direct loads as
    // the stages, issued ahead of them: the wait for them then leaves the
    // prologue stages in flight (a load into registers would make the
    // compiler wait for every earlier load, the stages included). A wave's
    // Q rows (lane (l16, lg), load kk: 16 bytes at column 8lg + 32kk) go to
    // its own 1 KB pieces of the last ring slot, which the first step
    // refills only after its barrier; rows past the block read the block's
    // last row and are zeroed in registers.
    bf16x8 qf[KK];  // read from LDS once the loads have landed
    uint16_t* qlds = slot(std::integral_constant<int, NS - 1>{}) + wave * (KK * 512);
    if (active) {
      const uint16_t* src = qb + qo_offset(p, nbeg, g, row0 + min(row, rows_here - 1), D) + lg * 8;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) load_lds16(src + kk * 32, qlds + kk * 512);
    }
    const bool tree_keys = thi * kStage > P;  // the segment reaches tree keys: masks needed
    if (tree_keys) {
      // 64 parents per load (the region is rounded up to 64 entries; lanes
      // past N repeat the last parent)
      for (int c0 = wave * 64; c0 < N; c0 += kThreadsS)
        load_lds4(p.parent + nbeg + min(c0 + lane, N - 1), par + c0);
      for (int i = tid; i < nn_blk * words; i += kThreadsS) anc[i] = 0u;
    }

    // Every load of a wave lies in page wave/2 of its stage (K rows 8*wave..
    // 8*wave+7, and V^T blocks KI*wave .. KI*wave+KI-1 of D/32 per page), so
    // a wave needs one page id per stage, a scalar. A page past the sequence
    // is read from page 0; its keys, like slots past the sequence in the
    // last page, are masked and their V rows zeroed in registers. Ids outside
    // the pool are reported and also replaced by page 0.
    const int wpg = wave >> 1;
    bool bad_page = false;
    auto load_id = [&](int tile) __attribute__((always_inline)) -> int {
      const int x = page_idx[min(pbase + tile * 4 + wpg, pend)];
      const bool live = tile < thi && tile * kStage + wpg * kPage < L;
      const bool in_pool = unsigned(x) < unsigned(p.num_pages);
      bad_page |= live && !in_pool;
      return (live && in_pool) ? x : 0;
    };
    // Each load is a scalar block address plus the lane's fixed offset.
    // Stages past the segment are issued as dummies (every lane reads the
    // same 16 bytes of page 0, and the slot is never read), so every step
    // waits for the same number of loads.
    auto issue = [&](uint16_t* sb, int id, bool live) __attribute__((always_inline)) {
      const size_t blk = (size_t(id) * p.Hkv + g) * head_block;
#pragma unroll
      for (int j = 0; j < KI; ++j)
        load_lds16(kp + blk + (live ? k_off[j] : 0), sb + (8 * wave + j * KROWS) * D);
#pragma unroll
      for (int j = 0; j < KI; ++j) {
        const int q = KI * wave + j;
        load_lds16(vp + blk + (live ? v_off[j] : 0), sb + kStage * D + wpg * (D * kPage) + (q % VPI) * 512);
      }
    };

    // Online softmax state of the lane's row. Scores stay raw dot products;
    // the exponent is exp2(c*s - off) with c = scale*log2(e) and off =
    // c*m_ref. The reference m_ref is raised only when a new raw max exceeds
    // it by more than kLazy/c (then acc and l are rescaled), so p <= 2^kLazy
    // and most tiles skip the rescale. Whether any row must raise is decided
    // from each lane's own eight scores (the row max passes the threshold iff
    // one of its lanes' maxima does), so the cross-lane row max is formed
    // only on the tiles that raise.
    constexpr float kLazy = 8.f;
    const float cs = p.scale_log2;
    float m_ref = -INFINITY, off_ = 0.f, l_run = 0.f;
    f32x4 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // One stage of a row tile: NH = 2 computes both 32-key halves, NH = 1
    // the wave's own half. Stages of prefix keys only (all but the last one
    // or two of a pair) take a single straight-line path for all halves: one
    // raise decision for the stage, no mask, no tail.
    auto compute_plain = [&](const uint16_t* sb, auto nh_c) __attribute__((always_inline)) {
      constexpr int NH = decltype(nh_c)::value;
      f32x4 s[NH][2];
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) {
        const int kt2 = NH == 2 ? hh : half;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          s[hh][h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) {
            const bf16x8 ka = *reinterpret_cast<const bf16x8*>(sb + (kt2 * 32 + 4 * h) * D + kaddr[kk]);
            s[hh][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[kk], s[hh][h], 0, 0, 0);
          }
        }
      }
      float mloc = -INFINITY;
#pragma unroll
      for (int hh = 0; hh < NH; ++hh)
        mloc = fmax_(mloc, fmax_(fmax_(fmax_(s[hh][0][0], s[hh][0][1]), fmax_(s[hh][0][2], s[hh][0][3])),
                                 fmax_(fmax_(s[hh][1][0], s[hh][1][1]), fmax_(s[hh][1][2], s[hh][1][3]))));
      const bool need = (mloc > m_ref) & ((m_ref == -INFINITY) | (cs * (mloc - m_ref) > kLazy));
      if (__builtin_amdgcn_ballot_w64(need)) {
        const float mt = max_across_groups(mloc);
        const bool raise = (mt > m_ref) & ((m_ref == -INFINITY) | (cs * (mt - m_ref) > kLazy));
        const float m_new = raise ? mt : m_ref;
        const float off_new = m_new == -INFINITY ? 0.f : cs * m_new;
        const float alpha = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(off_ - off_new);
        m_ref = m_new;
        off_ = off_new;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
      }
      bf16x8 pb[NH];
      float ls = 0.f;
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float pv = __builtin_amdgcn_exp2f(fmaf(s[hh][h][e], cs, -off_));
            ls += pv;
            pb[hh][4 * h + e] = static_cast<__bf16>(pv);
          }
        }
      }
      l_run += ls;
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) {
        const int kt2 = NH == 2 ? hh : half;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const bf16x8 va = *reinterpret_cast<const bf16x8*>(sb + kt2 * (2 * D * kPage) + dt * 256 + vaddr);
          acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[hh], acc[dt], 0, 0, 0);
        }
      }
    };
    auto compute = [&](const uint16_t* sb, int tile, auto nh_c) __attribute__((always_inline)) {
      constexpr int NH = decltype(nh_c)::value;
      const int t0 = tile * kStage;
      if (t0 + kStage <= P) {
        compute_plain(sb, nh_c);
        return;
      }
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) {
        const int kt2 = NH == 2 ? hh : half;
        f32x4 s[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          s[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) {
            const bf16x8 ka = *reinterpret_cast<const bf16x8*>(sb + (kt2 * 32 + 4 * h) * D + kaddr[kk]);
            s[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[kk], s[h], 0, 0, 0);
          }
        }
        const int k0 = t0 + kt2 * 32;
        if (k0 + 32 > P) {
          // Tree or tail keys: prefix keys stay visible; tree key P+j needs
          // bit j of the row's ancestor bitset; keys >= L are hidden. The
          // 64-bit window of bitset words starting at wa covers every j the
          // lane tests (tree indices below 0 read as ones).
          const int jlo = k0 - P;
          const int wa = jlo >= 0 ? (jlo >> 5) : -1;
          const int jb = jlo - 32 * wa;
          const int nl = min((row0 + row) / p.G - first_node, nn_blk - 1);
          const uint32_t* arow = anc + nl * words;
          const uint32_t lo_w = arow[min(max(wa, 0), words - 1)];
          const uint32_t hi_w = arow[min(wa + 1, words - 1)];
          const uint32_t lo = wa < 0 ? ~0u : (wa < words ? lo_w : 0u);
          const uint32_t hi = wa + 1 < words ? hi_w : 0u;
          const uint64_t win = uint64_t(lo) | (uint64_t(hi) << 32);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int dk = lg * 8 + h * 4 + e;
              const bool vis = (k0 + dk < L) & (row < rows_here) & (((win >> (jb + dk)) & 1u) != 0);
              s[h][e] = vis ? s[h][e] : -INFINITY;
            }
          }
        }
        const float mloc = fmax_(fmax_(fmax_(s[0][0], s[0][1]), fmax_(s[0][2], s[0][3])),
                                 fmax_(fmax_(s[1][0], s[1][1]), fmax_(s[1][2], s[1][3])));
        const bool need = (mloc > m_ref) & ((m_ref == -INFINITY) | (cs * (mloc - m_ref) > kLazy));
        if (__builtin_amdgcn_ballot_w64(need)) {
          const float mt = max_across_groups(mloc);
          const bool raise = (mt > m_ref) & ((m_ref == -INFINITY) | (cs * (mt - m_ref) > kLazy));
          const float m_new = raise ? mt : m_ref;
          const float off_new = m_new == -INFINITY ? 0.f : cs * m_new;
          const float alpha = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(off_ - off_new);
          m_ref = m_new;
          off_ = off_new;
          l_run *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
        }
        bf16x8 pb;
        float ls = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float pv = __builtin_amdgcn_exp2f(fmaf(s[h][e], cs, -off_));
            ls += pv;
            pb[4 * h + e] = static_cast<__bf16>(pv);
          }
        }
        l_run += ls;
        if (k0 + 32 <= L) {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const bf16x8 va = *reinterpret_cast<const bf16x8*>(sb + kt2 * (2 * D * kPage) + dt * 256 + vaddr);
            acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, acc[dt], 0, 0, 0);
          }
        } else {
          // The sequence ends inside this half: V rows of keys >= L may hold
          // anything (unused slots, page 0), so they are zeroed before the
          // PV product (p is 0 there, but 0 * NaN is not).
          const int keep = L - (k0 + 8 * lg);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const uint4 raw = *reinterpret_cast<const uint4*>(sb + kt2 * (2 * D * kPage) + dt * 256 + vaddr);
            const bf16x8 va = __builtin_bit_cast(bf16x8, keep_first(raw, keep));
            acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, acc[dt], 0, 0, 0);
          }
        }
      }
    };

    // Prologue: stages tlo .. tlo+NS-2 in flight.
    static_for<0, NS - 1>([&](auto j_c) __attribute__((always_inline)) {
      constexpr int J = decltype(j_c)::value;
      issue(slot(j_c), load_id(tlo + J), tlo + J < thi);
    });
    int idn = load_id(tlo + NS - 1);  // page id of the next stage to issue

    // This wave's Q and parent loads have landed (the stages stay pending).
    wait_vm<(NS - 1) * NI>();
    // The ancestor bitsets are built while the first stages load.
    if (tree_keys) {
      stage_barrier();  // every wave's parent loads landed, the bitsets cleared
      link_anc(p, first_node, nn_blk, words, anc, par);
      stage_barrier();
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(qlds + kk * 512 + lane * 8);
      qf[kk] = active && row < rows_here ? v : bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }

    // Step i (stage i in slot J = (i - tlo) % NS): wait for this wave's
    // loads of stage i (NS-2 later stages stay pending), barrier (every
    // wave's loads landed; every wave is done with the slot of stage i-1),
    // issue stage i+NS-1 into that slot, compute stage i.
    auto step = [&](int i, auto j_c, auto nh_c) __attribute__((always_inline)) {
      constexpr int J = decltype(j_c)::value;
      wait_vm<(NS - 2) * NI>();
      stage_barrier();
      issue(slot(std::integral_constant<int, J + NS - 1>{}), idn, i + NS - 1 < thi);
      if (active) compute(slot(j_c), i, nh_c);
      idn = load_id(i + NS);
    };
    // Unrolled NS times so every slot is a compile-time object; the last
    // thi - i < NS stages run straight-line.
    auto run = [&](auto nh_c) __attribute__((always_inline)) {
      int i = tlo;
      for (; i + NS <= thi; i += NS)
        static_for<0, NS>([&](auto j_c) __attribute__((always_inline)) {
          step(i + decltype(j_c)::value, j_c, nh_c);
        });
      static_for<0, NS - 1>([&](auto j_c) __attribute__((always_inline)) {
        if (i + decltype(j_c)::value < thi) step(i + decltype(j_c)::value, j_c, nh_c);
      });
    };
    if (ksplit)
      run(std::integral_constant<int, 1>{});
    else
      run(std::integral_constant<int, 2>{});
    wait_vm<0>();  // the dummy stages have landed before the slots are reused
    if (bad_page) raise_status(p.status, TV_DEV_PAGES);

    // Row sums: the four lane groups of a row hold disjoint key subsets.
    l_run += shfl_xor(l_run, 16);
    l_run += shfl_xor(l_run, 32);

    // Key-split waves: the half-1 wave of a row tile hands (off, l, acc) to
    // the half-0 wave through LDS (slot 0; every stage load has landed).
    if (ksplit) {
      __syncthreads();
      float* xacc = reinterpret_cast<float*>(s0);  // [4 row tiles][16][D]
      if (active && half == 1) {
        float* dst = xacc + (rt * 16 + l16) * D + lg * 4;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(dst + dt * 16) = acc[dt];
        if (lg == 0) {
          s_xol[(rt * 16 + l16) * 2] = off_ + (m_ref == -INFINITY ? -INFINITY : 0.f);
          s_xol[(rt * 16 + l16) * 2 + 1] = l_run;
        }
      }
      __syncthreads();
      if (active && half == 0) {
        const float* src = xacc + (rt * 16 + l16) * D + lg * 4;
        const float o2 = s_xol[(rt * 16 + l16) * 2];
        const float l2 = s_xol[(rt * 16 + l16) * 2 + 1];
        const float o1 = m_ref == -INFINITY ? -INFINITY : off_;
        const float om = fmaxf(o1, o2);
        const float a1 = o1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(o1 - om);
        const float a2 = o2 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(o2 - om);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          acc[dt] = acc[dt] * a1 + *reinterpret_cast<const f32x4*>(src + dt * 16) * a2;
        l_run = l_run * a1 + l2 * a2;
        off_ = om == -INFINITY ? 0.f : om;
        m_ref = om;  // only its -inf-ness is used below
      }
      active = active && half == 0;
    }

    if (whole) {
      if (active && row < rows_here) {
        const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
        uint16_t* dst = static_cast<uint16_t*>(p.out) + qo_offset(p, nbeg, g, row0 + row, D) + lg * 4;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          uint2 pk;
          pk.x = pack_bf16x2(acc[dt][0] * inv, acc[dt][1] * inv);
          pk.y = pack_bf16x2(acc[dt][2] * inv, acc[dt][3] * inv);
          *reinterpret_cast<uint2*>(dst + dt * 16) = pk;
        }
      }
      continue;
    }

    // Cut pair: publish (offset, l, acc) of this share's part of it; the
    // offset is in log2 units (-inf when no key was visible).
    const size_t slot_id = cut_slot(lw, tlo);
    if (active && row < rows_here) {
      const size_t base = slot_id * kRowsPB + row;
      float* dst = p.part_o + base * D + lg * 4;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(dst + dt * 16) = acc[dt];
      if (lg == 0) {
        p.part_ml[base * 2] = m_ref == -INFINITY ? -INFINITY : off_;
        p.part_ml[base * 2 + 1] = l_run;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 VALU kernel: 256 threads, 32 rows per block, 32-key tiles; one
// workgroup per (request, kv head, row block, key split).

struct Item {
  int r, g, rb, c;
  int nbeg, N, P, L, R, row0, rows_here, nch, kbeg, kend, pbase;
  int first_node, nn;
  size_t slot, pair;
};

__device__ inline bool decode_item(const AttnParams& p, Item& it, int rows_pb) {
  const int per = gridDim.x >> 3;
  const int s = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (s >= p.grid_real) return false;
  it.rb = s % p.rb_max;
  int t = s / p.rb_max;
  it.c = t % p.c_max;
  t /= p.c_max;
  it.g = t % p.Hkv;
  it.r = t / p.Hkv;
  it.slot = s;
  it.pair = size_t(it.r) * p.Hkv * p.rb_max + size_t(it.g) * p.rb_max + it.rb;
  it.nbeg = p.node_indptr[it.r];
  it.N = p.node_indptr[it.r + 1] - it.nbeg;
  it.P = p.prefix_len[it.r];
  if (it.N <= 0) return false;
  if (it.N > p.max_nodes || it.P < 0 || it.P > p.max_kv_len - it.N) {
    if (threadIdx.x == 0 && it.rb == 0 && it.c == 0) raise_status(p.status, TV_DEV_SHAPE);
    return false;
  }
  it.L = it.P + it.N;
  it.R = it.N * p.G;
  it.row0 = it.rb * rows_pb;
  if (it.row0 >= it.R) return false;
  it.rows_here = min(rows_pb, it.R - it.row0);
  it.nch = ceil_div(it.L, p.chunk_len);
  if (it.c >= it.nch) return false;
  it.kbeg = it.c * p.chunk_len;
  it.kend = min(it.L, it.kbeg + p.chunk_len);
  it.pbase = p.page_indptr[it.r];
  const int npg = p.page_indptr[it.r + 1] - it.pbase;
  if (npg < ceil_div(it.L, kPage)) {
    if (threadIdx.x == 0 && it.c == 0 && it.rb == 0) raise_status(p.status, TV_DEV_PAGES);
    return false;
  }
  it.first_node = it.row0 / p.G;
  it.nn = (it.row0 + it.rows_here - 1) / p.G - it.first_node + 1;
  return true;
}

template <int D>
__global__ __launch_bounds__(256) void attn_valu_kernel(AttnParams p) {
  constexpr int ROWS_PB = 32;
  constexpr int TK = 32;
  constexpr int EPT = ROWS_PB * D / 256;  // output elements per thread
  __shared__ float q_lds[ROWS_PB][D + 1];
  __shared__ float k_lds[TK][D + 1];
  __shared__ float v_lds[TK][D];
  __shared__ float s_lds[ROWS_PB][TK + 1];
  __shared__ float s_alpha[ROWS_PB];
  __shared__ float s_m[ROWS_PB];
  __shared__ float s_l[ROWS_PB];
  __shared__ float s_M[ROWS_PB];
  __shared__ float s_invL[ROWS_PB];
  __shared__ int s_last;
  extern __shared__ uint32_t anc_lds[];  // [nn][words], then [max_nodes] parents

  Item it;
  if (!decode_item(p, it, ROWS_PB)) return;
  const int tid = threadIdx.x;
  const int words = ceil_div(it.N, 32);
  if (it.kend > it.P) {
    int* par = reinterpret_cast<int*>(anc_lds + (ROWS_PB / p.G + 2) * p.words);
    build_anc(p, it.nbeg, it.N, it.first_node, it.nn, words, anc_lds, par);
    __syncthreads();
  }

  const float* qf = static_cast<const float*>(p.q);
  const float* kp = static_cast<const float*>(p.k_pages);
  const float* vp = static_cast<const float*>(p.v_pages);
  for (int idx = tid; idx < ROWS_PB * D; idx += 256) {
    const int row = idx / D, d = idx - (idx / D) * D;
    q_lds[row][d] =
        (row < it.rows_here) ? qf[qo_offset(p, it.nbeg, it.g, it.row0 + row, D) + d] : 0.f;
  }
  if (tid < ROWS_PB) {
    s_m[tid] = -INFINITY;
    s_l[tid] = 0.f;
  }
  float o[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) o[i] = 0.f;

  const size_t head_block = size_t(kPage) * D;
  for (int t0 = it.kbeg; t0 < it.kend; t0 += TK) {
    __syncthreads();
    for (int idx = tid; idx < TK * D; idx += 256) {
      const int kl = idx / D, d = idx - (idx / D) * D;
      const int key = t0 + kl;
      float kv = 0.f, vv = 0.f;
      if (key < it.kend) {
        int phys = p.page_indices[it.pbase + (key >> 4)];
        if (unsigned(phys) >= unsigned(p.num_pages)) {
          raise_status(p.status, TV_DEV_PAGES);
          phys = 0;
        }
        const size_t base = (size_t(phys) * p.Hkv + it.g) * head_block;
        kv = kp[base + size_t(key & 15) * D + d];
        vv = vp[base + size_t(d) * kPage + (key & 15)];
      }
      k_lds[kl][d] = kv;
      v_lds[kl][d] = vv;
    }
    __syncthreads();
    {
      const int kl = tid & (TK - 1);
      const int key = t0 + kl;
      for (int row = tid >> 5; row < ROWS_PB; row += 256 / TK) {
        float acc = 0.f;
        for (int d = 0; d < D; ++d) acc = fmaf(q_lds[row][d], k_lds[kl][d], acc);
        float v = acc * p.scale_log2;
        bool vis = row < it.rows_here && key < it.kend;
        if (vis && key >= it.P) {
          const int j = key - it.P;
          const int nl = (it.row0 + row) / p.G - it.first_node;
          vis = (anc_lds[nl * words + (j >> 5)] >> (j & 31)) & 1u;
        }
        s_lds[row][kl] = vis ? v : -INFINITY;
      }
    }
    __syncthreads();
    if (tid < ROWS_PB) {
      const int row = tid;
      float mt = -INFINITY;
      for (int k = 0; k < TK; ++k) mt = fmaxf(mt, s_lds[row][k]);
      const float m_new = fmaxf(s_m[row], mt);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2f(s_m[row] - m_use);
      float ls = 0.f;
      for (int k = 0; k < TK; ++k) {
        const float pv = exp2f(s_lds[row][k] - m_use);
        s_lds[row][k] = pv;
        ls += pv;
      }
      s_l[row] = s_l[row] * alpha + ls;
      s_m[row] = m_new;
      s_alpha[row] = alpha;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int idx = tid + 256 * i;
      const int row = idx / D, d = idx - (idx / D) * D;
      float a = o[i] * s_alpha[row];
      for (int k = 0; k < TK; ++k) a = fmaf(s_lds[row][k], v_lds[k][d], a);
      o[i] = a;
    }
  }
  __syncthreads();

  if (it.nch == 1) {
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int idx = tid + 256 * i;
      const int row = idx / D, d = idx - (idx / D) * D;
      if (row < it.rows_here) {
        const float l = s_l[row];
        static_cast<float*>(p.out)[qo_offset(p, it.nbeg, it.g, it.row0 + row, D) + d] =
            l > 0.f ? o[i] / l : 0.f;
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int idx = tid + 256 * i;
    const int row = idx / D, d = idx - (idx / D) * D;
    if (row < it.rows_here) p.part_o[(it.slot * ROWS_PB + row) * D + d] = o[i];
  }
  if (tid < it.rows_here) {
    p.part_ml[(it.slot * ROWS_PB + tid) * 2] = s_m[tid];
    p.part_ml[(it.slot * ROWS_PB + tid) * 2 + 1] = s_l[tid];
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = atomicAdd(&p.counters[it.pair], 1u);
    const bool last = old == uint32_t(it.nch - 1);
    if (last) p.counters[it.pair] = 0u;
    s_last = last ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  // Merge the splits of this (request, kv head, row block) in split order.
  auto chunk_slot = [&](int c) {
    return ((size_t(it.r) * p.Hkv + it.g) * p.c_max + c) * p.rb_max + it.rb;
  };
  for (int row = tid; row < it.rows_here; row += 256) {
    float M = -INFINITY;
    for (int c = 0; c < it.nch; ++c) M = fmaxf(M, p.part_ml[(chunk_slot(c) * ROWS_PB + row) * 2]);
    float L = 0.f;
    if (M != -INFINITY)
      for (int c = 0; c < it.nch; ++c) {
        const float* ml = p.part_ml + (chunk_slot(c) * ROWS_PB + row) * 2;
        L += ml[1] * exp2f(ml[0] - M);
      }
    s_M[row] = M;
    s_invL[row] = L > 0.f ? 1.f / L : 0.f;
  }
  __syncthreads();
  for (int idx = tid; idx < it.rows_here * D; idx += 256) {
    const int row = idx / D, d = idx - (idx / D) * D;
    const float M = s_M[row];
    float acc = 0.f;
    if (M != -INFINITY)
      for (int c = 0; c < it.nch; ++c) {
        const size_t base = chunk_slot(c) * ROWS_PB + row;
        acc += exp2f(p.part_ml[base * 2] - M) * p.part_o[base * D + d];
      }
    static_cast<float*>(p.out)[qo_offset(p, it.nbeg, it.g, it.row0 + row, D) + d] =
        acc * s_invL[row];
  }
}

}  // namespace

bool plan_attn(const tv_attn_desc& d, AttnPlan* out) {
  AttnPlan pl{};
  if (d.batch < 1 || d.num_kv_heads < 1 || d.num_q_heads < d.num_kv_heads ||
      d.num_q_heads % d.num_kv_heads != 0 || (d.head_dim != 64 && d.head_dim != 128) ||
      d.page_size != kPage || d.max_nodes < 1 || d.max_nodes > 1024 || d.max_kv_len < 1 ||
      d.max_kv_len < d.max_nodes || d.num_pages < 1 || d.max_depth < 0 ||
      (d.dtype != TV_BF16 && d.dtype != TV_FP32))
    return false;
  pl.mfma = d.dtype == TV_BF16;
  pl.group = d.num_q_heads / d.num_kv_heads;
  pl.rows_pb = pl.mfma ? kRowsPB : 32;
  const long long rows = (long long)d.max_nodes * pl.group;
  pl.rb_max = int((rows + pl.rows_pb - 1) / pl.rows_pb);
  pl.words = (d.max_nodes + 31) / 32;
  const long long pairs = (long long)d.batch * d.num_kv_heads * pl.rb_max;
  size_t off = kHeaderBytes;
  pl.off_counters = off;
  off = align256(off + size_t(pairs) * sizeof(uint32_t));
  if (pl.mfma) {
    if (d.batch > 4096) return false;  // tile offsets live in LDS
    const long long tiles = pairs * ((d.max_kv_len + kStage - 1) / kStage);
    if (tiles * kCostBig + pairs * kCostPair > 0x7fffffffLL) return false;  // units fit an int
    // A power of two (>= 8, the XCD count) so share bounds are shifts.
    long long want = (tiles + kMinTilesPerWG - 1) / kMinTilesPerWG;
    if (want > kMaxWG) want = kMaxWG;
    long long nwg = 8;
    int lg = 3;
    while (nwg < want) {
      nwg *= 2;
      ++lg;
    }
    pl.nwg = int(nwg);
    pl.lg_nwg = lg;
    pl.grid = size_t(nwg);
    pl.slots = 2 * size_t(nwg);
    const int nn_max = kRowsPB / pl.group + 2;
    pl.dyn_lds = size_t(d.batch + 1 + ((d.max_nodes + 63) & ~63)) * sizeof(int) +  // parents by 64
                 size_t(nn_max) * pl.words * sizeof(uint32_t);
    // Stage ring depth: four 64-key slots when they fit next to the
    // dynamic arrays in the 160 KB of LDS, else two.
    const size_t slot_bytes = size_t(2) * kStage * d.head_dim * sizeof(uint16_t);
    const size_t fixed = 4 * 16 * 2 * sizeof(float) + kWavesS * sizeof(int);
    pl.ns = (4 * slot_bytes + fixed + pl.dyn_lds <= kLdsBytes) ? 4 : 2;
    if (2 * slot_bytes + fixed + pl.dyn_lds > kLdsBytes) return false;
  } else {
    const long long target_items = 1024;
    long long chunk = ((long long)d.max_kv_len * pairs + target_items - 1) / target_items;
    chunk = chunk < 128 ? 128 : chunk;
    chunk = (chunk + 31) / 32 * 32;
    const long long full = ((long long)d.max_kv_len + 31) / 32 * 32;
    if (chunk > full) chunk = full;
    pl.chunk_len = int(chunk);
    pl.c_max = int((d.max_kv_len + chunk - 1) / chunk);
    pl.slots = size_t(pairs) * pl.c_max;
    pl.grid = (pl.slots + 7) / 8 * 8;
    if (pl.grid > 0x7fffffffULL) return false;
    const int nn_max = pl.rows_pb / pl.group + 2;
    pl.dyn_lds = size_t(nn_max) * pl.words * sizeof(uint32_t) + size_t(d.max_nodes) * sizeof(int);
  }
  pl.off_desc = off;
  off = align256(off + (pl.mfma ? size_t(pl.nwg) * 3 * sizeof(int4) : 0));
  pl.off_ml = off;
  off = align256(off + pl.slots * pl.rows_pb * 2 * sizeof(float));
  pl.off_o = off;
  off = align256(off + pl.slots * pl.rows_pb * size_t(d.head_dim) * sizeof(float));
  pl.total_bytes = off;
  *out = pl;
  return true;
}

hipError_t launch_attn(const tv_attn_desc& d, const AttnPlan& pl, const AttnArgs& a,
                       hipStream_t stream) {
  AttnParams p{};
  p.q = a.q;
  p.k_pages = a.k_pages;
  p.v_pages = a.v_pages;
  p.page_indptr = a.page_indptr;
  p.page_indices = a.page_indices;
  p.prefix_len = a.prefix_len;
  p.node_indptr = a.node_indptr;
  p.parent = a.parent;
  p.out = a.out;
  char* ws = static_cast<char*>(a.workspace);
  p.status = reinterpret_cast<uint32_t*>(ws);
  p.counters = reinterpret_cast<uint32_t*>(ws + pl.off_counters);
  p.merge_desc = reinterpret_cast<int4*>(ws + pl.off_desc);
  p.part_ml = reinterpret_cast<float*>(ws + pl.off_ml);
  p.part_o = reinterpret_cast<float*>(ws + pl.off_o);
  p.B = d.batch;
  p.Hq = d.num_q_heads;
  p.Hkv = d.num_kv_heads;
  p.G = pl.group;
  p.num_pages = d.num_pages;
  p.max_nodes = d.max_nodes;
  p.max_kv_len = d.max_kv_len;
  p.words = pl.words;
  p.rb_max = pl.rb_max;
  p.c_max = pl.c_max;
  p.chunk_len = pl.chunk_len;
  p.grid_real = int(pl.slots);
  p.nwg = pl.nwg;
  p.lg_nwg = pl.lg_nwg;
  const float scale = d.sm_scale > 0.f ? d.sm_scale : 1.f / sqrtf(float(d.head_dim));
  p.scale_log2 = scale * kLog2e;
  const dim3 grid(unsigned(pl.grid)), block(256);
  const size_t lds = pl.dyn_lds;
  if (pl.mfma) {
    // Streaming pass (whole pairs written, cut pairs left as partials), then
    // the merge of the cut pairs; the kernel boundary orders the two.
    const dim3 mgrid(unsigned(pl.nwg) * (kRowsPB / 16));
    const dim3 sblock(kThreadsS);
    if (d.head_dim == 128) {
      if (pl.ns == 4)
        attn_stream_kernel<128, 4><<<grid, sblock, lds, stream>>>(p, a.page_indices, a.node_indptr, a.prefix_len, a.page_indptr);
      else
        attn_stream_kernel<128, 2><<<grid, sblock, lds, stream>>>(p, a.page_indices, a.node_indptr, a.prefix_len, a.page_indptr);
      hipLaunchKernelGGL(attn_merge_kernel<128>, mgrid, block, 0, stream, p);
    } else {
      if (pl.ns == 4)
        attn_stream_kernel<64, 4><<<grid, sblock, lds, stream>>>(p, a.page_indices, a.node_indptr, a.prefix_len, a.page_indptr);
      else
        attn_stream_kernel<64, 2><<<grid, sblock, lds, stream>>>(p, a.page_indices, a.node_indptr, a.prefix_len, a.page_indptr);
      hipLaunchKernelGGL(attn_merge_kernel<64>, mgrid, block, 0, stream, p);
    }
  } else {
    if (d.head_dim == 128)
      hipLaunchKernelGGL(attn_valu_kernel<128>, grid, block, lds, stream, p);
    else
      hipLaunchKernelGGL(attn_valu_kernel<64>, grid, block, lds, stream, p);
  }
  return hipGetLastError();
}

}  // namespace tv
