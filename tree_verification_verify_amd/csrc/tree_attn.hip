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
//    A fixed grid of persistent workgroups splits that list into equal
//    contiguous shares (stream-K), so uneven prefixes balance exactly. A
//    pair wholly inside one share is finished in registers and written out;
//    a pair cut by share boundaries leaves fp32 partials (offset, l, acc),
//    which a second, small kernel merges in share order (deterministic; the
//    kernel boundary makes the partials visible, so the streaming kernel
//    needs no fences, counters or waiting). Shares are laid out XCD by XCD,
//    so the row blocks of one kv head run on one XCD and share its L2.
//  * 4 waves x 32 rows. S^T = K Q^T and O^T += V^T P^T on
//    v_mfma_f32_16x16x32_bf16; both keep a row on lane%16, so the online
//    softmax rescale is lane-local and P never leaves registers (the PV key
//    order is permuted to match the S^T accumulator layout).
//  * V pages are stored transposed ([D][16] per page and head), so every
//    16-byte global load lands in LDS unchanged and each MFMA operand is two
//    8-byte LDS reads; K tiles are stored as loaded ([key][D], padded rows).
//  * Loads of the next 64-key stage are issued before the MFMA work on the
//    current one (register staging, LDS double buffer).
//  * The ancestor mask is a per-node bitset built in LDS when a segment
//    reaches the tree's own keys, and consulted only in those tiles.
// fp32 path (small validation shapes): a VALU kernel, one workgroup per
// (request, kv head, row block, key split), with the same partial format.
#include "tv_device.hpp"
#include "tv_internal.hpp"

namespace tv {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kRowsPB = 128;     // rows per row block (bf16 path)
constexpr int kStage = 64;       // keys per stage / tile (bf16 path)
constexpr int kMaxWG = 512;      // persistent workgroups: 2 per CU on 256 CUs
constexpr int kMinTilesPerWG = 2;

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
// (nn rows of `words`), walking parent links staged in LDS (`par`, the
// request's N parents). Caller synchronises before and after.
__device__ inline void build_anc(const AttnParams& p, int nbeg, int N, int first_node, int nn,
                                 int words, uint32_t* anc, int* par) {
  for (int i = threadIdx.x; i < nn * words; i += blockDim.x) anc[i] = 0u;
  for (int i = threadIdx.x; i < N; i += blockDim.x) par[i] = p.parent[nbeg + i];
  __syncthreads();
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

// Tiles of request r (all kv heads and row blocks); 0 for an empty or
// rejected request (rejections are reported once, by `report`).
__device__ inline int request_tiles(const AttnParams& p, int r, bool report) {
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
  return p.Hkv * ceil_div(N * p.G, kRowsPB) * ceil_div(L, kStage);
}

// Share [a_w, b_w) of the T tiles given to logical workgroup w of n = 2^lg.
__device__ inline int share_begin(int T, int w, int lg) {
  return int((uint64_t(T) * uint32_t(w)) >> lg);
}

// Logical workgroup whose share contains tile x (x < T): the largest w with
// share_begin(w) <= x.
__device__ inline int share_of(int T, int x, int lg) {
  const int n = 1 << lg;
  int w = int(float(x) * float(n) / float(T));
  w = min(max(w, 0), n - 1);
  while (w > 0 && share_begin(T, w, lg) > x) --w;
  while (w + 1 < n && share_begin(T, w + 1, lg) <= x) ++w;
  return w;
}

// Partial slot of logical workgroup w for a pair starting at tile ps: a
// share holds at most two cut pairs, the one it starts inside (slot 2w) and
// the one it ends inside (slot 2w+1).
__device__ inline size_t cut_slot(int T, int w, int lg, int ps) {
  return ps < share_begin(T, w, lg) ? size_t(2 * w) : size_t(2 * w + 1);
}

// Block-wide tile offsets of every request: off[r] = first tile of request
// r in the flat (request, kv head, row block, tile) order, off[B] = T.
// Rejected requests (reported once when `report`) contribute no tiles.
__device__ inline int scan_tiles(const AttnParams& p, int* off, int* s_scan, bool report) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = ceil_div(p.B, 256);
  const int r0 = min(p.B, tid * per), r1 = min(p.B, r0 + per);
  int mine = 0;
  for (int r = r0; r < r1; ++r) {
    const int t = request_tiles(p, r, report);
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
#pragma unroll
  for (int w = 0; w < 4; ++w) {
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

// Merge kernel: workgroup w merges the cut pair whose first inner share
// boundary is a_w (a_{w-1} <= ps < a_w < pe), combining the partials of
// every share that holds part of it, in share order (deterministic).
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnParams p) {
  constexpr int D4 = D / 4;
  constexpr int IPT = kRowsPB * D4 / 256;  // float4 items per thread
  __shared__ float s_M[kRowsPB];
  __shared__ float s_invL[kRowsPB];
  __shared__ int s_scan[4];
  extern __shared__ int off[];  // [B + 1]
  const int w = blockIdx.x;
  if (w == 0) return;
  const int T = scan_tiles(p, off, s_scan, false);
  const int aw = share_begin(T, w, p.lg_nwg);
  if (aw >= T) return;
  const int r = request_of(off, p.B, aw);
  const int nbeg = p.node_indptr[r];
  const int N = p.node_indptr[r + 1] - nbeg;
  const int L = p.prefix_len[r] + N;
  const int R = N * p.G;
  const int nrb = ceil_div(R, kRowsPB);
  const int nt = ceil_div(L, kStage);
  const int pir = (aw - off[r]) / nt;
  const int ps = off[r] + pir * nt, pe = ps + nt;
  if (!(ps < aw && share_begin(T, w - 1, p.lg_nwg) <= ps)) return;
  const int g = pir / nrb;
  const int row0 = (pir - g * nrb) * kRowsPB;
  const int rows_here = min(kRowsPB, R - row0);
  const int w0 = share_of(T, ps, p.lg_nwg), w1 = share_of(T, pe - 1, p.lg_nwg);

  for (int row = threadIdx.x; row < rows_here; row += blockDim.x) {
    float M = -INFINITY;
    for (int v = w0; v <= w1; ++v) {
      if (share_begin(T, v + 1, p.lg_nwg) == share_begin(T, v, p.lg_nwg)) continue;
      M = fmaxf(M, p.part_ml[(cut_slot(T, v, p.lg_nwg, ps) * kRowsPB + row) * 2]);
    }
    float Ls = 0.f;
    if (M != -INFINITY) {
      for (int v = w0; v <= w1; ++v) {
        if (share_begin(T, v + 1, p.lg_nwg) == share_begin(T, v, p.lg_nwg)) continue;
        const float* ml = p.part_ml + (cut_slot(T, v, p.lg_nwg, ps) * kRowsPB + row) * 2;
        Ls += ml[1] * exp2f(ml[0] - M);
      }
    }
    s_M[row] = M;
    s_invL[row] = Ls > 0.f ? 1.f / Ls : 0.f;
  }
  __syncthreads();
  float4 acc[IPT];
#pragma unroll
  for (int k = 0; k < IPT; ++k) acc[k] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int v = w0; v <= w1; ++v) {
    if (share_begin(T, v + 1, p.lg_nwg) == share_begin(T, v, p.lg_nwg)) continue;
    const size_t slot = cut_slot(T, v, p.lg_nwg, ps);
    float4 o[IPT];
    float m[IPT];
#pragma unroll
    for (int k = 0; k < IPT; ++k) {  // all loads of this share first
      const int idx = threadIdx.x + 256 * k;
      const int row = idx / D4;
      const size_t base = slot * kRowsPB + row;
      o[k] = row < rows_here ? *reinterpret_cast<const float4*>(p.part_o + base * D + (idx - row * D4) * 4)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
      m[k] = row < rows_here ? p.part_ml[base * 2] : -INFINITY;
    }
#pragma unroll
    for (int k = 0; k < IPT; ++k) {
      const int row = (threadIdx.x + 256 * k) / D4;
      const float Mr = row < rows_here ? s_M[row] : -INFINITY;
      const float sc = (m[k] == -INFINITY) ? 0.f : exp2f(m[k] - Mr);
      acc[k].x += sc * o[k].x;
      acc[k].y += sc * o[k].y;
      acc[k].z += sc * o[k].z;
      acc[k].w += sc * o[k].w;
    }
  }
#pragma unroll
  for (int k = 0; k < IPT; ++k) {
    const int idx = threadIdx.x + 256 * k;
    const int row = idx / D4;
    if (row >= rows_here) continue;
    const float inv = s_invL[row];
    uint2 pk;
    pk.x = pack_bf16x2(acc[k].x * inv, acc[k].y * inv);
    pk.y = pack_bf16x2(acc[k].z * inv, acc[k].w * inv);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + qo_offset(p, nbeg, g, row0 + row, D) +
                              (idx - row * D4) * 4) = pk;
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel: 256 threads = 4 waves x 32 rows; persistent over tiles.
template <int D>
__global__ __launch_bounds__(256, 2) void attn_stream_kernel(AttnParams p) {
  constexpr int KK = D / 32;          // 32-wide k-steps of the QK product
  constexpr int DT = D / 16;          // 16-wide d tiles of the PV product
  constexpr int KS = D + 8;           // LDS row stride of K (bf16 elements)
  constexpr int VS = kStage + 4;      // LDS row stride of V^T: 34 words, so the 8-byte operand
                                      // reads of 16 (32) lanes hit distinct banks with 32 (64) banks
  constexpr int PCH = 2 * D;          // 16-byte chunks per (page, head) block
  constexpr int CPT = 4 * PCH / 256;  // chunks per thread per stage (K, and V)
  constexpr int DB = D / 8;           // 16-byte chunks per K row

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][kStage * KS];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][D * VS];
  __shared__ int s_scan[4];
  extern __shared__ int dyn_lds[];
  int* off = dyn_lds;                                                 // [B + 1]
  int* par = dyn_lds + p.B + 1;                                       // [max_nodes]
  uint32_t* anc = reinterpret_cast<uint32_t*>(par + p.max_nodes);     // [nn][words]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int l16 = lane & 15;
  const int lg = lane >> 4;
  const int lw = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);

  const int T = scan_tiles(p, off, s_scan, lw == 0);
  const int a = share_begin(T, lw, p.lg_nwg);
  const int b = share_begin(T, lw + 1, p.lg_nwg);
  if (a >= b) return;

  int r = request_of(off, p.B, a);  // request holding tile a

  const uint16_t* qb = static_cast<const uint16_t*>(p.q);
  const uint16_t* kp = static_cast<const uint16_t*>(p.k_pages);
  const uint16_t* vp = static_cast<const uint16_t*>(p.v_pages);
  const size_t head_block = size_t(kPage) * D;  // elements per (page, head)

  int c = a;
  while (c < b) {
    while (off[r + 1] <= c) ++r;
    const int nbeg = p.node_indptr[r];
    const int N = p.node_indptr[r + 1] - nbeg;
    const int P = p.prefix_len[r];
    const int L = P + N;
    const int R = N * p.G;
    const int nrb = ceil_div(R, kRowsPB);
    const int nt = ceil_div(L, kStage);
    const int local = c - off[r];
    const int pir = local / nt;
    const int g = pir / nrb;
    const int rb = pir - g * nrb;
    const int ps = off[r] + pir * nt;  // pair's first tile
    const int pe = ps + nt;            // pair's end tile
    const int seg_end = min(b, pe);
    const int tlo = c - ps, thi = seg_end - ps;
    const bool whole = ps >= a && pe <= b;
    const int row0 = rb * kRowsPB;
    const int rows_here = min(kRowsPB, R - row0);
    const int pbase = p.page_indptr[r];
    const int words = ceil_div(N, 32);
    const int first_node = row0 / p.G;
    const int nn_blk = (row0 + rows_here - 1) / p.G - first_node + 1;
    c = seg_end;

    __syncthreads();  // LDS of the previous segment is no longer read
    if (thi * kStage > P) build_anc(p, nbeg, N, first_node, nn_blk, words, anc, par);

    // Wave roles. Row tile t holds block rows 16t..16t+15. With five or
    // more row tiles each wave takes two (rtA, rtB) and every key; with
    // three or four, one each; with one or two row tiles the waves also
    // split the 64 keys of a stage into 32-key halves (hmask), and the two
    // halves of a row tile are merged through LDS at the end of the segment.
    const int nrt = ceil_div(rows_here, 16);
    int rtA, rtB, hmask;
    if (nrt >= 5) {
      rtA = 2 * wave < nrt ? 2 * wave : -1;
      rtB = 2 * wave + 1 < nrt ? 2 * wave + 1 : -1;
      hmask = 3;
    } else if (nrt >= 3) {
      rtA = wave < nrt ? wave : -1;
      rtB = -1;
      hmask = 3;
    } else if (nrt == 2) {
      rtA = wave & 1;
      rtB = -1;
      hmask = 1 << (wave >> 1);
    } else {
      rtA = wave < 2 ? 0 : -1;
      rtB = -1;
      hmask = 1 << (wave & 1);
    }
    const bool ksplit = nrt <= 2;
    bool active = rtA >= 0;
    const bool two = rtB >= 0;
    const int rowA = rtA * 16 + l16;  // block-local rows of this lane
    const int rowB = rtB * 16 + l16;

    bf16x8 qf[2][KK];
#pragma unroll
    for (int w2 = 0; w2 < 2; ++w2) {
      const int row = w2 == 0 ? rowA : rowB;
      const bool ok = (w2 == 0 ? rtA >= 0 : two) && row < rows_here;
      if (ok) {
        const uint16_t* src = qb + qo_offset(p, nbeg, g, row0 + row, D) + lg * 8;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qf[w2][kk] = *reinterpret_cast<const bf16x8*>(src + kk * 32);
      } else {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qf[w2][kk] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }

    // Stage loads: thread chunk j covers 16 bytes of page (j*256+tid)/PCH of
    // the stage, at the same offset in its K and its V^T block. Loads never
    // branch: a page past the sequence is read from page 0 and, like slots
    // past the sequence in the last page, zeroed when it is committed to LDS.
    const int pend = p.page_indptr[r + 1] - 1;  // last listed page (>= pbase)
    uint4 kreg[CPT], vreg[CPT];
    int ids[4];         // raw page ids of the next stage to issue (unchecked)
    bool bad_page = false;
    auto page_ids = [&](int tile) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        ids[j] = p.page_indices[min(pbase + ((tile * kStage + j * kPage) >> 4), pend)];
    };
    auto issue = [&](int tile) {
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int cidx = tid + 256 * j;
        const int pg = cidx / PCH;
        const int o = cidx - pg * PCH;
        int id = pg == 0 ? ids[0] : pg == 1 ? ids[1] : pg == 2 ? ids[2] : ids[3];
        const bool live = tile * kStage + pg * kPage < L;
        const bool in_pool = unsigned(id) < unsigned(p.num_pages);
        bad_page |= live && !in_pool;
        id = (live && in_pool) ? id : 0;
        const size_t blk = (size_t(id) * p.Hkv + g) * head_block + size_t(o) * 8;
        kreg[j] = *reinterpret_cast<const uint4*>(kp + blk);
        vreg[j] = *reinterpret_cast<const uint4*>(vp + blk);
      }
    };
    auto commit = [&](int buf, int tile) {
      const int tail = L - tile * kStage;  // keys of this tile inside the sequence
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int cidx = tid + 256 * j;
        const int pg = cidx / PCH;
        const int o = cidx - pg * PCH;
        const int kip = o / DB;
        uint4 kv = kreg[j], vv = vreg[j];
        if (tail < kStage) {
          kv = pg * kPage + kip < tail ? kv : make_uint4(0, 0, 0, 0);
          vv = keep_first(vv, tail - (pg * kPage + (o & 1) * 8));
        }
        *reinterpret_cast<uint4*>(&k_lds[buf][(pg * kPage + kip) * KS + (o - kip * DB) * 8]) = kv;
        uint2* vdst = reinterpret_cast<uint2*>(&v_lds[buf][(o >> 1) * VS + pg * kPage + (o & 1) * 8]);
        vdst[0] = make_uint2(vv.x, vv.y);  // rows are 8-byte aligned only
        vdst[1] = make_uint2(vv.z, vv.w);
      }
    };

    // Online softmax state per row (w2 = 0: rtA, 1: rtB). Scores stay raw
    // dot products; the exponent is exp2(c*s - off) with c = scale*log2(e)
    // and off = c*m_ref. The reference m_ref is raised only when a new raw
    // max exceeds it by more than kLazy/c (then acc and l are rescaled), so
    // p <= 2^kLazy and most tiles skip the rescale.
    constexpr float kLazy = 8.f;
    const float c = p.scale_log2;
    float m_ref[2] = {-INFINITY, -INFINITY};
    float off_[2] = {0.f, 0.f};
    float l_run[2] = {0.f, 0.f};
    f32x4 acc[DT][2];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      acc[dt][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc[dt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    page_ids(tlo);
    issue(tlo);
    if (tlo + 1 < thi) page_ids(tlo + 1);
    commit(0, tlo);
    if (tlo + 1 < thi) {
      issue(tlo + 1);
      if (tlo + 2 < thi) page_ids(tlo + 2);
    }
    __syncthreads();
    int buf = 0;
    for (int tile = tlo; tile < thi; ++tile) {
      const int t0 = tile * kStage;
      if (active) {
#pragma unroll
        for (int kt2 = 0; kt2 < 2; ++kt2) {
          if (!((hmask >> kt2) & 1)) continue;
          f32x4 s[2][2];  // [16-key half][w2]
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            s[h][0] = f32x4{0.f, 0.f, 0.f, 0.f};
            s[h][1] = f32x4{0.f, 0.f, 0.f, 0.f};
            const uint16_t* krow = &k_lds[buf][((2 * kt2 + h) * 16 + l16) * KS + lg * 8];
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
              const bf16x8 ka = *reinterpret_cast<const bf16x8*>(krow + kk * 32);
              s[h][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[0][kk], s[h][0], 0, 0, 0);
              if (two)
                s[h][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[1][kk], s[h][1], 0, 0, 0);
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
#pragma unroll
            for (int w2 = 0; w2 < 2; ++w2) {
              if (w2 == 1 && !two) continue;
              const int row = w2 == 0 ? rowA : rowB;
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
                  const int dk = h * 16 + lg * 4 + e;
                  const bool vis = (k0 + dk < L) & (row < rows_here) &
                                   (((win >> (jb + dk)) & 1u) != 0);
                  s[h][w2][e] = vis ? s[h][w2][e] : -INFINITY;
                }
              }
            }
          }
          bf16x8 pb[2];
#pragma unroll
          for (int w2 = 0; w2 < 2; ++w2) {
            if (w2 == 1 && !two) continue;
            float mt = fmaxf(fmaxf(fmaxf(s[0][w2][0], s[0][w2][1]), fmaxf(s[0][w2][2], s[0][w2][3])),
                             fmaxf(fmaxf(s[1][w2][0], s[1][w2][1]), fmaxf(s[1][w2][2], s[1][w2][3])));
            mt = fmaxf(mt, shfl_xor(mt, 16));
            mt = fmaxf(mt, shfl_xor(mt, 32));
            // Raise the reference when the row max passed it by > kLazy/c.
            const bool raise = mt > m_ref[w2] && (m_ref[w2] == -INFINITY || c * (mt - m_ref[w2]) > kLazy);
            if (__builtin_amdgcn_ballot_w64(raise)) {
              const float m_new = raise ? mt : m_ref[w2];
              const float off_new = m_new == -INFINITY ? 0.f : c * m_new;
              const float alpha = m_ref[w2] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(off_[w2] - off_new);
              m_ref[w2] = m_new;
              off_[w2] = off_new;
              l_run[w2] *= alpha;
#pragma unroll
              for (int dt = 0; dt < DT; ++dt) acc[dt][w2] *= alpha;
            }
            float ls = 0.f;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float pv = __builtin_amdgcn_exp2f(fmaf(s[h][w2][e], c, -off_[w2]));
                ls += pv;
                pb[w2][4 * h + e] = static_cast<__bf16>(pv);
              }
            }
            l_run[w2] += ls;
          }
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const uint16_t* vrow = &v_lds[buf][(dt * 16 + l16) * VS + kt2 * 32 + lg * 4];
            const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
            const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16);
            const uint4 w4 = make_uint4(lo.x, lo.y, hi.x, hi.y);
            const bf16x8 va = __builtin_bit_cast(bf16x8, w4);
            acc[dt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[0], acc[dt][0], 0, 0, 0);
            if (two)
              acc[dt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[1], acc[dt][1], 0, 0, 0);
          }
        }
      }
      if (tile + 1 < thi) {
        commit(buf ^ 1, tile + 1);
        if (tile + 2 < thi) {
          issue(tile + 2);
          if (tile + 3 < thi) page_ids(tile + 3);
        }
      }
      __syncthreads();
      buf ^= 1;
    }
    if (bad_page) raise_status(p.status, TV_DEV_PAGES);

    // Row sums: the four lane groups of a row hold disjoint key subsets.
#pragma unroll
    for (int w2 = 0; w2 < 2; ++w2) {
      float l = l_run[w2];
      l += shfl_xor(l, 16);
      l += shfl_xor(l, 32);
      l_run[w2] = l;
    }

    // Key-split waves: the second-half wave of a row tile hands (off, l, acc)
    // to the first-half wave through LDS (the stage buffers are free now).
    if (ksplit) {
      float* xacc = reinterpret_cast<float*>(&k_lds[0][0]);  // [2 row tiles][16][D]
      float* xol = xacc + 2 * 16 * D;                        // [2][16][2]
      if (active && hmask == 2) {
        float* dst = xacc + (rtA * 16 + l16) * D + lg * 4;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          *reinterpret_cast<f32x4*>(dst + dt * 16) = acc[dt][0];
        if (lg == 0) {
          xol[(rtA * 16 + l16) * 2] = off_[0] + (m_ref[0] == -INFINITY ? -INFINITY : 0.f);
          xol[(rtA * 16 + l16) * 2 + 1] = l_run[0];
        }
      }
      __syncthreads();
      if (active && hmask == 1) {
        const float* src = xacc + (rtA * 16 + l16) * D + lg * 4;
        const float o2 = xol[(rtA * 16 + l16) * 2];
        const float l2 = xol[(rtA * 16 + l16) * 2 + 1];
        const float o1 = m_ref[0] == -INFINITY ? -INFINITY : off_[0];
        const float om = fmaxf(o1, o2);
        const float a1 = o1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(o1 - om);
        const float a2 = o2 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(o2 - om);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          acc[dt][0] = acc[dt][0] * a1 + *reinterpret_cast<const f32x4*>(src + dt * 16) * a2;
        l_run[0] = l_run[0] * a1 + l2 * a2;
        off_[0] = om == -INFINITY ? 0.f : om;
        m_ref[0] = om;  // only its -inf-ness is used below
      }
      active = active && hmask == 1;
    }

    if (whole) {
      if (active) {
#pragma unroll
        for (int w2 = 0; w2 < 2; ++w2) {
          if (w2 == 1 && !two) continue;
          const int row = w2 == 0 ? rowA : rowB;
          if (row < rows_here) {
            const float inv = l_run[w2] > 0.f ? 1.f / l_run[w2] : 0.f;
            uint16_t* dst =
                static_cast<uint16_t*>(p.out) + qo_offset(p, nbeg, g, row0 + row, D) + lg * 4;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
              uint2 pk;
              pk.x = pack_bf16x2(acc[dt][w2][0] * inv, acc[dt][w2][1] * inv);
              pk.y = pack_bf16x2(acc[dt][w2][2] * inv, acc[dt][w2][3] * inv);
              *reinterpret_cast<uint2*>(dst + dt * 16) = pk;
            }
          }
        }
      }
      continue;
    }

    // Cut pair: publish (offset, l, acc) of this share's part of it; the
    // offset is in log2 units (-inf when no key was visible).
    const size_t slot = cut_slot(T, lw, p.lg_nwg, ps);
    if (active) {
#pragma unroll
      for (int w2 = 0; w2 < 2; ++w2) {
        if (w2 == 1 && !two) continue;
        const int row = w2 == 0 ? rowA : rowB;
        if (row < rows_here) {
          const size_t base = slot * kRowsPB + row;
          float* dst = p.part_o + base * D + lg * 4;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
            *reinterpret_cast<f32x4*>(dst + dt * 16) = acc[dt][w2];
          if (lg == 0) {
            p.part_ml[base * 2] = m_ref[w2] == -INFINITY ? -INFINITY : off_[w2];
            p.part_ml[base * 2 + 1] = l_run[w2];
          }
        }
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
    if (tiles > 0x7fffffffLL) return false;
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
    pl.dyn_lds = size_t(d.batch + 1 + d.max_nodes) * sizeof(int) +
                 size_t(nn_max) * pl.words * sizeof(uint32_t);
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
    const size_t merge_lds = size_t(d.batch + 1) * sizeof(int);
    if (d.head_dim == 128) {
      hipLaunchKernelGGL(attn_stream_kernel<128>, grid, block, lds, stream, p);
      hipLaunchKernelGGL(attn_merge_kernel<128>, grid, block, merge_lds, stream, p);
    } else {
      hipLaunchKernelGGL(attn_stream_kernel<64>, grid, block, lds, stream, p);
      hipLaunchKernelGGL(attn_merge_kernel<64>, grid, block, merge_lds, stream, p);
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
