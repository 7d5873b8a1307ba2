// Tree-masked attention over a paged prefix KV cache (one layer).
//
// What it computes follows SpecInfer's tree-based parallel decoding as the
// survey page's Timeline section describes it (tree tokens stored in the KV
// cache in topological order, each token attending to its ancestors only) and
// TreeSpark §3.2 step 3 / §4 (one target pass, per-step ancestor bitmask).
//
// Design (gfx950):
//  * Work item = (request r, kv head g, row block, key split). Rows are
//    (tree node x grouped q head), so one K/V tile staged in LDS serves every
//    node of the tree and all G = Hq/Hkv heads that share the kv head.
//  * bf16 path: 4 waves x 32 rows. S^T = K Q^T and O^T += V^T P^T with
//    v_mfma_f32_16x16x32_bf16; both outputs keep rows on lane%16 so the
//    online-softmax rescale is lane-local. P never leaves registers: the
//    PV key order is permuted to match the S^T output layout, and V is
//    transposed (with the same permutation) while it is written to LDS.
//  * The ancestor mask is a per-node bitset built in LDS in the prologue
//    and consulted only in tiles that reach the tree's own keys.
//  * Key splits write fp32 partials (m, l, unnormalised acc); the last split
//    to finish (device-scope counter) merges them in fixed split order, so
//    results are deterministic and one launch does the whole layer.
//  * fp32 path (small validation shapes): a VALU kernel with the same work
//    decomposition, partial format and merge.
#include "tv_device.hpp"
#include "tv_internal.hpp"

namespace tv {

namespace {

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
  int rb_max, c_max, chunk_len, grid_real;
  float scale_log2;
};

constexpr float kLog2e = 1.4426950408889634f;

// Common per-workgroup bookkeeping.
struct Item {
  int r, g, rb, c;
  int nbeg, N, P, L, R, row0, rows_here, nch, kbeg, kend, pbase;
  int first_node, nn;
  size_t slot, pair;
};

// blockIdx -> slot: XCD x (blocks x, x+8, ...) walks the contiguous slot range
// [x*S/8, (x+1)*S/8), so row blocks that share a K/V chunk run on one XCD
// and share its L2.
__device__ inline int remap_block(int b, int grid) {
  const int per = grid >> 3;
  return (b & 7) * per + (b >> 3);
}

template <int ROWS_PB>
__device__ inline bool decode_item(const AttnParams& p, Item& it) {
  const int s = remap_block(blockIdx.x, gridDim.x);
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
  if (it.N > p.max_nodes || it.P < 0 || it.P + it.N > p.max_kv_len) {
    if (threadIdx.x == 0 && it.rb == 0 && it.c == 0) raise_status(p.status, TV_DEV_SHAPE);
    return false;
  }
  it.L = it.P + it.N;
  it.R = it.N * p.G;
  it.row0 = it.rb * ROWS_PB;
  if (it.row0 >= it.R) return false;
  it.rows_here = min(ROWS_PB, it.R - it.row0);
  it.nch = (it.L + p.chunk_len - 1) / p.chunk_len;
  if (it.c >= it.nch) return false;
  it.kbeg = it.c * p.chunk_len;
  it.kend = min(it.L, it.kbeg + p.chunk_len);
  it.pbase = p.page_indptr[it.r];
  const int npg = p.page_indptr[it.r + 1] - it.pbase;
  if (npg * kPage < it.L) {
    if (threadIdx.x == 0 && it.c == 0 && it.rb == 0) raise_status(p.status, TV_DEV_PAGES);
    return false;
  }
  it.first_node = it.row0 / p.G;
  it.nn = (it.row0 + it.rows_here - 1) / p.G - it.first_node + 1;
  return true;
}

// Ancestor-or-self bitsets of the block's nodes in LDS (nn rows of `words`).
__device__ inline void build_anc(const AttnParams& p, const Item& it, uint32_t* anc) {
  for (int i = threadIdx.x; i < it.nn * p.words; i += blockDim.x) anc[i] = 0u;
  __syncthreads();
  for (int t = threadIdx.x; t < it.nn; t += blockDim.x) {
    uint32_t* row = anc + t * p.words;
    int j = it.first_node + t;
    while (true) {
      row[j >> 5] |= 1u << (j & 31);
      const int pj = p.parent[it.nbeg + j];
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
  __syncthreads();
}

__device__ inline int physical_page(const AttnParams& p, const Item& it, int key) {
  int phys = p.page_indices[it.pbase + (key >> 4)];
  if (unsigned(phys) >= unsigned(p.num_pages)) {
    raise_status(p.status, TV_DEV_PAGES);
    phys = 0;
  }
  return phys;
}

// Row i's element address in q / out.
__device__ inline size_t qo_offset(const AttnParams& p, const Item& it, int row, int D) {
  const int node = row / p.G;
  const int gh = row - node * p.G;
  return (size_t(it.nbeg + node) * p.Hq + size_t(it.g) * p.G + gh) * D;
}

__device__ inline size_t chunk_slot(const AttnParams& p, const Item& it, int c) {
  return ((size_t(it.r) * p.Hkv + it.g) * p.c_max + c) * p.rb_max + it.rb;
}

// Publish this split's partial and report whether this workgroup is the last
// split of its (request, kv head, row block) to finish.
__device__ inline bool arrive_last(const AttnParams& p, const Item& it, int* s_last) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = atomicAdd(&p.counters[it.pair], 1u);
    *s_last = (old == uint32_t(it.nch - 1)) ? 1 : 0;
  }
  __syncthreads();
  const bool last = *s_last != 0;
  if (last) __threadfence();
  return last;
}

// Merge the nch partials of the block in split order and write the output.
template <int ROWS_PB, int D, bool BF16_OUT>
__device__ inline void merge_and_store(const AttnParams& p, const Item& it, float* s_M,
                                       float* s_invL) {
  for (int row = threadIdx.x; row < it.rows_here; row += blockDim.x) {
    float M = -INFINITY;
    for (int c = 0; c < it.nch; ++c) {
      const float* ml = p.part_ml + (chunk_slot(p, it, c) * ROWS_PB + row) * 2;
      M = fmaxf(M, ml[0]);
    }
    float L = 0.f;
    if (M != -INFINITY) {
      for (int c = 0; c < it.nch; ++c) {
        const float* ml = p.part_ml + (chunk_slot(p, it, c) * ROWS_PB + row) * 2;
        L += ml[1] * exp2f(ml[0] - M);
      }
    }
    s_M[row] = M;
    s_invL[row] = (L > 0.f) ? 1.f / L : 0.f;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < it.rows_here * (D / 4); idx += blockDim.x) {
    const int row = idx / (D / 4);
    const int d4 = (idx - row * (D / 4)) * 4;
    const float M = s_M[row];
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    if (M != -INFINITY) {
      for (int c = 0; c < it.nch; ++c) {
        const size_t base = chunk_slot(p, it, c) * ROWS_PB + row;
        const float w = exp2f(p.part_ml[base * 2] - M);
        const float4 a = *reinterpret_cast<const float4*>(p.part_o + base * D + d4);
        o.x += w * a.x;
        o.y += w * a.y;
        o.z += w * a.z;
        o.w += w * a.w;
      }
    }
    const float inv = s_invL[row];
    const size_t off = qo_offset(p, it, it.row0 + row, D) + d4;
    if (BF16_OUT) {
      uint2 pk;
      pk.x = pack_bf16x2(o.x * inv, o.y * inv);
      pk.y = pack_bf16x2(o.z * inv, o.w * inv);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + off) = pk;
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(p.out) + off) =
          make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
    }
  }
}

// Column of key k (0..31 within a tile) in the transposed V tile: keys
// {4j..4j+3, 16+4j..16+4j+3} are stored contiguously at 8j, matching the key
// order the S^T accumulator hands to the PV product.
__device__ inline int vt_col(int k) {
  return (k < 16) ? (8 * (k >> 2) + (k & 3)) : (8 * ((k - 16) >> 2) + 4 + (k & 3));
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel: 256 threads = 4 waves x 32 rows = 128 rows per block.
template <int D>
__global__ __launch_bounds__(256) void attn_mfma_kernel(AttnParams p) {
  constexpr int ROWS_PB = 128;
  constexpr int KK = D / 32;          // 32-wide k-steps of the QK product
  constexpr int DT = D / 16;          // 16-wide d tiles of the PV product
  constexpr int KSTR = D + 8;         // LDS row stride of K (bf16 elements)
  constexpr int VSTR = 32 + 8;        // LDS row stride of V^T (bf16 elements)
  constexpr int DB = D / 8;           // 16-byte blocks per K/V row
  constexpr int KJOBS = 32 * DB / 256;  // K 16-byte loads per thread per tile
  constexpr int VJOBS = 16 * DB;        // V key-pair jobs per tile (<= 256)

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][32 * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[2][D * VSTR];
  __shared__ float s_M[ROWS_PB];
  __shared__ float s_invL[ROWS_PB];
  __shared__ int s_last;
  extern __shared__ uint32_t anc_lds[];

  Item it;
  if (!decode_item<ROWS_PB>(p, it)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int lg = lane >> 4;

  const bool tree_in_chunk = it.kend > it.P;
  if (tree_in_chunk) build_anc(p, it, anc_lds);

  const uint16_t* qb = static_cast<const uint16_t*>(p.q);
  const uint16_t* kp = static_cast<const uint16_t*>(p.k_pages);
  const uint16_t* vp = static_cast<const uint16_t*>(p.v_pages);

  // Q^T operands for this wave's 32 rows (2 row tiles of 16).
  const int wrow0 = it.row0 + wave * 32;
  const bool wave_active = wave * 32 < it.rows_here;
  bf16x8 qf[2][KK];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int row = wrow0 + rt * 16 + l16;
    if (wave_active && row < it.R) {
      const uint16_t* src = qb + qo_offset(p, it, row, D) + lg * 8;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        qf[rt][kk] = *reinterpret_cast<const bf16x8*>(src + kk * 32);
    } else {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        qf[rt][kk] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }

  const size_t head_stride = size_t(kPage) * D;                    // one (page, head) block
  const size_t page_stride = size_t(p.Hkv) * head_stride;

  uint4 kreg[KJOBS];
  uint4 vreg[2];
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int j = 0; j < KJOBS; ++j) {
      const int job = tid + 256 * j;
      const int kl = job / DB;
      const int db = job - kl * DB;
      const int key = t0 + kl;
      if (key < it.kend) {
        const int phys = physical_page(p, it, key);
        const uint16_t* src = kp + size_t(phys) * page_stride + size_t(it.g) * head_stride +
                              size_t(key & 15) * D + db * 8;
        kreg[j] = *reinterpret_cast<const uint4*>(src);
      } else {
        kreg[j] = make_uint4(0, 0, 0, 0);
      }
    }
    if (tid < VJOBS) {
      const int pr = tid / DB;
      const int db = tid - pr * DB;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int key = t0 + 2 * pr + h;
        if (key < it.kend) {
          const int phys = physical_page(p, it, key);
          const uint16_t* src = vp + size_t(phys) * page_stride + size_t(it.g) * head_stride +
                                size_t(key & 15) * D + db * 8;
          vreg[h] = *reinterpret_cast<const uint4*>(src);
        } else {
          vreg[h] = make_uint4(0, 0, 0, 0);
        }
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int j = 0; j < KJOBS; ++j) {
      const int job = tid + 256 * j;
      const int kl = job / DB;
      const int db = job - kl * DB;
      *reinterpret_cast<uint4*>(&k_lds[buf][kl * KSTR + db * 8]) = kreg[j];
    }
    if (tid < VJOBS) {
      const int pr = tid / DB;
      const int db = tid - pr * DB;
      const int col = vt_col(2 * pr);
      const uint32_t* a = reinterpret_cast<const uint32_t*>(&vreg[0]);
      const uint32_t* b = reinterpret_cast<const uint32_t*>(&vreg[1]);
      uint32_t* dst = reinterpret_cast<uint32_t*>(&vt_lds[buf][(db * 8) * VSTR + col]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t lo = (a[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
        const uint32_t hi = (b[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
        dst[e * (VSTR / 2)] = lo | (hi << 16);
      }
    }
  };

  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};
  f32x4 acc[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    acc[dt][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc[dt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  load_tile(it.kbeg);
  store_tile(0);
  __syncthreads();
  int buf = 0;
  for (int t0 = it.kbeg; t0 < it.kend; t0 += 32) {
    const bool has_next = t0 + 32 < it.kend;
    if (has_next) load_tile(t0 + 32);

    if (wave_active) {
      f32x4 s[2][2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        s[kt][0] = f32x4{0.f, 0.f, 0.f, 0.f};
        s[kt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        const uint16_t* krow = &k_lds[buf][(kt * 16 + l16) * KSTR + lg * 8];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + kk * 32);
          s[kt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[0][kk], s[kt][0], 0, 0, 0);
          s[kt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[1][kk], s[kt][1], 0, 0, 0);
        }
      }
      const bool need_mask = (t0 + 32 > it.P) || (t0 + 32 > it.kend);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const int row = wrow0 + rt * 16 + l16;
        const int nl = row / p.G - it.first_node;
        float mt = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float v = s[kt][rt][e] * p.scale_log2;
            if (need_mask) {
              const int key = t0 + kt * 16 + lg * 4 + e;
              bool vis = key < it.kend && row < it.R;
              if (vis && key >= it.P) {
                const int j = key - it.P;
                vis = (anc_lds[nl * p.words + (j >> 5)] >> (j & 31)) & 1u;
              }
              v = vis ? v : -INFINITY;
            }
            s[kt][rt][e] = v;
            mt = fmaxf(mt, v);
          }
        }
        mt = fmaxf(mt, shfl_xor(mt, 16));
        mt = fmaxf(mt, shfl_xor(mt, 32));
        const float m_new = fmaxf(m_run[rt], mt);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2f(m_run[rt] - m_use);
        m_run[rt] = m_new;
        float ls = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float pv = exp2f(s[kt][rt][e] - m_use);
            s[kt][rt][e] = pv;
            ls += pv;
          }
        }
        l_run[rt] = l_run[rt] * alpha + ls;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[dt][rt] *= alpha;
      }
      bf16x8 pb[2];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pb[rt][e] = static_cast<__bf16>(s[0][rt][e]);
          pb[rt][4 + e] = static_cast<__bf16>(s[1][rt][e]);
        }
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(&vt_lds[buf][(dt * 16 + l16) * VSTR + lg * 8]);
        acc[dt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[0], acc[dt][0], 0, 0, 0);
        acc[dt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[1], acc[dt][1], 0, 0, 0);
      }
    }

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  // Row sums: the four lane groups of a row hold disjoint key subsets.
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    float l = l_run[rt];
    l += shfl_xor(l, 16);
    l += shfl_xor(l, 32);
    l_run[rt] = l;
  }

  if (it.nch == 1) {
    if (wave_active) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const int row = wrow0 + rt * 16 + l16;
        if (row < it.R && row < it.row0 + ROWS_PB) {
          const float inv = l_run[rt] > 0.f ? 1.f / l_run[rt] : 0.f;
          uint16_t* dst = static_cast<uint16_t*>(p.out) + qo_offset(p, it, row, D) + lg * 4;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            uint2 pk;
            pk.x = pack_bf16x2(acc[dt][rt][0] * inv, acc[dt][rt][1] * inv);
            pk.y = pack_bf16x2(acc[dt][rt][2] * inv, acc[dt][rt][3] * inv);
            *reinterpret_cast<uint2*>(dst + dt * 16) = pk;
          }
        }
      }
    }
    return;
  }

  // Split: publish (m, l, acc) for this chunk.
  if (wave_active) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int prow = wave * 32 + rt * 16 + l16;
      if (prow < it.rows_here) {
        const size_t base = it.slot * ROWS_PB + prow;
        float* dst = p.part_o + base * D + lg * 4;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          *reinterpret_cast<float4*>(dst + dt * 16) =
              make_float4(acc[dt][rt][0], acc[dt][rt][1], acc[dt][rt][2], acc[dt][rt][3]);
        if (lg == 0) {
          p.part_ml[base * 2] = m_run[rt];
          p.part_ml[base * 2 + 1] = l_run[rt];
        }
      }
    }
  }
  if (!arrive_last(p, it, &s_last)) return;
  merge_and_store<ROWS_PB, D, true>(p, it, s_M, s_invL);
  if (threadIdx.x == 0) p.counters[it.pair] = 0u;
}

// ---------------------------------------------------------------------------
// fp32 VALU kernel: 256 threads, 32 rows per block, 32-key tiles.
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
  extern __shared__ uint32_t anc_lds[];

  Item it;
  if (!decode_item<ROWS_PB>(p, it)) return;
  const int tid = threadIdx.x;
  if (it.kend > it.P) build_anc(p, it, anc_lds);

  const float* qf = static_cast<const float*>(p.q);
  const float* kp = static_cast<const float*>(p.k_pages);
  const float* vp = static_cast<const float*>(p.v_pages);
  for (int idx = tid; idx < ROWS_PB * D; idx += 256) {
    const int row = idx / D, d = idx - (idx / D) * D;
    q_lds[row][d] = (row < it.rows_here) ? qf[qo_offset(p, it, it.row0 + row, D) + d] : 0.f;
  }
  if (tid < ROWS_PB) {
    s_m[tid] = -INFINITY;
    s_l[tid] = 0.f;
  }
  float o[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) o[i] = 0.f;

  const size_t head_stride = size_t(kPage) * D;
  const size_t page_stride = size_t(p.Hkv) * head_stride;
  for (int t0 = it.kbeg; t0 < it.kend; t0 += TK) {
    __syncthreads();
    for (int idx = tid; idx < TK * D; idx += 256) {
      const int kl = idx / D, d = idx - (idx / D) * D;
      const int key = t0 + kl;
      float kv = 0.f, vv = 0.f;
      if (key < it.kend) {
        const int phys = physical_page(p, it, key);
        const size_t off = size_t(phys) * page_stride + size_t(it.g) * head_stride +
                           size_t(key & 15) * D + d;
        kv = kp[off];
        vv = vp[off];
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
          vis = (anc_lds[nl * p.words + (j >> 5)] >> (j & 31)) & 1u;
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
        static_cast<float*>(p.out)[qo_offset(p, it, it.row0 + row, D) + d] =
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
  if (!arrive_last(p, it, &s_last)) return;
  merge_and_store<ROWS_PB, D, false>(p, it, s_M, s_invL);
  if (threadIdx.x == 0) p.counters[it.pair] = 0u;
}

}  // namespace

// Keys per split: enough splits to give ~1024 work items at max_kv_len, but
// no split shorter than 128 keys (each split costs a rows x D fp32 partial).
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
  pl.rows_pb = pl.mfma ? 128 : 32;
  const long rows = long(d.max_nodes) * pl.group;
  pl.rb_max = int((rows + pl.rows_pb - 1) / pl.rows_pb);
  const long pairs = long(d.batch) * d.num_kv_heads * pl.rb_max;
  const long target_items = 1024;
  long chunk = (long(d.max_kv_len) * pairs + target_items - 1) / target_items;
  chunk = chunk < 128 ? 128 : chunk;
  chunk = (chunk + 31) / 32 * 32;
  const long full = (long(d.max_kv_len) + 31) / 32 * 32;
  if (chunk > full) chunk = full;
  pl.chunk_len = int(chunk);
  pl.c_max = int((d.max_kv_len + chunk - 1) / chunk);
  pl.words = (d.max_nodes + 31) / 32;
  pl.slots = size_t(pairs) * pl.c_max;
  pl.grid = (pl.slots + 7) / 8 * 8;
  if (pl.grid > 0x7fffffffULL) return false;
  size_t off = kHeaderBytes;
  pl.off_counters = off;
  off = align256(off + size_t(pairs) * sizeof(uint32_t));
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
  const float scale = d.sm_scale > 0.f ? d.sm_scale : 1.f / sqrtf(float(d.head_dim));
  p.scale_log2 = scale * kLog2e;
  const int nn_max = pl.rows_pb / pl.group + 2;
  const size_t anc_bytes = size_t(nn_max) * pl.words * sizeof(uint32_t);
  const dim3 grid(unsigned(pl.grid)), block(256);
  if (pl.mfma) {
    if (d.head_dim == 128)
      hipLaunchKernelGGL(attn_mfma_kernel<128>, grid, block, anc_bytes, stream, p);
    else
      hipLaunchKernelGGL(attn_mfma_kernel<64>, grid, block, anc_bytes, stream, p);
  } else {
    if (d.head_dim == 128)
      hipLaunchKernelGGL(attn_valu_kernel<128>, grid, block, anc_bytes, stream, p);
    else
      hipLaunchKernelGGL(attn_valu_kernel<64>, grid, block, anc_bytes, stream, p);
  }
  return hipGetLastError();
}

}  // namespace tv
