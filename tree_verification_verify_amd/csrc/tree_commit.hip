// Commit of the accepted path's K/V: in-place compaction by a gather.
//
// The survey page's Systems section (KV handling) describes the reference
// EAGLE implementation compacting the accepted slots in place with gathers
// over the accepted positions; SpecInfer (survey, Timeline) keeps tree tokens
// in the KV cache in topological order, so node i of request r sits at logical
// position P_r + i and a root path visits increasing node indices. For request
// r with n = out_len[r] path nodes, in every layer and kv head, logical
// position P_r + j takes the K/V of logical position kv_keep[r][j]
// (j = 0 .. n-1). A path node's index is at least its depth, so no
// destination P_r + j is the source of a later entry; within a chunk every
// source is read before any destination is written.
//
// One workgroup per (request, layer). K rows ([page][head][slot][D]) move as
// 16-byte pieces; V is transposed within each page ([page][head][D][slot]), so
// a token's V is one element per channel: the writes run with the entry index
// fastest, so a channel's run of consecutive destination slots is one
// contiguous store. Every store is non-temporal: a moved V column dirties one
// line in each of 32 rows of its page block, and stores kept in L2 left that
// many dirty lines for the end of the kernel to write back.
#include "tv_device.hpp"
#include "tv_internal.hpp"

namespace tv {

namespace {

constexpr int kCommitThreads = 256;
constexpr int kPairs = 32;  // (moved entry, kv head) pairs per chunk

struct CommitParams {
  void* k;
  void* v;
  long long layer_stride;  // elements
  const int32_t* page_indptr;
  const int32_t* page_indices;
  const int32_t* prefix_len;
  const int32_t* kv_keep;
  const int32_t* out_len;
  uint32_t* status;
  int B, L, Hkv, num_pages, W, max_nodes;
};

// One workgroup per (request, layer). The keep-list is checked (and its
// page ids looked up) in blocks of 256 entries, one per thread; the entries
// that move (kv_keep[j] != P + j) are compacted into an LDS list, and their
// (entry, kv head) pairs are moved kPairs at a time, heads outer and entries
// fastest, all loads of a chunk in flight together.
template <int D, typename T>
__global__ __launch_bounds__(kCommitThreads) void kv_commit_kernel(CommitParams p) {
  constexpr int KP = D * int(sizeof(T)) / 16;  // 16-byte pieces per K row
  constexpr int KI = (kPairs * KP + kCommitThreads - 1) / kCommitThreads;  // K items per thread
  constexpr int VI = (kPairs * D + kCommitThreads - 1) / kCommitThreads;   // V items per thread
  __shared__ int s_src[kCommitThreads], s_spg[kCommitThreads], s_dpg[kCommitThreads];
  __shared__ int s_dsl[kCommitThreads];  // destination slot within its page
  __shared__ int s_wcount[kCommitThreads / 64];
  __shared__ int s_bad;

  const int layer = blockIdx.x % p.L;
  const int r = blockIdx.x / p.L;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  // The request's scalars and this thread's keep-list entry load together
  // (every entry j < W of the row is in the array), one round trip.
  const int32_t* keep = p.kv_keep + size_t(r) * p.W;
  const int n = p.out_len[r];
  const int P = p.prefix_len[r];
  const int pbase = p.page_indptr[r];
  const int npg = p.page_indptr[r + 1] - pbase;
  const int keep_t = tid < p.W ? keep[tid] : 0;
  const int keep_prev = tid >= 1 && tid - 1 < p.W ? keep[tid - 1] : 0;
  if (n < 1) return;  // nothing accepted (or a path error reported upstream)
  const bool reporter = layer == 0 && tid == 0;
  if (n > p.W) {
    if (reporter) raise_status(p.status, TV_DEV_SHAPE);
    return;
  }

  // Entry j is valid when the list starts at P, increases strictly, stays
  // in [P + j, P + max_nodes) and its source and destination lie in listed
  // pages with ids inside the pool. The whole list is checked before
  // anything moves, so every workgroup of the request takes the same
  // decision: lists longer than one block get a checking pass of their own;
  // a shorter list is checked while its moving entries are gathered.
  auto check = [&](int j, int s, int prev, int& ps, int& pd) -> int {
    bool ok = P >= 0 && s >= P + j && s < P + p.max_nodes && (j == 0 ? s == P : s > prev);
    ok = ok && s / kPage < npg && (P + j) / kPage < npg;
    if (!ok) return 1;
    ps = p.page_indices[pbase + s / kPage];
    pd = p.page_indices[pbase + (P + j) / kPage];
    return (unsigned(ps) >= unsigned(p.num_pages) || unsigned(pd) >= unsigned(p.num_pages)) ? 2 : 0;
  };
  if (tid == 0) s_bad = 0;
  __syncthreads();
  if (n > kCommitThreads) {
    for (int j = tid; j < n; j += kCommitThreads) {
      int ps, pd;
      const int bad = check(j, keep[j], j > 0 ? keep[j - 1] : 0, ps, pd);
      if (bad) atomicOr(&s_bad, bad);
    }
    __syncthreads();
    if (s_bad) {
      if (reporter) raise_status(p.status, (s_bad & 2) ? TV_DEV_PAGES : TV_DEV_PATH);
      return;
    }
  }

  T* kb = static_cast<T*>(p.k) + size_t(layer) * size_t(p.layer_stride);
  T* vb = static_cast<T*>(p.v) + size_t(layer) * size_t(p.layer_stride);
  const size_t head_block = size_t(kPage) * D;  // elements per (page, head)

  for (int j0 = 0; j0 < n; j0 += kCommitThreads) {
    // Gather (and, for a one-block list, check) the entries of this block
    // that move; entries already in place stay.
    const int j = j0 + tid;
    int s = 0, spg = 0, dpg = 0;
    bool mv = false;
    if (j < n) {
      s = j0 == 0 ? keep_t : keep[j];
      const int bad = check(j, s, j0 == 0 ? keep_prev : keep[j - 1], spg, dpg);
      if (bad) atomicOr(&s_bad, bad);
      mv = !bad && s != P + j;
    }
    const uint64_t mask = __builtin_amdgcn_ballot_w64(mv);
    if (lane == 0) s_wcount[wave] = __builtin_popcountll(mask);
    __syncthreads();
    if (s_bad) {  // only a one-block list can get here with an error
      if (reporter) raise_status(p.status, (s_bad & 2) ? TV_DEV_PAGES : TV_DEV_PATH);
      return;
    }
    int before = 0, m = 0;
    for (int w = 0; w < kCommitThreads / 64; ++w) {
      before += w < wave ? s_wcount[w] : 0;
      m += s_wcount[w];
    }
    if (mv) {
      const int at = before + __builtin_popcountll(mask & ((uint64_t(1) << lane) - 1));
      s_src[at] = s;
      s_spg[at] = spg;
      s_dpg[at] = dpg;
      s_dsl[at] = (P + j) % kPage;
    }
    __syncthreads();
    // Pairs (moved entry e, head h) as q = h * m + e, kPairs at a time. Each
    // thread loads all its items of a chunk into registers (every load in
    // flight together), the barrier orders every read before any write,
    // then the thread stores the same items at their destinations.
    const int npairs = m * p.Hkv;
    for (int q0 = 0; q0 < npairs; q0 += kPairs) {
      const int c = min(kPairs, npairs - q0);
      uint4 kr[KI];
      T vr[VI];
#pragma unroll
      for (int k = 0; k < KI; ++k) {
        const int i = tid + k * kCommitThreads;
        if (i < c * KP) {
          const int q = q0 + i / KP, piece = i % KP;
          const int h = q / m, e = q - h * m;
          const T* row = kb + (size_t(s_spg[e]) * p.Hkv + h) * head_block + size_t(s_src[e] % kPage) * D;
          kr[k] = reinterpret_cast<const uint4*>(row)[piece];
        }
      }
#pragma unroll
      for (int k = 0; k < VI; ++k) {
        const int i = tid + k * kCommitThreads;
        if (i < c * D) {
          const int ch = i / c, qq = i - ch * c;  // pair fastest: consecutive destination slots
          const int q = q0 + qq;
          const int h = q / m, e = q - h * m;
          vr[k] = vb[(size_t(s_spg[e]) * p.Hkv + h) * head_block + size_t(ch) * kPage + s_src[e] % kPage];
        }
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < KI; ++k) {
        const int i = tid + k * kCommitThreads;
        if (i < c * KP) {
          const int q = q0 + i / KP, piece = i % KP;
          const int h = q / m, e = q - h * m;
          T* row = kb + (size_t(s_dpg[e]) * p.Hkv + h) * head_block + size_t(s_dsl[e]) * D;
          typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
          __builtin_nontemporal_store(__builtin_bit_cast(u32x4, kr[k]), reinterpret_cast<u32x4*>(row) + piece);
        }
      }
#pragma unroll
      for (int k = 0; k < VI; ++k) {
        const int i = tid + k * kCommitThreads;
        if (i < c * D) {
          const int ch = i / c, qq = i - ch * c;
          const int q = q0 + qq;
          const int h = q / m, e = q - h * m;
          __builtin_nontemporal_store(vr[k], vb + (size_t(s_dpg[e]) * p.Hkv + h) * head_block + size_t(ch) * kPage + s_dsl[e]);
        }
      }
      __syncthreads();  // every store of this chunk precedes the next chunk's reads
    }
  }
}

}  // namespace

hipError_t launch_kv_commit(const tv_attn_desc& d, int32_t num_layers, long long layer_stride,
                            void* k_pages, void* v_pages, const int32_t* page_indptr,
                            const int32_t* page_indices, const int32_t* prefix_len,
                            const int32_t* kv_keep, const int32_t* out_len, int32_t max_depth,
                            uint32_t* status, hipStream_t stream) {
  CommitParams p{};
  p.k = k_pages;
  p.v = v_pages;
  p.layer_stride = layer_stride;
  p.page_indptr = page_indptr;
  p.page_indices = page_indices;
  p.prefix_len = prefix_len;
  p.kv_keep = kv_keep;
  p.out_len = out_len;
  p.status = status;
  p.B = d.batch;
  p.L = num_layers;
  p.Hkv = d.num_kv_heads;
  p.num_pages = d.num_pages;
  p.W = max_depth + 1;
  p.max_nodes = d.max_nodes;
  const dim3 grid(unsigned((long long)d.batch * num_layers)), block(kCommitThreads);
  if (d.dtype == TV_BF16) {
    if (d.head_dim == 128)
      hipLaunchKernelGGL((kv_commit_kernel<128, uint16_t>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((kv_commit_kernel<64, uint16_t>), grid, block, 0, stream, p);
  } else {
    if (d.head_dim == 128)
      hipLaunchKernelGGL((kv_commit_kernel<128, uint32_t>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((kv_commit_kernel<64, uint32_t>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace tv
