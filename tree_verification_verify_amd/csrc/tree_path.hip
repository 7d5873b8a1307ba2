// Longest accepted path, tree metadata and the workspace fill kernel.
//
// Path: TreeSpark §3.2 step 3 (commit the longest surviving root path plus
// one correction/bonus token), §5.1 (tau = accepted drafts + 1) and the
// explainer's "exactly one path is accepted"; the keep-list of logical KV
// positions is what the survey page's Systems section calls EAGLE's
// retrieve_indices compaction input.
// Metadata: per-depth positions and ancestor bitmasks (TreeSpark §3.2 step 3,
// §4).
#include "tv_device.hpp"
#include "tv_internal.hpp"

namespace tv {

namespace {

// Rows of a request staged in LDS for the walk (larger requests read them
// from memory at every level).
constexpr int kPathStage = 1024;

// One wave per request: from the root, find the unique flagged child with a
// ballot over the request's rows, descend, repeat. A request of at most
// kPathStage rows has its parents, flags, tokens and next tokens staged in
// LDS first (one load round trip for the request instead of one per level
// and one for the emitted tokens) and its path kept there, so the outputs
// are written by all lanes after the walk.
__global__ __launch_bounds__(64) void accept_path_kernel(
    int32_t batch, int32_t width, const int32_t* node_indptr, const int32_t* parent,
    const int32_t* tokens, const int8_t* flag, const int32_t* next_token,
    const int32_t* prefix_len, int32_t* path_nodes, int32_t* out_tokens, int32_t* out_len,
    int32_t* kv_keep, uint32_t* status) {
  __shared__ int s_par[kPathStage];
  __shared__ int8_t s_flag[kPathStage];
  __shared__ int s_path[kPathStage];
  __shared__ int s_tok[kPathStage], s_nt[kPathStage];
  const int r = blockIdx.x;
  const int lane = threadIdx.x;
  const int nbeg = node_indptr[r];
  const int N = node_indptr[r + 1] - nbeg;
  const int P = prefix_len[r];
  int32_t* pn = path_nodes + size_t(r) * width;
  int32_t* ot = out_tokens + size_t(r) * width;
  int32_t* kk = kv_keep + size_t(r) * width;
  const bool staged = N <= kPathStage;
  if (staged) {
    for (int i = lane; i < N; i += 64) {
      s_par[i] = parent[nbeg + i];
      s_flag[i] = flag[nbeg + i];
      s_tok[i] = tokens[nbeg + i];
      s_nt[i] = next_token[nbeg + i];
    }
  }
  for (int i = lane; i < width; i += 64) {
    pn[i] = -1;
    ot[i] = -1;
    kk[i] = -1;
  }
  if (N <= 0) {
    if (lane == 0) out_len[r] = 0;
    return;
  }
  __syncthreads();  // the staged rows are visible to every lane
  int v = 0;
  int len = 1;
  bool error = false;
  if (lane == 0) {
    if (staged) {
      s_path[0] = 0;
    } else {
      pn[0] = 0;
      kk[0] = P;
    }
  }
  while (true) {
    int found = -1;
    int nfound = 0;
    for (int base = v + 1; base < N; base += 64) {
      const int i = base + lane;
      bool hit = false;
      if (i < N) hit = staged ? (s_par[i] == v && s_flag[i] == 1) : (parent[nbeg + i] == v && flag[nbeg + i] == 1);
      const unsigned long long m = __ballot(hit);
      if (m) {
        if (found < 0) found = base + __ffsll(static_cast<long long>(m)) - 1;
        nfound += __popcll(m);
      }
    }
    if (nfound > 1) {
      error = true;
      break;
    }
    if (found < 0) break;
    if (len >= width) {  // deeper than max_depth
      error = true;
      break;
    }
    if (lane == 0) {
      if (staged) {
        s_path[len] = found;
      } else {
        pn[len] = found;
        ot[len - 1] = tokens[nbeg + found];
        kk[len] = P + found;
      }
    }
    v = found;
    ++len;
  }
  if (staged && !error) {
    __syncthreads();  // lane 0's path entries are visible
    for (int i = lane; i < len; i += 64) {
      const int node = s_path[i];
      pn[i] = node;
      kk[i] = P + node;
      ot[i] = i + 1 < len ? s_tok[s_path[i + 1]] : s_nt[v];
    }
  }
  if (lane == 0) {
    if (error) {
      out_len[r] = -1;
      raise_status(status, TV_DEV_PATH);
    } else {
      if (!staged) ot[len - 1] = next_token[nbeg + v];
      out_len[r] = len;
    }
  }
}

// One thread per row: depth and ancestor bitset by walking to the root;
// first child / next sibling by scanning later rows (parent[i] < i).
__global__ __launch_bounds__(256) void tree_meta_kernel(
    int32_t batch, int32_t words, const int32_t* node_indptr, const int32_t* parent,
    int32_t* depth, uint32_t* anc_bits, int32_t* first_child, int32_t* next_sibling,
    uint32_t* status) {
  const int r = blockIdx.y;
  const int nbeg = node_indptr[r];
  const int N = node_indptr[r + 1] - nbeg;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N) return;
  if (N > words * 32) {
    if (i == 0) raise_status(status, TV_DEV_SHAPE);
    return;
  }
  uint32_t* bits = anc_bits ? anc_bits + size_t(nbeg + i) * words : nullptr;
  if (bits)
    for (int w = 0; w < words; ++w) bits[w] = 0u;
  int j = i;
  int dep = 0;
  while (true) {
    if (bits) bits[j >> 5] |= 1u << (j & 31);
    const int pj = parent[nbeg + j];
    if (j == 0) {
      if (pj != -1) raise_status(status, TV_DEV_TREE);
      break;
    }
    if (pj < 0 || pj >= j) {
      raise_status(status, TV_DEV_TREE);
      break;
    }
    j = pj;
    ++dep;
  }
  if (depth) depth[nbeg + i] = dep;
  if (first_child || next_sibling) {
    const int pi = i > 0 ? parent[nbeg + i] : -2;
    int fc = -1, ns = -1;
    for (int k = i + 1; k < N && (fc < 0 || ns < 0); ++k) {
      const int pk = parent[nbeg + k];
      if (fc < 0 && pk == i) fc = k;
      if (ns < 0 && pk == pi) ns = k;
    }
    if (first_child) first_child[nbeg + i] = fc;
    if (next_sibling) next_sibling[nbeg + i] = ns;
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint4* p, size_t n16, uint8_t* tail,
                                                        size_t ntail) {
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

}  // namespace

hipError_t launch_accept_path(int32_t batch, int32_t max_depth, const int32_t* node_indptr,
                              const int32_t* parent, const int32_t* tokens,
                              const int8_t* flag, const int32_t* next_token,
                              const int32_t* prefix_len, int32_t* path_nodes,
                              int32_t* out_tokens, int32_t* out_len, int32_t* kv_keep,
                              uint32_t* status, hipStream_t stream) {
  hipLaunchKernelGGL(accept_path_kernel, dim3(batch), dim3(64), 0, stream, batch, max_depth + 1,
                     node_indptr, parent, tokens, flag, next_token, prefix_len, path_nodes,
                     out_tokens, out_len, kv_keep, status);
  return hipGetLastError();
}

hipError_t launch_tree_meta(int32_t batch, int32_t max_nodes, const int32_t* node_indptr,
                            const int32_t* parent, int32_t* depth, uint32_t* anc_bits,
                            int32_t* first_child, int32_t* next_sibling, uint32_t* status,
                            hipStream_t stream) {
  const int words = (max_nodes + 31) / 32;
  const dim3 grid((max_nodes + 255) / 256, batch);
  hipLaunchKernelGGL(tree_meta_kernel, grid, dim3(256), 0, stream, batch, words, node_indptr,
                     parent, depth, anc_bits, first_child, next_sibling, status);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* ptr, size_t bytes, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  const size_t ntail = bytes - n16 * 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream,
                     static_cast<uint4*>(ptr), n16, static_cast<uint8_t*>(ptr) + n16 * 16, ntail);
  return hipGetLastError();
}

}  // namespace tv
