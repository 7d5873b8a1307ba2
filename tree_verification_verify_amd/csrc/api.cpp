// C ABI of libtreeverify: argument checks, workspace layout and launches.
// Host-detectable errors are returned before anything is enqueued; nothing
// here allocates device memory or synchronises (tv_device_status aside).
#include <stdio.h>
#include <string.h>

#include <vector>

#include "tv_device.hpp"
#include "tv_internal.hpp"

namespace {

thread_local char g_last_hip_error[256] = "";

tv_status hip_fail(hipError_t e, const char* where) {
  snprintf(g_last_hip_error, sizeof(g_last_hip_error), "%s: %s", where, hipGetErrorString(e));
  return TV_ERR_HIP;
}

bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

}  // namespace

extern "C" {

int32_t tv_version(void) { return 1; }

const char* tv_last_hip_error(void) { return g_last_hip_error; }

const char* tv_status_string(tv_status s) {
  switch (s) {
    case TV_OK: return "ok";
    case TV_ERR_NULL: return "required pointer is NULL";
    case TV_ERR_SHAPE: return "inconsistent or unsupported sizes";
    case TV_ERR_DTYPE: return "unsupported dtype";
    case TV_ERR_WORKSPACE: return "workspace too small or misaligned";
    case TV_ERR_TREE: return "parent array is not a topologically ordered tree";
    case TV_ERR_PAGES: return "page table does not cover the request or page id out of range";
    case TV_ERR_HIP: return "HIP runtime error";
    case TV_ERR_LOGITS: return "non-finite logits, bad temperature or missing draft logits";
    case TV_ERR_PATH: return "invalid accepted path (two accepted siblings, deeper than max_depth) or keep-list";
    case TV_ERR_TIMEOUT: return "team barrier exceeded its spin limit";
  }
  return "unknown status";
}

size_t tv_attn_workspace_size(const tv_attn_desc* desc) {
  if (!desc) return 0;
  tv::AttnPlan pl;
  if (!tv::plan_attn(*desc, &pl)) return 0;
  return pl.total_bytes;
}

size_t tv_sample_workspace_size(const tv_sample_desc* desc) {
  if (!desc) return 0;
  tv::SamplePlan pl;
  if (!tv::plan_sample(*desc, &pl)) return 0;
  return pl.total_bytes;
}

tv_status tv_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!workspace) return TV_ERR_NULL;
  if (workspace_bytes < tv::kHeaderBytes || !aligned256(workspace)) return TV_ERR_WORKSPACE;
  hipError_t e = tv::launch_fill_zero(workspace, workspace_bytes, stream);
  if (e != hipSuccess) return hip_fail(e, "tv_workspace_init");
  return TV_OK;
}

tv_status tv_device_status(const void* workspace, hipStream_t stream, uint32_t* bits_out) {
  if (!workspace) return TV_ERR_NULL;
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "tv_device_status sync");
  uint32_t bits = 0;
  e = hipMemcpy(&bits, workspace, sizeof(bits), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "tv_device_status read");
  if (bits_out) *bits_out = bits;
  if (bits & TV_DEV_TIMEOUT) return TV_ERR_TIMEOUT;
  if (bits & TV_DEV_TREE) return TV_ERR_TREE;
  if (bits & TV_DEV_PAGES) return TV_ERR_PAGES;
  if (bits & TV_DEV_SHAPE) return TV_ERR_SHAPE;
  if (bits & TV_DEV_LOGITS) return TV_ERR_LOGITS;
  if (bits & TV_DEV_PATH) return TV_ERR_PATH;
  return TV_OK;
}

tv_status tree_verify_attn(const tv_attn_desc* desc, const void* q, const void* k_pages,
                           const void* v_pages, const int32_t* page_indptr,
                           const int32_t* page_indices, const int32_t* prefix_len,
                           const int32_t* node_indptr, const int32_t* parent, void* out,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!desc) return TV_ERR_NULL;
  if (desc->dtype != TV_BF16 && desc->dtype != TV_FP32) return TV_ERR_DTYPE;
  tv::AttnPlan pl;
  if (!tv::plan_attn(*desc, &pl)) return TV_ERR_SHAPE;
  if (!q || !k_pages || !v_pages || !page_indptr || !page_indices || !prefix_len ||
      !node_indptr || !parent || !out || !workspace)
    return TV_ERR_NULL;
  if (workspace_bytes < pl.total_bytes || !aligned256(workspace)) return TV_ERR_WORKSPACE;
  tv::AttnArgs a{q, k_pages, v_pages, page_indptr, page_indices, prefix_len,
                 node_indptr, parent, out, workspace};
  hipError_t e = tv::launch_attn(*desc, pl, a, stream);
  if (e != hipSuccess) return hip_fail(e, "tree_verify_attn");
  return TV_OK;
}

tv_status tree_spec_sample(const tv_sample_desc* desc, const float* target_logits,
                           const float* draft_logits, const int32_t* tokens,
                           const int32_t* node_indptr, const int32_t* parent,
                           const float* temperature, const float* uniforms,
                           int8_t* accept_flag, int32_t* next_token, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  if (!desc) return TV_ERR_NULL;
  tv::SamplePlan pl;
  if (!tv::plan_sample(*desc, &pl)) return TV_ERR_SHAPE;
  if (!target_logits || !tokens || !node_indptr || !parent || !temperature || !uniforms ||
      !accept_flag || !next_token || !workspace)
    return TV_ERR_NULL;
  if (workspace_bytes < pl.total_bytes || !aligned256(workspace)) return TV_ERR_WORKSPACE;
  tv::SampleArgs a{target_logits, draft_logits, tokens, node_indptr, parent, temperature,
                   uniforms, accept_flag, next_token, workspace};
  hipError_t e = tv::launch_sample(*desc, pl, a, stream);
  if (e != hipSuccess) return hip_fail(e, "tree_spec_sample");
  return TV_OK;
}

tv_status tree_spec_sample_noalloc(const tv_sample_desc* desc, const float* target_logits,
                                   const float* draft_logits, const int32_t* tokens,
                                   const int32_t* node_indptr, const int32_t* parent,
                                   const float* temperature, const float* uniforms,
                                   int8_t* accept_flag, int32_t* next_token, uint32_t* status,
                                   hipStream_t stream) {
  if (!desc) return TV_ERR_NULL;
  tv::SamplePlan pl;
  if (!tv::plan_sample(*desc, &pl)) return TV_ERR_SHAPE;
  if (desc->batch > TV_SAMPLE_STATIC_MAX_BATCH) return TV_ERR_SHAPE;
  if (!target_logits || !tokens || !node_indptr || !parent || !temperature || !uniforms ||
      !accept_flag || !next_token || !status)
    return TV_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(status) & 3u) != 0) return TV_ERR_WORKSPACE;
  tv::SampleArgs a{target_logits, draft_logits, tokens, node_indptr, parent, temperature,
                   uniforms, accept_flag, next_token, nullptr};
  hipError_t e = tv::launch_sample_static(*desc, a, status, stream);
  if (e != hipSuccess) return hip_fail(e, "tree_spec_sample_noalloc");
  return TV_OK;
}

tv_status tree_accept_path(int32_t batch, int32_t max_depth, const int32_t* node_indptr,
                           const int32_t* parent, const int32_t* tokens,
                           const int8_t* accept_flag, const int32_t* next_token,
                           const int32_t* prefix_len, int32_t* path_nodes,
                           int32_t* out_tokens, int32_t* out_len, int32_t* kv_keep,
                           void* status_workspace, hipStream_t stream) {
  if (batch < 1 || max_depth < 0 || max_depth > 65535) return TV_ERR_SHAPE;
  if (!node_indptr || !parent || !tokens || !accept_flag || !next_token || !prefix_len ||
      !path_nodes || !out_tokens || !out_len || !kv_keep)
    return TV_ERR_NULL;
  hipError_t e = tv::launch_accept_path(batch, max_depth, node_indptr, parent, tokens,
                                        accept_flag, next_token, prefix_len, path_nodes,
                                        out_tokens, out_len, kv_keep,
                                        static_cast<uint32_t*>(status_workspace), stream);
  if (e != hipSuccess) return hip_fail(e, "tree_accept_path");
  return TV_OK;
}

tv_status tree_kv_commit(const tv_attn_desc* desc, int32_t num_layers, int64_t layer_stride,
                         void* k_pages, void* v_pages, const int32_t* page_indptr,
                         const int32_t* page_indices, const int32_t* prefix_len,
                         const int32_t* kv_keep, const int32_t* out_len, int32_t max_depth,
                         void* status_workspace, hipStream_t stream) {
  if (!desc) return TV_ERR_NULL;
  const tv_attn_desc& d = *desc;
  if (d.dtype != TV_BF16 && d.dtype != TV_FP32) return TV_ERR_DTYPE;
  if (d.batch < 1 || d.num_kv_heads < 1 || (d.head_dim != 64 && d.head_dim != 128) ||
      d.num_pages < 1 || d.max_nodes < 1 || num_layers < 1 || max_depth < 0 || max_depth > 65535)
    return TV_ERR_SHAPE;
  const long long pool = (long long)d.num_pages * d.num_kv_heads * tv::kPage * d.head_dim;
  const int elem = d.dtype == TV_BF16 ? 2 : 4;
  if (layer_stride < pool || (layer_stride * elem) % 16 != 0) return TV_ERR_SHAPE;
  if ((long long)d.batch * num_layers > 0x7fffffffLL) return TV_ERR_SHAPE;
  if (!k_pages || !v_pages || !page_indptr || !page_indices || !prefix_len || !kv_keep || !out_len)
    return TV_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(k_pages) | reinterpret_cast<uintptr_t>(v_pages)) & 15u)
    return TV_ERR_SHAPE;
  hipError_t e = tv::launch_kv_commit(d, num_layers, layer_stride, k_pages, v_pages, page_indptr,
                                      page_indices, prefix_len, kv_keep, out_len, max_depth,
                                      static_cast<uint32_t*>(status_workspace), stream);
  if (e != hipSuccess) return hip_fail(e, "tree_kv_commit");
  return TV_OK;
}

tv_status tree_draw_siblings(int32_t rows, int32_t vocab, const float* draft_logits,
                             const int32_t* counts, const float* temperature, uint32_t stream_id,
                             uint64_t seed, int32_t* tokens, void* status_workspace,
                             hipStream_t stream) {
  if (rows < 1 || vocab < 1 || rows > 0x7fffffff) return TV_ERR_SHAPE;
  if (!draft_logits || !counts || !temperature || !tokens) return TV_ERR_NULL;
  hipError_t e = tv::launch_draw_siblings(rows, vocab, draft_logits, counts, temperature, stream_id,
                                          seed, tokens, static_cast<uint32_t*>(status_workspace),
                                          stream);
  if (e != hipSuccess) return hip_fail(e, "tree_draw_siblings");
  return TV_OK;
}

tv_status tree_expand_step(int32_t batch, int32_t vocab, int32_t k_in, int32_t k,
                           const float* draft_logits, const int32_t* frontier,
                           int32_t cand_capacity, int32_t cand_offset, float* cand_value,
                           int32_t* cand_token, int32_t* cand_parent, int32_t* next_frontier,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (batch < 1 || k < 1 || k > tv::kMaxExpand || k_in < 1 || k_in > tv::kMaxExpand ||
      vocab < k || cand_offset < 0 || cand_capacity < 1 ||
      long(cand_offset) + long(k_in) * k > long(cand_capacity) ||
      long(batch) * k_in > 0x7fffffffL)
    return TV_ERR_SHAPE;
  if (!draft_logits || !cand_value || !cand_token || !cand_parent || !next_frontier)
    return TV_ERR_NULL;
  if (workspace && !aligned256(workspace)) return TV_ERR_WORKSPACE;
  hipError_t e = tv::launch_expand_step(batch, vocab, k_in, k, draft_logits, frontier,
                                        cand_capacity, cand_offset, cand_value, cand_token,
                                        cand_parent, next_frontier, workspace, workspace_bytes,
                                        stream);
  if (e != hipSuccess) return hip_fail(e, "tree_expand_step");
  return TV_OK;
}

size_t tv_expand_workspace_size(int32_t batch, int32_t k_in, int32_t k) {
  if (batch < 1 || k < 1 || k > tv::kMaxExpand || k_in < 1 || k_in > tv::kMaxExpand) return 0;
  return tv::expand_workspace_bytes(batch, k_in, k);
}

tv_status tree_rerank(int32_t batch, int32_t num_cand, int32_t cand_capacity, int32_t m,
                      const float* cand_value, const int32_t* cand_token,
                      const int32_t* cand_parent, int32_t* out_parent, int32_t* out_token,
                      int32_t* out_count, void* status_workspace, hipStream_t stream) {
  if (batch < 1 || num_cand < 1 || num_cand > cand_capacity || num_cand > tv::kMaxRerank ||
      m < 1 || m >= 0x7fffffff)
    return TV_ERR_SHAPE;
  if (!cand_value || !cand_token || !cand_parent || !out_parent || !out_token || !out_count)
    return TV_ERR_NULL;
  hipError_t e = tv::launch_rerank(batch, num_cand, cand_capacity, m, cand_value, cand_token,
                                   cand_parent, out_parent, out_token, out_count,
                                   static_cast<uint32_t*>(status_workspace), stream);
  if (e != hipSuccess) return hip_fail(e, "tree_rerank");
  return TV_OK;
}

namespace {
bool spark_desc_ok(const tv_spark_desc& d) {
  return d.batch >= 1 && d.batch <= tv::kSparkMaxBatch && d.max_siblings >= 1 &&
         d.max_siblings <= tv::kSparkMaxSiblings && d.vocab >= d.max_siblings + 1 &&
         d.vocab <= tv::kSparkMaxVocab && d.rank >= 32 &&
         d.rank <= 256 && d.rank % 32 == 0 && d.depths >= 1 && d.depths <= tv::kSparkMaxDepths &&
         d.max_nodes >= 1 && d.max_nodes <= tv::kSparkMaxNodes && d.calib_a == d.calib_a &&
         d.calib_b == d.calib_b;
}
}  // namespace

size_t tv_spark_workspace_size(const tv_spark_desc* desc) {
  if (!desc || !spark_desc_ok(*desc)) return 0;
  return tv::spark_workspace_bytes(*desc);
}

tv_status tree_spark_build(const tv_spark_desc* desc, const float* base_logits, const void* w1,
                           const void* w2, const int32_t* anchor, const float* temperature,
                           const float* theta, uint32_t stream_id, uint64_t seed,
                           int32_t* out_parent, int32_t* out_token, int32_t* out_count,
                           float* out_logsurv, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  if (!desc) return TV_ERR_NULL;
  if (!spark_desc_ok(*desc)) return TV_ERR_SHAPE;
  if (!base_logits || !w1 || !w2 || !anchor || !temperature || !theta || !out_parent ||
      !out_token || !out_count || !workspace)
    return TV_ERR_NULL;
  if (workspace_bytes < tv::spark_workspace_bytes(*desc) || !aligned256(workspace))
    return TV_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(w1) & 15u) || (reinterpret_cast<uintptr_t>(w2) & 15u) ||
      (reinterpret_cast<uintptr_t>(base_logits) & 15u))
    return TV_ERR_SHAPE;
  tv::SparkArgs a{base_logits, w1, w2, anchor, temperature, theta, stream_id, seed,
                  out_parent, out_token, out_count, out_logsurv, workspace};
  hipError_t e = tv::launch_spark(*desc, a, stream);
  if (e != hipSuccess) return hip_fail(e, "tree_spark_build");
  return TV_OK;
}

tv_status tv_tree_meta(int32_t batch, int32_t max_nodes, const int32_t* node_indptr,
                       const int32_t* parent, int32_t* depth, uint32_t* anc_bits,
                       int32_t* first_child, int32_t* next_sibling, void* status_workspace,
                       hipStream_t stream) {
  if (batch < 1 || max_nodes < 1 || max_nodes > (1 << 16)) return TV_ERR_SHAPE;
  if (!node_indptr || !parent) return TV_ERR_NULL;
  hipError_t e = tv::launch_tree_meta(batch, max_nodes, node_indptr, parent, depth, anc_bits,
                                      first_child, next_sibling,
                                      static_cast<uint32_t*>(status_workspace), stream);
  if (e != hipSuccess) return hip_fail(e, "tv_tree_meta");
  return TV_OK;
}

tv_status tv_validate_tree(int32_t batch, const int32_t* node_indptr_host,
                           const int32_t* parent_host, int32_t max_nodes, int32_t max_depth) {
  if (!node_indptr_host || !parent_host) return TV_ERR_NULL;
  if (batch < 1 || node_indptr_host[0] != 0) return TV_ERR_SHAPE;
  std::vector<int32_t> depth;
  for (int r = 0; r < batch; ++r) {
    const int a = node_indptr_host[r], b = node_indptr_host[r + 1];
    const int n = b - a;
    if (n < 0) return TV_ERR_SHAPE;
    if (n > max_nodes) return TV_ERR_TREE;
    if (n == 0) continue;
    depth.assign(size_t(n), 0);
    if (parent_host[a] != -1) return TV_ERR_TREE;
    for (int i = 1; i < n; ++i) {
      const int p = parent_host[a + i];
      if (p < 0 || p >= i) return TV_ERR_TREE;
      depth[i] = depth[p] + 1;
      if (depth[i] > max_depth) return TV_ERR_TREE;
    }
  }
  return TV_OK;
}

tv_status tv_validate_pages(int32_t batch, const int32_t* page_indptr_host,
                            const int32_t* page_indices_host, const int32_t* prefix_len_host,
                            const int32_t* node_indptr_host, int32_t num_pages,
                            int32_t page_size) {
  if (!page_indptr_host || !page_indices_host || !prefix_len_host || !node_indptr_host)
    return TV_ERR_NULL;
  if (batch < 1 || page_size != tv::kPage || num_pages < 1) return TV_ERR_SHAPE;
  if (page_indptr_host[0] != 0) return TV_ERR_PAGES;
  for (int r = 0; r < batch; ++r) {
    const long L = long(prefix_len_host[r]) + (node_indptr_host[r + 1] - node_indptr_host[r]);
    const long np = long(page_indptr_host[r + 1]) - page_indptr_host[r];
    if (prefix_len_host[r] < 0 || np < 0) return TV_ERR_PAGES;
    if (np * page_size < L) return TV_ERR_PAGES;
    for (long k = page_indptr_host[r]; k < page_indptr_host[r + 1]; ++k) {
      const int pg = page_indices_host[k];
      if (pg < 0 || pg >= num_pages) return TV_ERR_PAGES;
    }
  }
  return TV_OK;
}

}  // extern "C"
