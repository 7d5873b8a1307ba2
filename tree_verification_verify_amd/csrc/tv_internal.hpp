// Host-side plans and launcher declarations shared by api.cpp and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tree_verify.h"

namespace tv {

// Launch geometry of tree_verify_attn, derived from the descriptor only, so
// the workspace size is known without touching the GPU.
struct AttnPlan {
  bool mfma;          // bf16 MFMA kernel (true) or fp32 VALU kernel
  int group;          // G = Hq / Hkv
  int rows_pb;        // rows (node x grouped head) per row block
  int rb_max;         // row blocks per (request, kv head)
  int words;          // 32-bit words per ancestor bitset row
  // fp32 VALU kernel: one workgroup per (request, kv head, row block, split)
  int chunk_len;      // keys per split (multiple of 32)
  int c_max;          // splits per (request, kv head) at max_kv_len
  // bf16 MFMA kernel: persistent workgroups, each streaming an equal share of
  // the 64-key tiles of all (request, kv head, row block) pairs
  int nwg;            // workgroups (a power of two >= 8)
  int lg_nwg;         // log2(nwg)
  int ns;             // stage ring slots (4, or 2 when LDS is short)
  size_t slots;       // partial-result slots
  size_t grid;        // launch size (multiple of 8: XCD-aware remap)
  size_t dyn_lds;     // dynamic LDS bytes per workgroup
  size_t off_counters, off_desc, off_ml, off_o, total_bytes;
};

struct SamplePlan {
  int threads;        // threads per workgroup
  size_t off_req;     // per-request blocks (barrier counter, tag sequence, exchange slots)
  size_t total_bytes;
};

bool plan_attn(const tv_attn_desc& d, AttnPlan* out);
bool plan_sample(const tv_sample_desc& d, SamplePlan* out);

// Limit of the kernels' bounded waits in real-time counter ticks (100 MHz):
// 0.2 s, or TREEVERIFY_TEAM_WAIT_US microseconds when that variable is set.
uint64_t wait_ticks();

struct AttnArgs {
  const void* q;
  const void* k_pages;
  const void* v_pages;
  const int32_t* page_indptr;
  const int32_t* page_indices;
  const int32_t* prefix_len;
  const int32_t* node_indptr;
  const int32_t* parent;
  void* out;
  void* workspace;
};

hipError_t launch_attn(const tv_attn_desc& d, const AttnPlan& plan, const AttnArgs& a,
                       hipStream_t stream);

struct SampleArgs {
  const float* target;
  const float* draft;
  const int32_t* tokens;
  const int32_t* node_indptr;
  const int32_t* parent;
  const float* temperature;
  const float* uniforms;
  int8_t* flag;
  int32_t* next_token;
  void* workspace;
};

hipError_t launch_sample(const tv_sample_desc& d, const SamplePlan& plan, const SampleArgs& a,
                         hipStream_t stream);
// Bytes of one request's block of sampler synchronisation state (greedy
// barrier counter, exchange tag sequence, exchange words).
constexpr size_t kSampleReqBytes = 2304;
// One launch of the walk with its status word and per-request blocks given
// (a.workspace unused).
hipError_t launch_sample_core(const tv_sample_desc& d, const SampleArgs& a, uint32_t* status,
                              char* req, hipStream_t stream);
// The walk with its per-request blocks in the library's static device array
// (cleared first) and its status bits in *status.
hipError_t launch_sample_static(const tv_sample_desc& d, const SampleArgs& a, uint32_t* status,
                                hipStream_t stream);

hipError_t launch_accept_path(int32_t batch, int32_t max_depth, const int32_t* node_indptr,
                              const int32_t* parent, const int32_t* tokens,
                              const int8_t* flag, const int32_t* next_token,
                              const int32_t* prefix_len, int32_t* path_nodes,
                              int32_t* out_tokens, int32_t* out_len, int32_t* kv_keep,
                              uint32_t* status, hipStream_t stream);

hipError_t launch_tree_meta(int32_t batch, int32_t max_nodes, const int32_t* node_indptr,
                            const int32_t* parent, int32_t* depth, uint32_t* anc_bits,
                            int32_t* first_child, int32_t* next_sibling, uint32_t* status,
                            hipStream_t stream);

hipError_t launch_kv_commit(const tv_attn_desc& d, int32_t num_layers, long long layer_stride,
                            void* k_pages, void* v_pages, const int32_t* page_indptr,
                            const int32_t* page_indices, const int32_t* prefix_len,
                            const int32_t* kv_keep, const int32_t* out_len, int32_t max_depth,
                            uint32_t* status, hipStream_t stream);

hipError_t launch_draw_siblings(int32_t rows, int32_t vocab, const float* draft_logits,
                                const int32_t* counts, const float* temperature, uint32_t stream_id,
                                uint64_t seed, int32_t* tokens, uint32_t* status,
                                hipStream_t stream);

// Draft-tree construction (expansion round, rerank).
constexpr int kMaxRerank = 4096;  // candidates per request the rerank holds in LDS
constexpr int kMaxExpand = 16;    // children per node and frontier slots per round
constexpr int kMaxSplit = 8;      // workgroups per row in rounds with few rows
size_t expand_workspace_bytes(int32_t batch, int32_t k_in, int32_t k);
hipError_t launch_expand_step(int32_t batch, int32_t vocab, int32_t k_in, int32_t k,
                              const float* logits, const int32_t* frontier, int32_t cap,
                              int32_t offset, float* value, int32_t* token, int32_t* parent,
                              int32_t* next, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);
hipError_t launch_rerank(int32_t batch, int32_t num_cand, int32_t cap, int32_t m,
                         const float* value, const int32_t* token, const int32_t* parent,
                         int32_t* out_parent, int32_t* out_token, int32_t* out_count,
                         uint32_t* status, hipStream_t stream);

hipError_t launch_fill_zero(void* ptr, size_t bytes, hipStream_t stream);

// TreeSpark best-first construction.
constexpr int kSparkMaxNodes = 64;      // drafted nodes per tree
constexpr int kSparkMaxSiblings = 16;   // children per node
constexpr int kSparkRowsPerRound = 4;   // expansions per request per round
constexpr int kSparkMaxBatch = 256;
constexpr int kSparkMaxRows = kSparkMaxBatch * kSparkRowsPerRound;
constexpr int kSparkMaxDepths = 16;
constexpr int kSparkMaxVocab = 1 << 22;  // w2 (V x r bf16) stays under 4 GB: 32-bit load offsets
// Segments per expanded row in the statistics phase: at most one item per
// workgroup, at most kSparkMaxSeg.
constexpr int kSparkMaxSeg = 32;
__host__ __device__ inline int spark_segments(int rows, int nwg) {
  if (rows <= 0) return 1;
  const int s = nwg / rows;
  return s < 1 ? 1 : (s > kSparkMaxSeg ? kSparkMaxSeg : s);
}
struct SparkArgs {
  const float* base_logits;
  const void* w1;
  const void* w2;
  const int32_t* anchor;
  const float* temperature;
  const float* theta;
  uint32_t stream_id;
  uint64_t seed;
  int32_t* out_parent;
  int32_t* out_token;
  int32_t* out_count;
  float* out_logsurv;
  void* workspace;
};
size_t spark_workspace_bytes(const tv_spark_desc& d);
hipError_t launch_spark(const tv_spark_desc& d, const SparkArgs& a, hipStream_t stream);

}  // namespace tv
