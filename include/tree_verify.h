/*
 * tree_verify.h — C ABI of libtreeverify, tree verification for tree-based
 * speculative decoding on AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages; sections named, not line numbers):
 *   [survey]    "Tree-based speculative decoding: draft trees win latency,
 *               lose batches, return cost-aware", sections Timeline,
 *               Taxonomy, Systems.
 *   [TreeSpark] TreeSpark: Markov-conditioned draft trees (paper 2609.22098),
 *               §3.1, §3.2 (step 3), §3.3 (Proposition 1), §4, §5.1.
 *   [explainer] tree-vs-chain explainer, "Red flags & common mistakes".
 *
 * Conventions (all entry points)
 *   - Array arguments are DEVICE pointers unless the name ends in _host.
 *   - The caller owns every buffer, the workspace included. The library never
 *     allocates device memory, never synchronises (tv_device_status aside)
 *     and keeps no per-call state outside the workspace (the one exception,
 *     tree_spec_sample_noalloc, uses a fixed device array of the library's
 *     own). Host-side argument errors are returned before anything is
 *     launched.
 *   - Calls are stream-ordered and re-entrant; concurrent streams need
 *     distinct workspaces. A workspace must be zero-filled once
 *     (tv_workspace_init) before its first use and then belongs to one
 *     entry point: calls keep synchronisation state in it between calls.
 *     A tree_spec_sample workspace keeps that state per request at fixed
 *     offsets, so it serves any later call whose batch fits the size it
 *     was sized for. A tree_verify_attn workspace is laid out by its
 *     descriptor: before reusing it with another descriptor, zero-fill it
 *     again.
 *   - Anomalies found on the device (bad parent, page id out of range, too
 *     few pages, NaN/Inf logits, two accepted siblings, a stalled team
 *     barrier) set bits of a status word at the start of the workspace; they
 *     never fault. Read it with tv_device_status; clear it with
 *     tv_workspace_init.
 *   - Trees are flattened in topological order: request r owns rows
 *     node_indptr[r] .. node_indptr[r+1]-1; parent[] holds request-local
 *     indices with parent[0] = -1 and 0 <= parent[i] < i; siblings appear in
 *     ascending index in draw order ([survey] Timeline: tree tokens stored in
 *     the KV cache by topology; [TreeSpark] §1: sibling draw order).
 */
#ifndef TREE_VERIFY_H
#define TREE_VERIFY_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TV_OK = 0,
  TV_ERR_NULL = 1,       /* a required pointer is NULL */
  TV_ERR_SHAPE = 2,      /* inconsistent or unsupported sizes */
  TV_ERR_DTYPE = 3,      /* unsupported element type */
  TV_ERR_WORKSPACE = 4,  /* workspace too small or misaligned */
  TV_ERR_TREE = 5,       /* parent array violates the topological rules */
  TV_ERR_PAGES = 6,      /* page table does not cover a request or id out of range */
  TV_ERR_HIP = 7,        /* a HIP runtime call failed (tv_last_hip_error) */
  TV_ERR_LOGITS = 8,     /* NaN or Inf logits, or draft logits missing at T > 0 */
  TV_ERR_PATH = 9,       /* invalid accepted path (two accepted siblings, too deep) or keep-list */
  TV_ERR_TIMEOUT = 10    /* a team barrier exceeded its spin limit */
} tv_status;

typedef enum { TV_FP32 = 0, TV_BF16 = 1 } tv_dtype;

/* Verification rule of tree_spec_sample at T > 0 ([survey] Taxonomy).
 * Without replacement (rule (c)): siblings are distinct draws, each from q
 * without the tokens drawn before it. With replacement (rule (b), SpecInfer's
 * multi-step speculative sampling, MCSD Algorithm 1): siblings are
 * independent draws from q. Each rule reproduces the target distribution
 * only for siblings drawn its own way. */
typedef enum { TV_RULE_WITHOUT_REPLACEMENT = 0, TV_RULE_WITH_REPLACEMENT = 1 } tv_rule;

/* What tree_spec_sample computes for greedy (T == 0) requests ([survey]
 * Taxonomy rule (a); [TreeSpark] §3.2 step 3: exact target-token matching).
 * Every node: the argmax of every target row and the match flag of every
 * node. Path: only the rows the walk visits are read; the accepted path,
 * emitted tokens and keep-list that tree_accept_path derives are the same. */
typedef enum { TV_GREEDY_EVERY_NODE = 0, TV_GREEDY_PATH = 1 } tv_greedy;

/* Bits of the device status word (first 4 bytes of a workspace). */
enum {
  TV_DEV_TREE = 1u << 0,
  TV_DEV_PAGES = 1u << 1,
  TV_DEV_LOGITS = 1u << 2,
  TV_DEV_PATH = 1u << 3,
  TV_DEV_TIMEOUT = 1u << 4,
  TV_DEV_SHAPE = 1u << 5
};

/* Attention problem description (host memory). Maxima bound every request
 * and size the launch and the workspace; the device rejects requests that
 * exceed them (status bit TV_DEV_SHAPE) instead of reading past a buffer. */
typedef struct {
  int32_t batch;         /* B >= 1 */
  int32_t num_q_heads;   /* Hq, a multiple of num_kv_heads */
  int32_t num_kv_heads;  /* Hkv; q head h reads kv head h / (Hq/Hkv) */
  int32_t head_dim;      /* D: 64 or 128 */
  int32_t page_size;     /* must be 16 */
  int32_t max_nodes;     /* >= max_r N_r, <= 1024 */
  int32_t max_depth;     /* >= deepest node (edges from the root) */
  int32_t max_kv_len;    /* >= max_r (P_r + N_r) */
  int32_t num_pages;     /* physical pages in k_pages / v_pages */
  tv_dtype dtype;        /* TV_BF16 (MFMA path) or TV_FP32 (VALU path) */
  float sm_scale;        /* softmax scale; 0 means 1/sqrt(D) */
} tv_attn_desc;

/* Sampler problem description (host memory). */
typedef struct {
  int32_t batch;         /* B >= 1 */
  int32_t vocab;         /* V >= 1 */
  int32_t max_nodes;     /* >= max_r N_r, <= 65536 */
  int32_t max_depth;     /* >= deepest node */
  int32_t rule;          /* tv_rule; 0 (a zero-filled desc) is without replacement */
  int32_t greedy;        /* tv_greedy; 0 (a zero-filled desc) is every node */
} tv_sample_desc;

/* ---- workspace -------------------------------------------------------- */

/* Bytes of workspace tree_verify_attn needs for desc (0 if desc is invalid).
 * Holds the status word, split-merge counters and fp32 partial results. */
size_t tv_attn_workspace_size(const tv_attn_desc* desc);

/* Bytes of workspace tree_spec_sample needs (0 if desc is invalid). */
size_t tv_sample_workspace_size(const tv_sample_desc* desc);

/* Zero-fill a workspace on stream (a fill kernel, safe under graph capture).
 * Required once before first use, and after any call that reported a
 * device error. */
tv_status tv_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Synchronise stream, read the status word of workspace, return the
 * highest-priority error it holds (TV_OK if none) and, if bits_out is not
 * NULL, the raw TV_DEV_* bits. Does not clear them. */
tv_status tv_device_status(const void* workspace, hipStream_t stream, uint32_t* bits_out);

/* ---- the hot path ----------------------------------------------------- */

/* Tree-masked attention, one layer ([survey] Timeline: SpecInfer's
 * tree-based parallel decoding — tree tokens in the KV cache in topological
 * order, attention masked to ancestors; [TreeSpark] §3.2 step 3: one target
 * pass with a tree attention mask; §4: ancestor-bitmask mask).
 *
 * For request r, q head h, local row i (logical position P_r + i):
 *   visible(i) = {0 .. P_r-1} U {P_r + j : j ancestor of i or j == i}
 *   out[i,h]   = sum_{t in visible(i)} softmax_t(sm_scale * q[i,h].K[t,g]) V[t,g],
 *   g = h / (Hq / Hkv).
 * Arguments:
 *   q        [T][Hq][D] in desc->dtype, T = node_indptr[B]
 *   k_pages  [num_pages][Hkv][16][D] in desc->dtype (one 16-token page per
 *            page and kv head, a key's D channels contiguous)
 *   v_pages  [num_pages][Hkv][D][16] in desc->dtype: V transposed within
 *            each page (one channel's 16 tokens contiguous), so a V tile
 *            is already in the layout the PV matrix product consumes.
 *            Logical position t of request r lives in physical page
 *            pg = page_indices[page_indptr[r] + t/16], slot s = t%16:
 *            K[t] = k_pages[pg][g][s][:], V[t] = v_pages[pg][g][:][s].
 *            The caller has already written the tree's own K/V at
 *            P_r .. P_r+N_r-1 (with RoPE at per-depth positions applied
 *            before the call). Slots past P_r+N_r in the last page are
 *            never used (their contents do not matter).
 *   page_indptr [B+1], page_indices [page_indptr[B]]  (int32)
 *   prefix_len [B]   P_r >= 0 (int32)
 *   node_indptr [B+1], parent [T]  (int32; see the tree conventions above)
 *   out      [T][Hq][D] in desc->dtype (bf16 rounded to nearest even from fp32)
 *   workspace >= tv_attn_workspace_size(desc) bytes, 256-byte aligned.
 * Returns TV_OK after launching; device-side problems go to the status word
 * (the affected rows are then unspecified, never out-of-bounds). */
tv_status tree_verify_attn(const tv_attn_desc* desc,
                           const void* q, const void* k_pages, const void* v_pages,
                           const int32_t* page_indptr, const int32_t* page_indices,
                           const int32_t* prefix_len, const int32_t* node_indptr,
                           const int32_t* parent, void* out,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Multi-step speculative sampling over the tree ([survey] Timeline and
 * Taxonomy rules (a), (c) and (b); [TreeSpark] §1 and §3.3, Proposition 1).
 *
 * Returns TV_ERR_SHAPE when desc->rule is not a tv_rule value or
 * desc->greedy not a tv_greedy value.
 * Row i of the logits is the distribution of the token AFTER node i
 * ([TreeSpark] §3.1, LM-shifted alignment). Per request r with T = temperature[r]:
 *   T == 0 (greedy exact match), desc->greedy == TV_GREEDY_EVERY_NODE:
 *     next_token[i] = argmax target row i (lowest index on ties) for EVERY
 *     node; accept_flag[i] = (tokens[i] == next_token[parent[i]]);
 *     accept_flag[root] = 1.
 *   T == 0, desc->greedy == TV_GREEDY_PATH: the same along the walk only.
 *     From the root v: next_token[v] = argmax target row v; every child c of
 *     v gets accept_flag[c] = (tokens[c] == next_token[v]); the walk moves
 *     to the first flagged child (draw order) and stops at a node with
 *     none. Nodes the walk never tests keep accept_flag 0 and next_token -1
 *     (non-finite logits are detected in the visited rows only).
 *   T > 0 (rejection walk): starting at the root v, with
 *     p = softmax(target_v / T), q = softmax(draft_v / T), the children
 *     c_1 < c_2 < ... of v (draw order) are tested in turn: c_j is accepted
 *     iff uniforms[c_j][0] < p_j(x_j) / q_j(x_j), where q_j is q with the
 *     tokens x_1..x_{j-1} removed and renormalised (desc->rule ==
 *     TV_RULE_WITHOUT_REPLACEMENT) or q itself (TV_RULE_WITH_REPLACEMENT), and
 *     p_j the residual (p_1 = p; after a rejection p_{j+1} = max(p_j - q_j, 0)
 *     renormalised).
 *     An accepted child becomes v. When no child is accepted (or v is a
 *     leaf) the walk stops: next_token[v] = smallest y with
 *     cumsum(p_final)[y] > uniforms[v][1] * sum(p_final), p_final being the
 *     residual (the target p at a leaf or when v has no children).
 *     accept_flag: 1 for the root and accepted nodes, 0 otherwise (tested
 *     and rejected, or never tested); next_token = -1 except at the stop node.
 * Arguments:
 *   target_logits, draft_logits [T][V] fp32; draft_logits may be NULL when
 *     every temperature is 0 (a T > 0 request then sets TV_DEV_LOGITS).
 *   tokens [T] int32 token of each node (root ignored); siblings distinct
 *     under the without-replacement rule, repeats allowed with replacement
 *     for T > 0 requests only. A greedy (T == 0) request needs distinct
 *     siblings under either rule: siblings that repeat the argmax token are
 *     all flagged, and tree_accept_path then reports TV_DEV_PATH.
 *   node_indptr [B+1], parent [T] int32; temperature [B] fp32 >= 0;
 *   uniforms [T][2] fp32 in [0,1).
 *   accept_flag [T] int8, next_token [T] int32: outputs.
 * Every single decision value (p(x), q(x), ratios, normalisers) is formed in
 * fp64; the vocabulary sums add fp32 exps (each from an fp64 argument, about
 * 1.5e-7 relative) in fp64. Decisions therefore match an fp64 reference
 * except within ~1e-6 of a threshold: an acceptance ratio, or a boundary of
 * the final draw's cumulative sum (in units of u).
 * Each request is walked by a team of workgroups that wait on one another
 * through the workspace; a launch never holds more workgroups than the
 * device keeps resident at once, so with no other kernels running alongside
 * every team is resident together. Members held back longer than the wait
 * limit (0.2 s) by concurrent work make the call set TV_DEV_TIMEOUT (outputs
 * then unspecified) instead of hanging. The environment variable
 * TREEVERIFY_TEAM_WAIT_US (microseconds), read at every launch, sets another
 * limit for this call and tree_spark_build. */
tv_status tree_spec_sample(const tv_sample_desc* desc,
                           const float* target_logits, const float* draft_logits,
                           const int32_t* tokens, const int32_t* node_indptr,
                           const int32_t* parent, const float* temperature,
                           const float* uniforms, int8_t* accept_flag,
                           int32_t* next_token,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* tree_spec_sample for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same computation, arguments and outputs as tree_spec_sample,
 * without the workspace: the walk's per-request exchange blocks (2304 bytes
 * each) live in a device array the library owns, sized for
 * TV_SAMPLE_STATIC_MAX_BATCH requests (2.25 MiB, one copy per GPU, held until
 * the process ends). Every call first clears the blocks it uses and *status
 * with a fill kernel; nothing is allocated and nothing is synchronised.
 *   status: caller-owned device word (4-byte aligned) that receives the
 *     TV_DEV_* bits of this call. It can be read with tv_device_status
 *     (passed as the workspace) and passed to tree_accept_path as its
 *     status_workspace.
 * desc->batch > TV_SAMPLE_STATIC_MAX_BATCH returns TV_ERR_SHAPE before any
 * launch. Every call on one GPU uses that GPU's one array: calls that
 * overlap on one GPU (several streams, or several host threads) race and
 * their results are undefined; order them on one stream. */
#define TV_SAMPLE_STATIC_MAX_BATCH 1024
tv_status tree_spec_sample_noalloc(const tv_sample_desc* desc,
                                   const float* target_logits, const float* draft_logits,
                                   const int32_t* tokens, const int32_t* node_indptr,
                                   const int32_t* parent, const float* temperature,
                                   const float* uniforms, int8_t* accept_flag,
                                   int32_t* next_token, uint32_t* status, hipStream_t stream);

/* Longest accepted path ([TreeSpark] §3.2 step 3: commit the longest
 * surviving root path plus one correction/bonus token; §5.1: tau = accepted
 * length + 1; [explainer] exactly one path is accepted; [survey] Systems:
 * the accepted slots feed KV compaction).
 * Per request: follow accept_flag from the root through the unique flagged
 * child. Outputs, each [B][max_depth+1] int32 padded with -1:
 *   path_nodes: request-local rows of the path, root first
 *   out_tokens: tokens of the path's non-root nodes, then next_token[stop]
 *   kv_keep:    logical KV positions prefix_len[r] + node of the path rows
 * and out_len [B] = path length (accepted drafts + 1). A node with two
 * flagged children, or a path longer than max_depth + 1, sets
 * out_len[r] = -1 (that request's three rows are then unspecified) and, if
 * status_workspace is not NULL, TV_DEV_PATH in its status word. */
tv_status tree_accept_path(int32_t batch, int32_t max_depth,
                           const int32_t* node_indptr, const int32_t* parent,
                           const int32_t* tokens, const int8_t* accept_flag,
                           const int32_t* next_token, const int32_t* prefix_len,
                           int32_t* path_nodes, int32_t* out_tokens,
                           int32_t* out_len, int32_t* kv_keep,
                           void* status_workspace, hipStream_t stream);

/* Commit of the accepted path's K/V ([survey] Systems, KV handling: the
 * reference EAGLE implementation compacts the accepted slots in place with
 * gathers over the accepted positions; [survey] Timeline: tree tokens sit in
 * the KV cache in topological order). For every request r with
 * n = out_len[r] >= 1, in every layer and kv head, logical position
 * prefix_len[r] + j takes the K and V of logical position kv_keep[r][j],
 * j = 0 .. n-1 (the layouts tree_accept_path writes; within a request every
 * source is read before its destination is written). Logical positions map
 * to pages as for tree_verify_attn; positions from prefix_len[r] + n on keep
 * whatever they held.
 *   desc: batch, num_kv_heads, head_dim (64|128), num_pages, max_nodes and
 *     dtype as for tree_verify_attn (other fields unused).
 *   k_pages, v_pages: num_layers page pools, layer l at element offset
 *     l * layer_stride (>= num_pages*Hkv*16*D; pools and layer starts 16-byte
 *     aligned); K pages [num_pages][Hkv][16][D], V pages [num_pages][Hkv][D][16].
 *     Modified in place.
 *   kv_keep [B][max_depth+1], out_len [B]: as written by tree_accept_path.
 *     Requests with out_len < 1 are left untouched.
 * The pages holding positions prefix_len[r] .. prefix_len[r]+n-1 must belong
 * to request r alone. A keep-list that does not start at prefix_len[r], is
 * not strictly increasing, has an entry below prefix_len[r] + j or at or past
 * prefix_len[r] + max_nodes, or reaches past the listed pages sets
 * TV_DEV_PATH (a page id outside the pool: TV_DEV_PAGES; out_len[r] >
 * max_depth + 1: TV_DEV_SHAPE) in status_workspace (if not NULL), and the
 * request is left untouched. */
tv_status tree_kv_commit(const tv_attn_desc* desc, int32_t num_layers, int64_t layer_stride,
                         void* k_pages, void* v_pages, const int32_t* page_indptr,
                         const int32_t* page_indices, const int32_t* prefix_len,
                         const int32_t* kv_keep, const int32_t* out_len, int32_t max_depth,
                         void* status_workspace, hipStream_t stream);

/* Children of each expanded node, drawn without replacement ([survey]
 * Timeline: Recursive Speculative Decoding draws tree siblings without
 * replacement via Gumbel-Top-k; [TreeSpark] §1, §3.3: siblings are drawn
 * without replacement from q_T, in a draw order the verifier replays).
 * For row r with k = counts[r] children (0..TV_MAX_CHILDREN) and temperature
 * T = temperature[r] >= 0: tokens[r][0..k-1] = the k tokens of largest
 * score, in descending score, lower token id first on ties, where
 * score(y) = d[y]/T - ln(-ln u(y)) at T > 0 and d[y] at T = 0; the rest of
 * tokens[r] is -1. u(y) = ((w >> 8) + 1/2) / 2^24 with w the (y % 4)-th word
 * of Philox4x32-10 (Salmon et al., SC 2011) at counter (y/4, r, stream_id, 0)
 * and key (seed mod 2^32, seed >> 32).
 *   draft_logits [rows][vocab] fp32 (rows 16-byte aligned when vocab % 4 == 0
 *     for the vector path); counts [rows] int32; temperature [rows] fp32;
 *   tokens [rows][TV_MAX_CHILDREN] int32 output.
 * The noise is computed in fp32 (the exact -ln u via log1p near u = 1), so
 * draws match an fp64 evaluation except where two scores lie within ~1e-5.
 * counts outside [0, TV_MAX_CHILDREN] set TV_DEV_SHAPE, a negative or
 * non-finite temperature or non-finite logits TV_DEV_LOGITS in
 * status_workspace (if not NULL); such a row's tokens are all -1. */
#define TV_MAX_CHILDREN 16
tv_status tree_draw_siblings(int32_t rows, int32_t vocab, const float* draft_logits,
                             const int32_t* counts, const float* temperature, uint32_t stream_id,
                             uint64_t seed, int32_t* tokens, void* status_workspace,
                             hipStream_t stream);

/* Draft-tree construction by expansion and rerank ([survey] Timeline:
 * EAGLE-2 expands the top-k nodes by path-product value and reranks to keep
 * the top-m; [survey] Taxonomy: the value is the cumulative draft probability
 * along the root path). Values are logs: value(node) = sum over its root
 * path of log softmax(draft row of the edge's parent)[token].
 *
 * Candidates are kept per request in caller-owned arrays of cand_capacity
 * entries, numbered in generation order. One expansion round:
 * tree_expand_step takes the k_in frontier nodes of every request (their
 * candidate ids; NULL frontier = every slot is the root, value 0) and their
 * draft logit rows, gives each node its k children = the k largest logits,
 * descending, lower token id first on ties, stores child (slot s, rank j) at
 * id cand_offset + s*k + j with value = value(frontier) + log q(token), and
 * writes the k best of the round's k_in*k new ids (value descending, lower
 * id on ties) to next_frontier, best first.
 *   draft_logits [batch][k_in][vocab] fp32 (the drafter's rows for the
 *     frontier slots, in slot order); frontier [batch][k_in] int32 or NULL;
 *   cand_value [batch][cand_capacity] fp32, cand_token and cand_parent
 *     [batch][cand_capacity] int32 (parent = candidate id, -1 = root): read
 *     below cand_offset, written at cand_offset .. cand_offset + k_in*k - 1;
 *   next_frontier [batch][k] int32 output.
 * 1 <= k, k_in <= 16, vocab >= k, cand_offset + k_in*k <= cand_capacity,
 * else TV_ERR_SHAPE. workspace: NULL, or 256-byte aligned (else
 * TV_ERR_WORKSPACE) with its status word at byte 0; when workspace_bytes >=
 * tv_expand_workspace_size(batch, k_in, k), a round of fewer than 512 rows
 * splits each row over several workgroups (partial results in the
 * workspace), which fills the chip in the root round; the split changes
 * only the summation order of the log-sum-exp. A frontier id outside [-1, cand_offset) sets
 * TV_DEV_TREE (the slot is expanded as the root); non-finite logits set
 * TV_DEV_LOGITS (in the workspace's status word, if any). The log-sum-exp is
 * formed in fp32 and combined in fp64, so values agree with an fp64
 * evaluation to ~1e-6; selections can differ only where two values lie that
 * close. Calls that share a workspace must not overlap. */
tv_status tree_expand_step(int32_t batch, int32_t vocab, int32_t k_in, int32_t k,
                           const float* draft_logits, const int32_t* frontier,
                           int32_t cand_capacity, int32_t cand_offset, float* cand_value,
                           int32_t* cand_token, int32_t* cand_parent, int32_t* next_frontier,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace with which tree_expand_step splits rounds of few rows
 * (0 if the sizes are invalid). */
size_t tv_expand_workspace_size(int32_t batch, int32_t k_in, int32_t k);

/* Rerank: keep the m best of candidates 0 .. num_cand-1 of every request
 * (value descending, lower id on ties; a child's value never exceeds its
 * parent's and its id is larger, so the kept set is closed under ancestors)
 * and emit the tree: out_parent / out_token [batch][m+1] int32 hold the root
 * (parent -1, token -1: the caller's last accepted token) at 0, then the
 * kept candidates in ascending id (topological order, siblings in draw
 * order) with request-local parents; -1 past out_count[b] = 1 + kept.
 * 1 <= num_cand <= min(cand_capacity, 4096), m >= 1, else TV_ERR_SHAPE. A kept
 * candidate whose parent is not kept (values not from tree_expand_step) sets
 * TV_DEV_TREE and is attached to the root. */
tv_status tree_rerank(int32_t batch, int32_t num_cand, int32_t cand_capacity, int32_t m,
                      const float* cand_value, const int32_t* cand_token,
                      const int32_t* cand_parent, int32_t* out_parent, int32_t* out_token,
                      int32_t* out_count, void* status_workspace, hipStream_t stream);

/* TreeSpark's best-first draft-tree construction with the calibrated theta
 * stop ([TreeSpark] §3.1-§3.5). The drafter's backbone gives each request
 * base logits U_1..U_b (one row per depth) and a shared rank-r Markov head
 * B(x, v) = <w1[x], w2[v]>; a node at depth d carrying token x has children
 * from q0 = softmax(U_{d+1} + B(x, .)) (§3.2 step 1). Slots (a node's next
 * child) are keyed by calibrated path survival, the sum of
 * log p_hat(q0) = log sigma(a logit(q0) + b) along the root path (§1, §3.4):
 * the most probable unused token at T == 0; at T > 0 the slot is keyed by
 * the admissible pre-draw bound S(v) p_hat(max unused q0) and its token is
 * the node's next draw without replacement from q_T = softmax(l / T)
 * (Gumbel-top-k with the Philox4x32-10 noise of tree_draw_siblings, counter
 * (y/4, request * (max_nodes+1) + node, stream_id, 0), key seed). The best
 * slot is materialised first (ties: the lower node index); a node opens its
 * first-child slot (below depth b) and its parent's next-sibling slot (up to
 * max_siblings children); expansion stops when the best key falls below
 * log theta[r] (theta 0: never) or the tree holds max_nodes drafted nodes
 * (§3.5). The result equals one-slot-at-a-time best-first expansion.
 *   base_logits [B][depths][V] fp32; w1, w2 [V][rank] bf16 (row-major);
 *   anchor [B] int32 (the root's token); temperature, theta [B] fp32.
 *   out_parent, out_token [B][max_nodes+1] int32: the root (parent -1,
 *     token -1) then the nodes in materialisation order (topological,
 *     siblings in draw order), -1 past out_count[b] = 1 + drafted nodes;
 *     out_logsurv [B][max_nodes+1] fp32 log path survival (may be NULL).
 *   workspace: tv_spark_workspace_size bytes, 256-byte aligned, zero-filled
 *     once (tv_workspace_init); it holds the status word and the state kept
 *     between calls; calls that share it must not overlap. After a call,
 *     its uint32 words 2 and 3 hold the rounds run and the rows expanded
 *     (each round reads w2 once and the base-logit row of every expansion).
 * Logits are formed by bf16 matrix products with fp32 accumulation, the
 * log-sum-exp in fp32 combined in fp64, the calibration in fp64: decisions
 * agree with an fp64 evaluation except where two keys, two logits or two
 * draw scores lie within ~1e-5. Non-finite logits set TV_DEV_LOGITS, an
 * anchor outside [0, V) TV_DEV_SHAPE. The call is one launch of as many
 * workgroups as the device keeps resident at once, which meet at grid
 * barriers: with no other kernels running alongside all of them are
 * resident together; workgroups held back longer than the wait limit
 * (0.2 s; TREEVERIFY_TEAM_WAIT_US, as for tree_spec_sample) by concurrent
 * work make the call set TV_DEV_TIMEOUT (outputs then unspecified;
 * re-initialise the workspace) instead of hanging. */
typedef struct {
  int32_t batch;         /* B, 1..256 */
  int32_t vocab;         /* V: max_siblings + 1 .. 4194304 */
  int32_t rank;          /* r: a multiple of 32, at most 256 */
  int32_t depths;        /* b: base-logit rows per request, 1..16 */
  int32_t max_nodes;     /* N: drafted nodes per tree, 1..64 */
  int32_t max_siblings;  /* K: children per node, 1..16 */
  float calib_a;         /* p_hat = sigma(calib_a logit(q0) + calib_b); */
  float calib_b;         /* the pages' fit: 0.67, -0.46 */
} tv_spark_desc;

size_t tv_spark_workspace_size(const tv_spark_desc* desc);

tv_status tree_spark_build(const tv_spark_desc* desc, const float* base_logits,
                           const void* w1, const void* w2, const int32_t* anchor,
                           const float* temperature, const float* theta,
                           uint32_t stream_id, uint64_t seed, int32_t* out_parent,
                           int32_t* out_token, int32_t* out_count, float* out_logsurv,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Tree metadata ([TreeSpark] §3.2 step 3 and §4: per-depth position ids and
 * ancestor bitmasks). For every row: depth (edges from the root),
 * anc_bits [T][ceil(max_nodes/32)] (bit j of word j/32 set iff j is an
 * ancestor of the row or the row itself), and children in draw order as
 * first_child / next_sibling (request-local, -1 = none). Any output may be
 * NULL. Bad parents set TV_DEV_TREE in status_workspace (if not NULL). */
tv_status tv_tree_meta(int32_t batch, int32_t max_nodes,
                       const int32_t* node_indptr, const int32_t* parent,
                       int32_t* depth, uint32_t* anc_bits,
                       int32_t* first_child, int32_t* next_sibling,
                       void* status_workspace, hipStream_t stream);

/* ---- host-side validators (host arrays; no GPU needed) ---------------- */

/* TV_ERR_TREE unless every request's parent array is topological, has a
 * single root at row 0, N_r <= max_nodes and depth <= max_depth. */
tv_status tv_validate_tree(int32_t batch, const int32_t* node_indptr_host,
                           const int32_t* parent_host, int32_t max_nodes,
                           int32_t max_depth);

/* TV_ERR_PAGES unless each request's listed pages cover P_r + N_r tokens and
 * every page id is in [0, num_pages). */
tv_status tv_validate_pages(int32_t batch, const int32_t* page_indptr_host,
                            const int32_t* page_indices_host,
                            const int32_t* prefix_len_host,
                            const int32_t* node_indptr_host, int32_t num_pages,
                            int32_t page_size);

const char* tv_status_string(tv_status status);
/* Message of the last failed HIP call on this thread ("" if none). */
const char* tv_last_hip_error(void);
int32_t tv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TREE_VERIFY_H */
