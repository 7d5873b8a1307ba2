// Host-side argument checks of libtreeverify under AddressSanitizer: every
// entry point's rejections (before any launch) and the host validators, on
// arrays sized exactly, so a read past an argument shows up. Built and run
// by tests/test_host_asan.py; needs no GPU (no call here reaches a launch).
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "tree_verify.h"

static int failures = 0;
#define EXPECT(cond)                                                \
  do {                                                              \
    if (!(cond)) {                                                  \
      std::printf("FAIL line %d: %s\n", __LINE__, #cond);           \
      ++failures;                                                   \
    }                                                               \
  } while (0)

int main() {
  // status strings, including an unknown code
  for (int s = 0; s <= 11; ++s) EXPECT(tv_status_string(tv_status(s)) != nullptr);

  // workspace sizes: valid, degenerate and overflowing descriptors
  tv_attn_desc ad{4, 32, 8, 128, 16, 32, 8, 8192, 4096, TV_BF16, 0.f};
  EXPECT(tv_attn_workspace_size(&ad) > 0);
  tv_attn_desc bad = ad;
  bad.num_q_heads = 30;  // not a multiple of the kv heads
  EXPECT(tv_attn_workspace_size(&bad) == 0);
  bad = ad;
  bad.head_dim = 96;
  EXPECT(tv_attn_workspace_size(&bad) == 0);
  bad = ad;
  bad.max_kv_len = 0x7fffffff;
  bad.batch = 4000;
  (void)tv_attn_workspace_size(&bad);  // must not overflow silently or crash
  EXPECT(tv_attn_workspace_size(nullptr) == 0);
  tv_sample_desc sd{64, 151936, 32, 8, TV_RULE_WITHOUT_REPLACEMENT};
  EXPECT(tv_sample_workspace_size(&sd) > 0);
  tv_sample_desc sbad = sd;
  sbad.rule = tv_rule(7);
  EXPECT(tv_sample_workspace_size(&sbad) == 0);
  sbad = sd;
  sbad.greedy = 2;
  EXPECT(tv_sample_workspace_size(&sbad) == 0);
  sbad.greedy = TV_GREEDY_PATH;
  EXPECT(tv_sample_workspace_size(&sbad) == tv_sample_workspace_size(&sd));
  sbad = sd;
  sbad.vocab = 0;
  EXPECT(tv_sample_workspace_size(&sbad) == 0);
  EXPECT(tv_expand_workspace_size(0, 4, 4) == 0);
  EXPECT(tv_expand_workspace_size(8, 4, 4) > 0);

  // entry points: NULL descriptors and pointers, bad shapes, small or
  // misaligned workspaces, all rejected before anything is launched
  alignas(256) static unsigned char ws[1024];
  void* fake = reinterpret_cast<void*>(uintptr_t(0x10000));
  const int32_t* fi = static_cast<const int32_t*>(fake);
  const float* ff = static_cast<const float*>(fake);
  EXPECT(tree_verify_attn(nullptr, fake, fake, fake, fi, fi, fi, fi, fi, fake, ws, sizeof ws, nullptr) ==
         TV_ERR_NULL);
  EXPECT(tree_verify_attn(&bad, fake, fake, fake, fi, fi, fi, fi, fi, fake, ws, sizeof ws, nullptr) ==
         TV_ERR_SHAPE);
  EXPECT(tree_verify_attn(&ad, nullptr, fake, fake, fi, fi, fi, fi, fi, fake, ws, sizeof ws, nullptr) ==
         TV_ERR_NULL);
  EXPECT(tree_verify_attn(&ad, fake, fake, fake, fi, fi, fi, fi, fi, fake, ws, sizeof ws, nullptr) ==
         TV_ERR_WORKSPACE);
  EXPECT(tree_verify_attn(&ad, fake, fake, fake, fi, fi, fi, fi, fi, fake, ws + 1, size_t(1) << 40,
                          nullptr) == TV_ERR_WORKSPACE);
  int8_t* fb = static_cast<int8_t*>(fake);
  int32_t* fo = static_cast<int32_t*>(fake);
  EXPECT(tree_spec_sample(nullptr, ff, ff, fi, fi, fi, ff, ff, fb, fo, ws, sizeof ws, nullptr) == TV_ERR_NULL);
  EXPECT(tree_spec_sample(&sbad, ff, ff, fi, fi, fi, ff, ff, fb, fo, ws, sizeof ws, nullptr) == TV_ERR_SHAPE);
  EXPECT(tree_spec_sample(&sd, ff, ff, fi, fi, fi, ff, ff, fb, fo, ws, sizeof ws, nullptr) == TV_ERR_WORKSPACE);
  EXPECT(tree_spec_sample(&sd, ff, ff, nullptr, fi, fi, ff, ff, fb, fo, ws, sizeof ws, nullptr) == TV_ERR_NULL);
  tv_sample_desc big = sd;
  big.batch = TV_SAMPLE_STATIC_MAX_BATCH + 1;
  EXPECT(tree_spec_sample_noalloc(&big, ff, ff, fi, fi, fi, ff, ff, fb, fo, reinterpret_cast<uint32_t*>(ws),
                                  nullptr) == TV_ERR_SHAPE);
  EXPECT(tree_spec_sample_noalloc(&sd, ff, ff, fi, fi, fi, ff, ff, fb, fo,
                                  reinterpret_cast<uint32_t*>(ws + 2), nullptr) == TV_ERR_WORKSPACE);
  EXPECT(tree_accept_path(0, 8, fi, fi, fi, fb, fi, fi, fo, fo, fo, fo, nullptr, nullptr) == TV_ERR_SHAPE);
  EXPECT(tree_accept_path(4, 70000, fi, fi, fi, fb, fi, fi, fo, fo, fo, fo, nullptr, nullptr) == TV_ERR_SHAPE);
  EXPECT(tree_accept_path(4, 8, nullptr, fi, fi, fb, fi, fi, fo, fo, fo, fo, nullptr, nullptr) == TV_ERR_NULL);
  EXPECT(tree_kv_commit(&ad, 0, 1, fake, fake, fi, fi, fi, fi, fi, 8, nullptr, nullptr) == TV_ERR_SHAPE);
  EXPECT(tree_kv_commit(&ad, 2, 16, fake, fake, fi, fi, fi, fi, fi, 8, nullptr, nullptr) == TV_ERR_SHAPE);
  EXPECT(tree_draw_siblings(0, 100, ff, fi, ff, 0, 0, fo, nullptr, nullptr) == TV_ERR_SHAPE);
  EXPECT(tree_draw_siblings(4, 100, nullptr, fi, ff, 0, 0, fo, nullptr, nullptr) == TV_ERR_NULL);
  float* fv = static_cast<float*>(fake);
  EXPECT(tree_expand_step(1, 100, 4, 8, ff, fi, 16, 0, fv, fo, fo, fo, nullptr, 0, nullptr) == TV_ERR_SHAPE);
  EXPECT(tree_rerank(1, 0, 16, 4, ff, fi, fi, fo, fo, fo, nullptr, nullptr) == TV_ERR_SHAPE);
  EXPECT(tv_tree_meta(1, 0, fi, fi, fo, reinterpret_cast<uint32_t*>(fake), fo, fo, nullptr, nullptr) ==
         TV_ERR_SHAPE);
  tv_spark_desc kd{};
  kd.batch = 4;
  kd.vocab = 1000;
  kd.rank = 64;
  kd.depths = 3;
  kd.max_nodes = 16;
  kd.max_siblings = 4;
  kd.calib_a = 0.67f;
  kd.calib_b = -0.46f;
  EXPECT(tv_spark_workspace_size(&kd) > 0);
  tv_spark_desc kbad = kd;
  kbad.rank = 48;
  EXPECT(tv_spark_workspace_size(&kbad) == 0);
  tv_spark_desc kbig = kd;
  kbig.vocab = (1 << 22) + 1;  // past the vocabulary limit (w2 under 4 GB)
  EXPECT(tv_spark_workspace_size(&kbig) == 0);
  kbig.vocab = 1 << 22;
  EXPECT(tv_spark_workspace_size(&kbig) > 0);
  EXPECT(tree_spark_build(&kbad, ff, fake, fake, fi, ff, ff, 0, 0, fo, fo, fo, fv, ws, sizeof ws, nullptr) ==
         TV_ERR_SHAPE);
  EXPECT(tree_spark_build(&kd, ff, fake, fake, fi, ff, ff, 0, 0, fo, fo, fo, fv, ws, sizeof ws, nullptr) ==
         TV_ERR_WORKSPACE);

  // host validators on exactly sized arrays
  {
    std::vector<int32_t> ip{0, 5, 5, 8};                  // a 5-row tree, an empty request, a chain
    std::vector<int32_t> par{-1, 0, 0, 1, 1, -1, 0, 1};
    EXPECT(tv_validate_tree(3, ip.data(), par.data(), 8, 8) == TV_OK);
    EXPECT(tv_validate_tree(3, ip.data(), par.data(), 4, 8) == TV_ERR_TREE);   // a tree past max_nodes
    EXPECT(tv_validate_tree(3, ip.data(), par.data(), 8, 1) == TV_ERR_TREE);   // too deep
    std::vector<int32_t> bad_par{-1, 0, 3, 1, 1, -1, 0, 1};                  // parent after the child
    EXPECT(tv_validate_tree(3, ip.data(), bad_par.data(), 8, 8) == TV_ERR_TREE);
    std::vector<int32_t> bad_root{0, 0, 0, 1, 1, -1, 0, 1};
    EXPECT(tv_validate_tree(3, ip.data(), bad_root.data(), 8, 8) == TV_ERR_TREE);
    std::vector<int32_t> dec{0, 5, 4, 8};
    EXPECT(tv_validate_tree(3, dec.data(), par.data(), 8, 8) == TV_ERR_SHAPE);
    EXPECT(tv_validate_tree(3, nullptr, par.data(), 8, 8) == TV_ERR_NULL);
    // pages: request r needs ceil((P_r + N_r) / 16) pages
    std::vector<int32_t> pip{0, 2, 3, 4};
    std::vector<int32_t> pidx{7, 1, 3, 0};
    std::vector<int32_t> pre{20, 4, 3};
    EXPECT(tv_validate_pages(3, pip.data(), pidx.data(), pre.data(), ip.data(), 8, 16) == TV_OK);
    std::vector<int32_t> pre_long{28, 4, 3};   // 28 + 5 = 33 > 32
    EXPECT(tv_validate_pages(3, pip.data(), pidx.data(), pre_long.data(), ip.data(), 8, 16) == TV_ERR_PAGES);
    std::vector<int32_t> pidx_bad{7, 1, 8, 0};  // page 8 of a pool of 8
    EXPECT(tv_validate_pages(3, pip.data(), pidx_bad.data(), pre.data(), ip.data(), 8, 16) == TV_ERR_PAGES);
    EXPECT(tv_validate_pages(3, pip.data(), pidx.data(), pre.data(), ip.data(), 8, 32) == TV_ERR_SHAPE);
  }
  std::printf("%s (%d failures)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
