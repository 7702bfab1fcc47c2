// Host-side argument validation of the C ABI (include/spec_verify.h), built
// with AddressSanitizer and UndefinedBehaviorSanitizer on the host code.
// Every call here is rejected by validation, or is an empty problem, so no
// kernel is launched and no GPU is needed; the sanitizers watch the
// validation arithmetic (size products near 2^31, alignment checks, pointer
// tests) and the workspace planners.  Prints "all checks passed" and exits 0
// when every status matches.
#include <stdint.h>
#include <stdio.h>

#include "spec_verify.h"

static int failures = 0;
static void expect(const char* what, int got, int want) {
  if (got != want) {
    printf("FAIL %s: status %d, expected %d\n", what, got, want);
    ++failures;
  }
}

int main() {
  void* const F = (void*)0x1000;        // never dereferenced
  float* const FF = (float*)F;
  int32_t* const FI = (int32_t*)F;
  const size_t BIG = (size_t)1 << 40;
  const char* s = spec_status_string((spec_status)99);
  if (!s) { printf("FAIL status string\n"); ++failures; }
  if (!spec_status_string((spec_status)-7)) { printf("FAIL status string\n"); ++failures; }
  expect("attn dtype", spec_verify_attention(F, F, F, nullptr, (float*)F, 2, 5, 8, 2, 128, 100,
                                            (spec_dtype)7, 0.1f, F, (size_t)1 << 40, nullptr),
         SPEC_ERR_UNSUPPORTED);
  expect("commit dtype", spec_commit_kv(F, F, (int32_t*)F, (int32_t*)F, (int32_t*)F, 2, 9, 8,
                                        128, 100, (spec_dtype)-3, nullptr),
         SPEC_ERR_UNSUPPORTED);
  for (int i = 0; i < 6; ++i)
    if (!spec_status_string((spec_status)i)) { printf("FAIL status %d\n", i); ++failures; }

  // verify attention
  expect("attn q null", spec_verify_attention(nullptr, F, F, nullptr, FF, 2, 5, 8, 2, 128, 100,
                                             SPEC_BF16, 0.1f, F, BIG, nullptr), SPEC_ERR_NULL);
  expect("attn Hq%Hkv", spec_verify_attention(F, F, F, nullptr, FF, 2, 5, 7, 2, 128, 100,
                                             SPEC_BF16, 0.1f, F, BIG, nullptr), SPEC_ERR_SHAPE);
  expect("attn T>64", spec_verify_attention(F, F, F, nullptr, FF, 2, 65, 8, 2, 128, 100,
                                           SPEC_BF16, 0.1f, F, BIG, nullptr), SPEC_ERR_UNSUPPORTED);
  expect("attn D", spec_verify_attention(F, F, F, nullptr, FF, 2, 5, 8, 2, 96, 100, SPEC_BF16,
                                        0.1f, F, BIG, nullptr), SPEC_ERR_UNSUPPORTED);
  expect("attn B*Hkv", spec_verify_attention(F, F, F, nullptr, FF, 1 << 30, 5, 8, 2, 128, 100,
                                            SPEC_BF16, 0.1f, F, BIG, nullptr), SPEC_ERR_UNSUPPORTED);
  expect("attn ctx+T int32", spec_verify_attention(F, F, F, nullptr, FF, 2, 5, 8, 2, 128,
                                                  0x7ffffffe, SPEC_BF16, 0.1f, F, BIG, nullptr),
         SPEC_ERR_UNSUPPORTED);
  expect("attn (ctx+T)D", spec_verify_attention(F, F, F, nullptr, FF, 2, 5, 8, 2, 128,
                                               (1 << 24) - 5, SPEC_BF16, 0.1f, F, BIG, nullptr),
         SPEC_ERR_UNSUPPORTED);
  expect("attn scale nan", spec_verify_attention(F, F, F, nullptr, FF, 2, 5, 8, 2, 128, 100,
                                                SPEC_BF16, 0.0f / 0.0f, F, BIG, nullptr),
         SPEC_ERR_SHAPE);
  expect("attn align", spec_verify_attention((char*)F + 4, F, F, nullptr, FF, 2, 5, 8, 2, 128,
                                            100, SPEC_BF16, 0.1f, F, BIG, nullptr),
         SPEC_ERR_UNSUPPORTED);
  expect("attn workspace", spec_verify_attention(F, F, F, nullptr, FF, 2, 5, 8, 2, 128, 100,
                                                SPEC_BF16, 0.1f, F, 16, nullptr),
         SPEC_ERR_WORKSPACE);
  expect("attn empty", spec_verify_attention(nullptr, nullptr, nullptr, nullptr, nullptr, 0, 5,
                                            8, 2, 128, 100, SPEC_BF16, 0.1f, nullptr, 0, nullptr),
         SPEC_OK);
  if (spec_verify_attention_workspace(64, 9, 32, 8, 128, 32768, SPEC_BF16) != 0 &&
      spec_verify_attention_workspace(8, 64, 32, 8, 128, 8192, SPEC_BF16) == 0) {
    printf("FAIL attention workspace sizes\n");
    ++failures;
  }
  expect("attn ws query bad", (int)spec_verify_attention_workspace(2, 65, 8, 2, 128, 10,
                                                                   SPEC_BF16), 0);
  // paged
  expect("paged page size", spec_verify_attention_paged(F, F, F, FI, nullptr, nullptr, FF, 2, 5,
                                                        8, 2, 128, 100, 3, 64, 64,
                                                        SPEC_PAGES_HND, SPEC_BF16, 0.1f, F, BIG,
                                                        nullptr), SPEC_ERR_UNSUPPORTED);
  expect("paged table short", spec_verify_attention_paged(F, F, F, FI, nullptr, nullptr, FF, 2,
                                                          5, 8, 2, 128, 100, 16, 64, 2,
                                                          SPEC_PAGES_HND, SPEC_BF16, 0.1f, F,
                                                          BIG, nullptr), SPEC_ERR_SHAPE);
  expect("paged layout", spec_verify_attention_paged(F, F, F, FI, nullptr, nullptr, FF, 2, 5, 8,
                                                     2, 128, 100, 16, 64, 64,
                                                     (spec_page_layout)7, SPEC_BF16, 0.1f, F,
                                                     BIG, nullptr), SPEC_ERR_UNSUPPORTED);
  // chain
  expect("chain null", spec_accept_chain(nullptr, FF, FI, FF, FF, 1.f, FI, FI, 4, 3, 1000, F, BIG,
                                         nullptr), SPEC_ERR_NULL);
  expect("chain tau", spec_accept_chain(FF, FF, FI, FF, FF, 0.f, FI, FI, 4, 3, 1000, F, BIG,
                                        nullptr), SPEC_ERR_SHAPE);
  expect("chain N", spec_accept_chain(FF, FF, FI, FF, FF, 1.f, FI, FI, 4, 64, 1000, F, BIG,
                                      nullptr), SPEC_ERR_UNSUPPORTED);
  expect("chain rows", spec_accept_chain(FF, FF, FI, FF, FF, 1.f, FI, FI, 1 << 29, 3, 1000, F,
                                         BIG, nullptr), SPEC_ERR_UNSUPPORTED);
  expect("chain V", spec_accept_chain(FF, FF, FI, FF, FF, 1.f, FI, FI, 4, 3, (1 << 24) + 1, F,
                                      BIG, nullptr), SPEC_ERR_UNSUPPORTED);
  expect("chain ws", spec_accept_chain(FF, FF, FI, FF, FF, 1.f, FI, FI, 4, 3, 1000, F, 8,
                                       nullptr), SPEC_ERR_WORKSPACE);
  expect("noalloc big", spec_accept_chain_noalloc(FF, FF, FI, FF, FF, 1.f, FI, FI, 4096, 8,
                                                  152064, nullptr), SPEC_ERR_WORKSPACE);
  expect("noalloc null", spec_accept_chain_noalloc(FF, nullptr, FI, FF, FF, 1.f, FI, FI, 4, 3,
                                                   1000, nullptr), SPEC_ERR_NULL);
  expect("noalloc empty", spec_accept_chain_noalloc(nullptr, nullptr, nullptr, nullptr, nullptr,
                                                    1.f, nullptr, nullptr, 0, 3, 1000, nullptr),
         SPEC_OK);
  // trees
  expect("tree T", spec_accept_tree(FF, FI, FI, FI, FI, FI, 2, 65, 500, F, BIG, nullptr),
         SPEC_ERR_UNSUPPORTED);
  expect("tree rows", spec_accept_tree(FF, FI, FI, FI, FI, FI, 1 << 26, 64, 500, F, BIG,
                                       nullptr), SPEC_ERR_UNSUPPORTED);
  expect("stree tau", spec_accept_tree_sampled(FF, FF, FI, FI, FF, FF, -1.f, FI, FI, FI, 4, 8,
                                               1000, F, BIG, nullptr), SPEC_ERR_SHAPE);
  expect("stree ws", spec_accept_tree_sampled(FF, FF, FI, FI, FF, FF, 1.f, FI, FI, FI, 4, 8, 1000,
                                              F, 8, nullptr), SPEC_ERR_WORKSPACE);
  // n-gram and commit
  expect("ngram n", spec_ngram_propose(FI, nullptr, FI, FI, 4, 1000, 8, 3, 2, F, BIG, nullptr),
         SPEC_ERR_SHAPE);
  expect("ngram nmax", spec_ngram_propose(FI, nullptr, FI, FI, 4, 1000, 8, 1, 17, F, BIG,
                                          nullptr), SPEC_ERR_UNSUPPORTED);
  expect("commit B*Hkv", spec_commit_kv(F, F, FI, FI, FI, 1 << 29, 9, 8, 128, 100, SPEC_BF16,
                                        nullptr), SPEC_ERR_UNSUPPORTED);
  expect("commit ctx", spec_commit_kv(F, F, FI, FI, FI, 2, 9, 8, 128, 0x7ffffffe, SPEC_BF16,
                                      nullptr), SPEC_ERR_UNSUPPORTED);
  expect("commit align", spec_commit_kv(F, (char*)F + 8, FI, FI, FI, 2, 9, 8, 128, 100,
                                        SPEC_BF16, nullptr), SPEC_ERR_UNSUPPORTED);
  if (failures) {
    printf("%d check(s) failed\n", failures);
    return 1;
  }
  printf("all checks passed\n");
  return 0;
}
