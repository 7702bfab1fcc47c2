// C ABI of the verify step: argument validation, launch plans and dispatch.
// Every check happens on the host before anything is enqueued.

#include "../../include/spec_verify.h"

#include <math.h>

#include "common.h"

namespace sv {
AttnPlan plan_attention(int B, int T, int Hq, int Hkv, int D, int ctx, int bf16);
hipError_t launch_attention(const AttnPlan& p, const void* q, const void* k, const void* v,
                            const int32_t* parents, float* out, int B, int T, int Hq, int Hkv,
                            int D, int ctx, int bf16, float scale, void* workspace,
                            hipStream_t st, const PagedKV* paged);
ChainPlan plan_chain(int B, int N, int V);
hipError_t launch_chain(const ChainPlan& p, const float* target, const float* draft,
                        const int32_t* tokens, const float* u_acc, const float* u_draw,
                        float temperature, int32_t* num_acc, int32_t* out, int B, int N, int V,
                        void* workspace, hipStream_t st);
hipError_t chain_scratch(hipStream_t st, void** ptr);
TreePlan plan_tree(int B, int T, int V);
hipError_t launch_tree(const TreePlan& p, const float* logits, const int32_t* tokens,
                       const int32_t* parents, int32_t* accept_len, int32_t* path,
                       int32_t* out, int B, int T, int V, void* workspace, hipStream_t st);
STreePlan plan_tree_sampled(int B, int T, int V);
hipError_t launch_tree_sampled(const STreePlan& p, const float* target, const float* draft,
                               const int32_t* tokens, const int32_t* parents,
                               const float* u_accept, const float* u_draw, float temperature,
                               int32_t* accept_len, int32_t* path, int32_t* out, int B, int T,
                               int V, void* workspace, hipStream_t st);
NgramPlan plan_ngram(int B, int L);
hipError_t launch_ngram(const NgramPlan& p, const int32_t* ctx, const int32_t* lens,
                        int32_t* num, int32_t* drafts, int B, int L, int N, int n_min,
                        int n_max, void* workspace, hipStream_t st);
hipError_t launch_commit(void* k, void* v, const int32_t* path, const int32_t* accept_len,
                         int32_t* new_len, int B, int T, int Hkv, int D, int ctx, int esize,
                         hipStream_t st);
}  // namespace sv

namespace {

spec_status check_attention(int B, int T, int Hq, int Hkv, int D, int ctx, spec_dtype dtype) {
  if (B < 0 || T < 0 || Hq < 1 || Hkv < 1 || D < 1 || ctx < 0) return SPEC_ERR_SHAPE;
  if (Hq % Hkv != 0) return SPEC_ERR_SHAPE;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ERR_UNSUPPORTED;
  if (T > SPEC_MAX_T || (D != 64 && D != 128)) return SPEC_ERR_UNSUPPORTED;
  // keep every element index of K/V below 2^31 per (sequence, KV head) unit
  if (((long long)ctx + T) * D >= (1ll << 31)) return SPEC_ERR_UNSUPPORTED;
  if ((long long)B * Hkv > SPEC_MAX_ROWS) return SPEC_ERR_UNSUPPORTED;   // int32 block ids
  return SPEC_OK;
}

spec_status check_chain(int B, int N, int V) {
  if (B < 0 || N < 0 || V < 1) return SPEC_ERR_SHAPE;
  if (V > SPEC_MAX_V || N > SPEC_MAX_T - 1) return SPEC_ERR_UNSUPPORTED;
  if ((long long)B * (2 * N + 1) > SPEC_MAX_ROWS) return SPEC_ERR_UNSUPPORTED;
  return SPEC_OK;
}

// Everything spec_accept_chain checks except the workspace.
spec_status check_chain_call(const float* target_logits, const float* draft_logits,
                             const int32_t* draft_tokens, const float* u_accept,
                             const float* u_draw, float temperature,
                             const int32_t* num_accepted, const int32_t* out_tokens, int B,
                             int N, int V) {
  const spec_status c = check_chain(B, N, V);
  if (c != SPEC_OK) return c;
  if (!(temperature > 0.f) || !isfinite(temperature)) return SPEC_ERR_SHAPE;
  if (B == 0) return SPEC_OK;
  if (!target_logits || !u_draw || !num_accepted || !out_tokens) return SPEC_ERR_NULL;
  if (N > 0 && (!draft_logits || !draft_tokens || !u_accept)) return SPEC_ERR_NULL;
  return SPEC_OK;
}

static_assert(sv::kChainScratchBytes == SPEC_CHAIN_NOALLOC_SCRATCH_BYTES,
              "the header states the scratch size");

spec_status check_ngram(int B, int L, int N, int n_min, int n_max) {
  if (B < 0 || L < 0 || N < 0 || n_min < 1 || n_max < n_min) return SPEC_ERR_SHAPE;
  if (N > SPEC_MAX_T - 1 || n_max > SPEC_NGRAM_MAX) return SPEC_ERR_UNSUPPORTED;
  return SPEC_OK;
}

spec_status check_tree(int B, int T, int V) {
  if (B < 0 || T < 0 || V < 1) return SPEC_ERR_SHAPE;
  if (V > SPEC_MAX_V || T > SPEC_MAX_T) return SPEC_ERR_UNSUPPORTED;
  if ((long long)B * T > SPEC_MAX_ROWS) return SPEC_ERR_UNSUPPORTED;
  return SPEC_OK;
}

}  // namespace

extern "C" {

const char* spec_status_string(spec_status s) {
  switch (s) {
    case SPEC_OK: return "ok";
    case SPEC_ERR_NULL: return "a required pointer is NULL";
    case SPEC_ERR_SHAPE: return "a size is negative or inconsistent";
    case SPEC_ERR_UNSUPPORTED: return "arguments are outside the supported limits";
    case SPEC_ERR_WORKSPACE: return "workspace is smaller than the queried size";
    case SPEC_ERR_HIP: return "the HIP runtime reported a launch error";
    default: break;
  }
  return "unknown status";
}

size_t spec_verify_attention_workspace(int B, int T, int Hq, int Hkv, int D, int ctx,
                                       spec_dtype dtype) {
  if (check_attention(B, T, Hq, Hkv, D, ctx, dtype) != SPEC_OK || B == 0 || T == 0) return 0;
  return sv::plan_attention(B, T, Hq, Hkv, D, ctx, dtype == SPEC_BF16).total_bytes;
}

spec_status spec_verify_attention(const void* q, const void* k, const void* v,
                                  const int32_t* parents, float* out, int B, int T, int Hq,
                                  int Hkv, int D, int ctx, spec_dtype dtype, float scale,
                                  void* workspace, size_t workspace_bytes, void* hip_stream) {
  const spec_status c = check_attention(B, T, Hq, Hkv, D, ctx, dtype);
  if (c != SPEC_OK) return c;
  if (!isfinite(scale) || !(scale > 0.f)) return SPEC_ERR_SHAPE;
  if (B == 0 || T == 0) return SPEC_OK;
  if (!q || !k || !v || !out || !workspace) return SPEC_ERR_NULL;
  // q, k, v and out are read and written 16 bytes per lane
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) % 16 != 0)
    return SPEC_ERR_UNSUPPORTED;
  const sv::AttnPlan p = sv::plan_attention(B, T, Hq, Hkv, D, ctx, dtype == SPEC_BF16);
  if (workspace_bytes < p.total_bytes) return SPEC_ERR_WORKSPACE;
  const hipError_t e = sv::launch_attention(p, q, k, v, parents, out, B, T, Hq, Hkv, D, ctx,
                                            dtype == SPEC_BF16, scale, workspace,
                                            (hipStream_t)hip_stream, nullptr);
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

size_t spec_verify_attention_paged_workspace(int B, int T, int Hq, int Hkv, int D, int max_ctx,
                                             spec_dtype dtype) {
  return spec_verify_attention_workspace(B, T, Hq, Hkv, D, max_ctx, dtype);
}

spec_status spec_verify_attention_paged(const void* q, const void* k_pages, const void* v_pages,
                                        const int32_t* block_table, const int32_t* ctx_lens,
                                        const int32_t* parents, float* out, int B, int T,
                                        int Hq, int Hkv, int D, int max_ctx, int page_size,
                                        int num_pages, int max_blocks, spec_page_layout layout,
                                        spec_dtype dtype, float scale, void* workspace,
                                        size_t workspace_bytes, void* hip_stream) {
  const spec_status c = check_attention(B, T, Hq, Hkv, D, max_ctx, dtype);
  if (c != SPEC_OK) return c;
  if (!isfinite(scale) || !(scale > 0.f)) return SPEC_ERR_SHAPE;
  if (page_size < 1 || num_pages < 1 || max_blocks < 1) return SPEC_ERR_SHAPE;
  if ((page_size & (page_size - 1)) != 0 || page_size > SPEC_MAX_PAGE_SIZE)
    return SPEC_ERR_UNSUPPORTED;
  if (layout != SPEC_PAGES_HND && layout != SPEC_PAGES_NHD) return SPEC_ERR_UNSUPPORTED;
  // the table must reach the longest sequence
  if ((long long)max_blocks * page_size < (long long)max_ctx + T) return SPEC_ERR_SHAPE;
  if (B == 0 || T == 0) return SPEC_OK;
  if (!q || !k_pages || !v_pages || !block_table || !out || !workspace) return SPEC_ERR_NULL;
  if (((uintptr_t)q | (uintptr_t)k_pages | (uintptr_t)v_pages | (uintptr_t)out) % 16 != 0)
    return SPEC_ERR_UNSUPPORTED;
  const sv::AttnPlan p = sv::plan_attention(B, T, Hq, Hkv, D, max_ctx, dtype == SPEC_BF16);
  if (workspace_bytes < p.total_bytes) return SPEC_ERR_WORKSPACE;
  sv::PagedKV pk;
  pk.block_table = block_table;
  pk.ctx_lens = ctx_lens;
  pk.page_size = page_size;
  pk.max_blocks = max_blocks;
  pk.num_pages = num_pages;
  pk.position_major = layout == SPEC_PAGES_NHD;
  const hipError_t e = sv::launch_attention(p, q, k_pages, v_pages, parents, out, B, T, Hq, Hkv,
                                            D, max_ctx, dtype == SPEC_BF16, scale, workspace,
                                            (hipStream_t)hip_stream, &pk);
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

size_t spec_accept_chain_workspace(int B, int N, int V) {
  if (check_chain(B, N, V) != SPEC_OK || B == 0) return 0;
  return sv::plan_chain(B, N, V).total_bytes;
}

spec_status spec_accept_chain(const float* target_logits, const float* draft_logits,
                              const int32_t* draft_tokens, const float* u_accept,
                              const float* u_draw, float temperature, int32_t* num_accepted,
                              int32_t* out_tokens, int B, int N, int V, void* workspace,
                              size_t workspace_bytes, void* hip_stream) {
  const spec_status c = check_chain_call(target_logits, draft_logits, draft_tokens, u_accept,
                                         u_draw, temperature, num_accepted, out_tokens, B, N, V);
  if (c != SPEC_OK || B == 0) return c;
  if (!workspace) return SPEC_ERR_NULL;
  const sv::ChainPlan p = sv::plan_chain(B, N, V);
  if (workspace_bytes < p.total_bytes) return SPEC_ERR_WORKSPACE;
  const hipError_t e = sv::launch_chain(p, target_logits, draft_logits, draft_tokens, u_accept,
                                        u_draw, temperature, num_accepted, out_tokens, B, N, V,
                                        workspace, (hipStream_t)hip_stream);
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

spec_status spec_accept_chain_noalloc(const float* target_logits, const float* draft_logits,
                                      const int32_t* draft_tokens, const float* u_accept,
                                      const float* u_draw, float temperature,
                                      int32_t* num_accepted, int32_t* out_tokens, int B, int N,
                                      int V, void* hip_stream) {
  const spec_status c = check_chain_call(target_logits, draft_logits, draft_tokens, u_accept,
                                         u_draw, temperature, num_accepted, out_tokens, B, N, V);
  if (c != SPEC_OK || B == 0) return c;
  const sv::ChainPlan p = sv::plan_chain(B, N, V);
  if (p.total_bytes > SPEC_CHAIN_NOALLOC_SCRATCH_BYTES) return SPEC_ERR_WORKSPACE;
  void* scratch = nullptr;
  if (sv::chain_scratch((hipStream_t)hip_stream, &scratch) != hipSuccess) return SPEC_ERR_HIP;
  const hipError_t e = sv::launch_chain(p, target_logits, draft_logits, draft_tokens, u_accept,
                                        u_draw, temperature, num_accepted, out_tokens, B, N, V,
                                        scratch, (hipStream_t)hip_stream);
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

size_t spec_accept_tree_workspace(int B, int T, int V) {
  if (check_tree(B, T, V) != SPEC_OK || B == 0 || T == 0) return 0;
  return sv::plan_tree(B, T, V).total_bytes;
}

spec_status spec_accept_tree(const float* target_logits, const int32_t* tokens,
                             const int32_t* parents, int32_t* accept_len, int32_t* path,
                             int32_t* out_tokens, int B, int T, int V, void* workspace,
                             size_t workspace_bytes, void* hip_stream) {
  const spec_status c = check_tree(B, T, V);
  if (c != SPEC_OK) return c;
  if (B == 0 || T == 0) return SPEC_OK;
  if (!target_logits || !tokens || !parents || !accept_len || !path || !out_tokens ||
      !workspace)
    return SPEC_ERR_NULL;
  const sv::TreePlan p = sv::plan_tree(B, T, V);
  if (workspace_bytes < p.total_bytes) return SPEC_ERR_WORKSPACE;
  const hipError_t e = sv::launch_tree(p, target_logits, tokens, parents, accept_len, path,
                                       out_tokens, B, T, V, workspace,
                                       (hipStream_t)hip_stream);
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

size_t spec_accept_tree_sampled_workspace(int B, int T, int V) {
  if (check_tree(B, T, V) != SPEC_OK || B == 0 || T == 0) return 0;
  return sv::plan_tree_sampled(B, T, V).total_bytes;
}

spec_status spec_accept_tree_sampled(const float* target_logits, const float* draft_logits,
                                     const int32_t* tokens, const int32_t* parents,
                                     const float* u_accept, const float* u_draw,
                                     float temperature, int32_t* accept_len, int32_t* path,
                                     int32_t* out_tokens, int B, int T, int V,
                                     void* workspace, size_t workspace_bytes,
                                     void* hip_stream) {
  const spec_status c = check_tree(B, T, V);
  if (c != SPEC_OK) return c;
  if (!(temperature > 0.f) || !isfinite(temperature)) return SPEC_ERR_SHAPE;
  if (B == 0 || T == 0) return SPEC_OK;
  if (!target_logits || !draft_logits || !tokens || !parents || !u_accept || !u_draw ||
      !accept_len || !path || !out_tokens || !workspace)
    return SPEC_ERR_NULL;
  const sv::STreePlan p = sv::plan_tree_sampled(B, T, V);
  if (workspace_bytes < p.total_bytes) return SPEC_ERR_WORKSPACE;
  const hipError_t e = sv::launch_tree_sampled(p, target_logits, draft_logits, tokens, parents,
                                               u_accept, u_draw, temperature, accept_len, path,
                                               out_tokens, B, T, V, workspace,
                                               (hipStream_t)hip_stream);
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

size_t spec_ngram_propose_workspace(int B, int L) {
  if (B < 1 || L < 0) return 0;
  return sv::plan_ngram(B, L).total_bytes;
}

spec_status spec_ngram_propose(const int32_t* context, const int32_t* context_lens,
                               int32_t* num_drafts, int32_t* drafts, int B, int L, int N,
                               int n_min, int n_max, void* workspace, size_t workspace_bytes,
                               void* hip_stream) {
  const spec_status c = check_ngram(B, L, N, n_min, n_max);
  if (c != SPEC_OK) return c;
  if (B == 0) return SPEC_OK;
  if (!num_drafts || !workspace || (L > 0 && !context) || (N > 0 && !drafts))
    return SPEC_ERR_NULL;
  const sv::NgramPlan p = sv::plan_ngram(B, L);
  if (workspace_bytes < p.total_bytes) return SPEC_ERR_WORKSPACE;
  const hipError_t e = sv::launch_ngram(p, context, context_lens, num_drafts, drafts, B, L, N,
                                        n_min, n_max, workspace, (hipStream_t)hip_stream);
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

spec_status spec_commit_kv(void* k, void* v, const int32_t* path, const int32_t* accept_len,
                           int32_t* new_len, int B, int T, int Hkv, int D, int ctx,
                           spec_dtype dtype, void* hip_stream) {
  if (B < 0 || T < 1 || Hkv < 1 || D < 1 || ctx < 0) return SPEC_ERR_SHAPE;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_ERR_UNSUPPORTED;
  if (T > SPEC_MAX_T || (D != 64 && D != 128)) return SPEC_ERR_UNSUPPORTED;
  if (((long long)ctx + T) * D >= (1ll << 31)) return SPEC_ERR_UNSUPPORTED;
  if ((long long)B * Hkv > SPEC_MAX_ROWS) return SPEC_ERR_UNSUPPORTED;   // int32 block ids
  if (B == 0) return SPEC_OK;
  if (!accept_len || !new_len) return SPEC_ERR_NULL;
  if (path != nullptr) {
    if (!k || !v) return SPEC_ERR_NULL;
    if (((uintptr_t)k | (uintptr_t)v) % 16 != 0) return SPEC_ERR_UNSUPPORTED;
  }
  const hipError_t e = sv::launch_commit(k, v, path, accept_len, new_len, B, T, Hkv, D, ctx,
                                         dtype == SPEC_BF16 ? 2 : 4, (hipStream_t)hip_stream);
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

}  // extern "C"
