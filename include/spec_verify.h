/*
 * spec_verify.h — C ABI of the speculative-decoding verify step for MI355X (gfx950).
 *
 * The verify step is the target model's single check of a batch of drafts:
 *
 *   1. verify attention — the target's pass over the accepted prefix plus the
 *      N draft positions is parallel over positions, so one pass yields a
 *      next-token distribution at each of the N+1 positions ("LLM Primer VI —
 *      Chapitre 9 — Décodage spéculatif", §9.1).  A draft tree is checked in
 *      the same single pass under a mask that encodes the tree (Primer §9.2 on
 *      EAGLE-2; "Parallel Decoding" glossary, "Medusa" → "Tree attention" and
 *      "L'attention en arbre : la brique commune").
 *   2. acceptance — for a chain, rejection sampling: keep draft x with
 *      probability min(1, p(x)/q(x)), else draw from the normalised (p − q)+ and
 *      drop the rest, so the output law is exactly the target's (Primer §9.1);
 *      for a tree, the longest path that agrees with the target, then the
 *      target's own choice (glossary "L'attention en arbre"; Primer §9.1–§9.2).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every data pointer is a caller-owned DEVICE buffer, dense row-major in the
 *    layout stated at each argument.  The library allocates no memory; scratch
 *    space comes from the caller's `workspace` (device memory, at least the
 *    size the matching *_workspace() query returns, no alignment beyond 256
 *    bytes required, contents need not be initialised).  The one exception is
 *    spec_accept_chain_noalloc, whose scratch is a static device array of the
 *    library; no other call keeps state between calls.
 *  - Work is enqueued asynchronously on `hip_stream` (a hipStream_t; NULL means
 *    the null stream).  Outputs are valid once that stream reaches the point
 *    after the call.  Concurrent calls must use distinct workspaces.
 *  - Errors: every call validates its arguments on the host before enqueuing
 *    anything and returns a spec_status; nothing is launched unless it returns
 *    SPEC_OK.  A launch failure reported by HIP gives SPEC_ERR_HIP.  Faults
 *    inside kernels surface at the caller's next synchronisation.  No
 *    exception crosses the ABI and the library never aborts.
 *  - Preconditions not checked on the device (results are unspecified but
 *    memory-safe if violated): logits are finite or -inf with a finite row
 *    maximum; parents satisfy parents[b][0] == -1 and 0 <= parents[b][i] < i.
 *    Out-of-range tokens and malformed parents never read out of bounds: such
 *    a draft or node is simply never accepted.
 *  - Empty problems (B == 0, or no query positions) return SPEC_OK without
 *    launching anything.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SPEC_OK = 0,
    SPEC_ERR_NULL = 1,         /* a required pointer is NULL                      */
    SPEC_ERR_SHAPE = 2,        /* a size is negative or inconsistent              */
    SPEC_ERR_UNSUPPORTED = 3,  /* valid but outside the supported limits          */
    SPEC_ERR_WORKSPACE = 4,    /* workspace_bytes below the queried size          */
    SPEC_ERR_HIP = 5,          /* the HIP runtime reported a launch error         */
    /* Not statuses: every int32 is a valid value of the type, so a C caller may
       pass any integer to spec_status_string. */
    SPEC_STATUS_INT32_MIN_ = -0x7fffffff - 1,
    SPEC_STATUS_INT32_MAX_ = 0x7fffffff
} spec_status;

typedef enum {
    SPEC_F32 = 0,              /* IEEE binary32                                   */
    SPEC_BF16 = 1,             /* bfloat16 (upper half of a binary32)             */
    /* not types: any int32 may be passed (others give SPEC_ERR_UNSUPPORTED) */
    SPEC_DTYPE_INT32_MIN_ = -0x7fffffff - 1,
    SPEC_DTYPE_INT32_MAX_ = 0x7fffffff
} spec_dtype;

/* Supported limits. */
#define SPEC_MAX_T 64          /* query positions (chain N+1, or tree nodes)      */
#define SPEC_MAX_V (1 << 24)   /* vocabulary size                                 */
#define SPEC_MAX_ROWS 0x7fffffff /* B·Hkv (attention), B·(2N+1) (chain), B·T (trees):
                                    block indices are 32-bit signed               */

/* Text for a status code (static storage; never NULL). */
const char* spec_status_string(spec_status status);

/* ---------------------------------------------------------------------------
 * Verify attention (Primer §9.1, §9.2; glossary "L'attention en arbre").
 *
 * For every sequence b, query position i < T and query head h:
 *
 *   O[b,i,h,:] = sum_{j in vis(b,i)} softmax_j(scale * <Q[b,i,h,:], K[b,g,j,:]>) * V[b,g,j,:]
 *
 * with g = h / (Hq/Hkv) (grouped-query attention) and the visible keys
 * vis(b,i) = {0 .. ctx-1} (the accepted prefix) ∪ {ctx + t : t is i or an
 * ancestor of i}.  A chain (parents == NULL) makes every earlier position an
 * ancestor, i.e. causal attention over the N+1 new positions.
 *
 *   q        [B, T, Hq, D]       dtype; already position-encoded
 *   k, v     [B, Hkv, ctx+T, D]  dtype; rows ctx..ctx+T-1 hold the T new
 *                                positions (appended before the call)
 *   parents  [B, T] int32 or NULL; tree: parents[b][0] = -1 (node 0 is the
 *            root, the last verified token), parents[b][i] < i
 *   out      [B, T, Hq, D] float32
 *   scale    softmax scale, normally 1/sqrt(D); must be finite and > 0
 *
 * Limits: 1 <= T <= 64, D in {64, 128}, Hkv >= 1, Hq % Hkv == 0, ctx >= 0,
 * (ctx + T)·D < 2^31, B·Hkv <= SPEC_MAX_ROWS; q, k, v and out 16-byte aligned
 * (SPEC_ERR_UNSUPPORTED otherwise).
 *
 * The workspace query takes the element type too: bf16 inputs run the
 * matrix-core kernel and fp32 inputs the vector kernel, whose key splits (and
 * so the partial results the workspace holds) differ.  It returns 0 for
 * arguments the call would reject and for empty problems.
 * ------------------------------------------------------------------------- */
size_t spec_verify_attention_workspace(int B, int T, int Hq, int Hkv, int D, int ctx,
                                       spec_dtype dtype);

spec_status spec_verify_attention(const void* q, const void* k, const void* v,
                                  const int32_t* parents, float* out,
                                  int B, int T, int Hq, int Hkv, int D, int ctx,
                                  spec_dtype dtype, float scale,
                                  void* workspace, size_t workspace_bytes,
                                  void* hip_stream);

/* ---------------------------------------------------------------------------
 * Verify attention over a paged KV cache.
 *
 * Serving engines keep the cache in pages ("LLM Primer VI", closing section
 * "Ce que prépare le Chapitre 9": paged KV is one of the runtime tools an
 * engine wires together with speculative decoding; "Parallel Decoding"
 * glossary, "Parallel decoding en production": the engines that run
 * speculation).  The operation is spec_verify_attention's, for every sequence
 * b with a prefix length of its own, ctx_b, and its keys and values in pages
 * of a shared pool: position i (0 <= i < ctx_b + T) of sequence b is row
 * i % page_size of page block_table[b][i / page_size]; positions ctx_b ..
 * ctx_b + T - 1 hold the T new positions.
 *
 *   q            [B, T, Hq, D]                 dtype
 *   k_pages,     SPEC_PAGES_HND: [num_pages, Hkv, page_size, D]
 *   v_pages      SPEC_PAGES_NHD: [num_pages, page_size, Hkv, D]   dtype
 *   block_table  [B, max_blocks] int32 page ids; entries past a sequence's
 *                last page are never read
 *   ctx_lens     [B] int32 prefix lengths, each in [0, max_ctx]; NULL: all max_ctx
 *   parents      [B, T] int32 or NULL, as for spec_verify_attention
 *   out          [B, T, Hq, D] float32
 *   max_ctx      the largest prefix length; sizes the launch and the workspace
 *                (spec_verify_attention_paged_workspace)
 *
 * Rows of a page past its sequence's length, and pages no table entry in
 * use names, are never read.  Not checked on the device (memory-safe, results
 * unspecified): ctx_lens outside [0, max_ctx] are clamped into it, page ids
 * outside [0, num_pages) are clamped into the pool.
 * Limits: those of spec_verify_attention, and page_size a power of two no
 * larger than SPEC_MAX_PAGE_SIZE, num_pages >= 1, max_blocks * page_size >=
 * max_ctx + T; q, k_pages, v_pages and out 16-byte aligned.  With equal
 * prefix lengths the result is bit-identical to spec_verify_attention's on
 * the same logical cache.
 * ------------------------------------------------------------------------- */
typedef enum {
    SPEC_PAGES_HND = 0,        /* a page holds each KV head's rows contiguously   */
    SPEC_PAGES_NHD = 1,        /* a page holds each position's KV heads together  */
    /* not layouts: any int32 may be passed (others give SPEC_ERR_UNSUPPORTED) */
    SPEC_PAGES_INT32_MIN_ = -0x7fffffff - 1,
    SPEC_PAGES_INT32_MAX_ = 0x7fffffff
} spec_page_layout;

#define SPEC_MAX_PAGE_SIZE (1 << 20)

size_t spec_verify_attention_paged_workspace(int B, int T, int Hq, int Hkv, int D, int max_ctx,
                                             spec_dtype dtype);

spec_status spec_verify_attention_paged(const void* q, const void* k_pages, const void* v_pages,
                                        const int32_t* block_table, const int32_t* ctx_lens,
                                        const int32_t* parents, float* out,
                                        int B, int T, int Hq, int Hkv, int D, int max_ctx,
                                        int page_size, int num_pages, int max_blocks,
                                        spec_page_layout layout, spec_dtype dtype, float scale,
                                        void* workspace, size_t workspace_bytes,
                                        void* hip_stream);

/* ---------------------------------------------------------------------------
 * Chain acceptance by rejection sampling (Primer §9.1).
 *
 * With p_i = softmax(target_logits[b,i,:] / temperature) (i = 0..N) and
 * q_i = softmax(draft_logits[b,i,:] / temperature) (i = 0..N-1):
 *   draft x_i is kept iff u_accept[b,i] < p_i(x_i) / q_i(x_i)  (q = 0 → +inf
 *   if p > 0, else 0); k = the first i not kept (N if all are kept);
 *   if k < N the committed token is drawn from w = (p_k − q_k)+ (or p_k when
 *   that sums to zero), else from w = p_N (the bonus token);
 *   the draw is y = min{j : C_j > u_draw[b,k] * C_{V-1}}, C_j the running sum
 *   of w in ascending token order (the last j with w_j > 0 if none).
 *
 *   target_logits  [B, N+1, V] float32
 *   draft_logits   [B, N, V]   float32
 *   draft_tokens   [B, N]      int32 (drafts drawn from q)
 *   u_accept       [B, N]      float32 in (0,1)
 *   u_draw         [B, N+1]    float32 in (0,1); only row k's is used
 *   temperature    > 0
 *   num_accepted   [B]         int32 out: k
 *   out_tokens     [B, N+1]    int32 out: x_0..x_{k-1}, y, then -1
 *
 * For N == 0 the pointers to draft_logits, draft_tokens and u_accept may be NULL.
 * Limits: N >= 0, 1 <= V <= SPEC_MAX_V, B·(2N+1) <= SPEC_MAX_ROWS.
 * ------------------------------------------------------------------------- */
size_t spec_accept_chain_workspace(int B, int N, int V);

spec_status spec_accept_chain(const float* target_logits, const float* draft_logits,
                              const int32_t* draft_tokens, const float* u_accept,
                              const float* u_draw, float temperature,
                              int32_t* num_accepted, int32_t* out_tokens,
                              int B, int N, int V,
                              void* workspace, size_t workspace_bytes, void* hip_stream);

/* ---------------------------------------------------------------------------
 * Chain acceptance without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.
 *
 * Arguments, results and errors are spec_accept_chain's, computed by the same
 * kernels.  The scratch they need (what spec_accept_chain_workspace sizes) is
 * a static device array of the library, SPEC_CHAIN_NOALLOC_SCRATCH_BYTES on
 * every GPU it runs on, held until the process ends; its address is looked up
 * once per device, at the first call there.  The call allocates nothing.
 * Problems that need more scratch (spec_accept_chain_workspace(B, N, V) >
 * SPEC_CHAIN_NOALLOC_SCRATCH_BYTES; for example B = 1024, N = 8, V = 152064
 * needs 1.6 MB) return SPEC_ERR_WORKSPACE before anything is enqueued.
 * Every call on one GPU uses the same array: calls ordered on one stream are
 * safe, calls that may overlap on one GPU (several streams, several host
 * threads) race and give unspecified results.
 * ------------------------------------------------------------------------- */
#define SPEC_CHAIN_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)

spec_status spec_accept_chain_noalloc(const float* target_logits, const float* draft_logits,
                                      const int32_t* draft_tokens, const float* u_accept,
                                      const float* u_draw, float temperature,
                                      int32_t* num_accepted, int32_t* out_tokens,
                                      int B, int N, int V, void* hip_stream);

/* ---------------------------------------------------------------------------
 * Greedy tree acceptance (glossary "L'attention en arbre : la brique commune";
 * Primer §9.1–§9.2).
 *
 * a_i = argmax_v target_logits[b,i,v] (lowest v among equal maxima) is the
 * target's own choice after node i.  Node 0 (the root) is accepted; node i > 0
 * is accepted iff its parent is accepted and tokens[b,i] == a_{parent(i)}.
 * The deepest accepted node l (lowest id among equally deep ones) ends the
 * accepted path root..l.
 *
 *   target_logits  [B, T, V]  float32, the target's logits at every node
 *   tokens         [B, T]     int32 draft token carried by each node (node 0 ignored)
 *   parents        [B, T]     int32, parents[b][0] = -1, parents[b][i] < i
 *   accept_len     [B]        int32 out: depth of l (number of accepted drafts)
 *   path           [B, T]     int32 out: node ids root..l, then -1
 *   out_tokens     [B, T]     int32 out: tokens of path nodes 1..l, then a_l, then -1
 *
 * Limits: 1 <= T <= 64, 1 <= V <= SPEC_MAX_V, B·T <= SPEC_MAX_ROWS.
 * ------------------------------------------------------------------------- */
size_t spec_accept_tree_workspace(int B, int T, int V);

spec_status spec_accept_tree(const float* target_logits, const int32_t* tokens,
                             const int32_t* parents,
                             int32_t* accept_len, int32_t* path, int32_t* out_tokens,
                             int B, int T, int V,
                             void* workspace, size_t workspace_bytes, void* hip_stream);

/* ---------------------------------------------------------------------------
 * Sampled (non-greedy) tree acceptance (Primer §9.1: keep a draft x with
 * probability min(1, p(x)/q(x)), else draw from the normalised (p − q)+, which
 * keeps the output distributed as the target's own sampling; Primer §9.2: the
 * target picks among several draft paths).
 *
 * p_n = softmax(target_logits[b,n,:] / temperature) and q_n =
 * softmax(draft_logits[b,n,:] / temperature); the children of node n are
 * candidates for the token after n, drawn independently from q_n.  The walk
 * starts at the root with ref = p_0.  At node n the children are tried in
 * increasing id order: child i (token x_i) is kept iff u_accept[b,i] <
 * ref(x_i) / q_n(x_i) (q = 0: +inf if ref(x) > 0, else 0; a token outside
 * [0, V) gives 0), and the walk moves to it with ref = p_i; after a rejection
 * ref becomes the normalised (ref − q_n)+ (p_n if that is empty).  When no
 * child of the current node l is kept, the emitted token y is drawn from ref
 * with u_draw[b,l]: y = min{j : C_j > u·C_{V-1}} over the running sum C of
 * ref in ascending token order (among tokens with positive weight).
 *
 *   target_logits, draft_logits  [B, T, V] float32 (row n of draft_logits is
 *                                the distribution node n's children came from)
 *   tokens         [B, T] int32 (node 0 ignored)
 *   parents        [B, T] int32, parents[b][0] = -1, parents[b][i] < i
 *   u_accept       [B, T] float32 in (0,1), node i's own ratio test (node 0 unused)
 *   u_draw         [B, T] float32 in (0,1), used at the node where the walk stops
 *   temperature    > 0
 *   accept_len     [B] int32 out: depth of l (number of kept drafts)
 *   path           [B, T] int32 out: node ids root..l, then -1
 *   out_tokens     [B, T] int32 out: tokens of path nodes 1..l, then y, then -1
 *
 * Precision: probabilities from float32-accurate exponentials (an exact
 * float64 argument split around the hardware exp2), every sum, ratio and
 * comparison in float64.  Limits: 1 <= T <= 64, 1 <= V <= SPEC_MAX_V,
 * B·T <= SPEC_MAX_ROWS.
 * ------------------------------------------------------------------------- */
size_t spec_accept_tree_sampled_workspace(int B, int T, int V);

spec_status spec_accept_tree_sampled(const float* target_logits, const float* draft_logits,
                                     const int32_t* tokens, const int32_t* parents,
                                     const float* u_accept, const float* u_draw,
                                     float temperature, int32_t* accept_len, int32_t* path,
                                     int32_t* out_tokens, int B, int T, int V,
                                     void* workspace, size_t workspace_bytes,
                                     void* hip_stream);

/* ---------------------------------------------------------------------------
 * n-gram (prompt-lookup) draft proposal ("LLM Primer VI", section "Pourquoi
 * ce chapitre existe": n-gram and suffix drafting among the draft algorithms;
 * §9.3: the largest speedups on highly repetitive loads; "Parallel Decoding"
 * glossary, "Parallel decoding en production": prompt lookup).
 *
 * For sequence b with history c[0..Lb-1] (Lb = context_lens[b], clamped to
 * [0, L]): for n = n_max down to n_min, the last n tokens are searched among
 * the earlier n-grams c[e-n+1..e], e <= Lb-2; the first n with an occurrence
 * wins and its most recent occurrence (largest e) is taken.  The drafts are
 * c[e+1 .. min(e+N, Lb-1)]; without an occurrence there is none.
 *
 *   context       [B, L] int32 token ids (positions >= context_lens[b] ignored)
 *   context_lens  [B] int32, or NULL (every history has L tokens)
 *   num_drafts    [B] int32 out: number of drafts (0..N)
 *   drafts        [B, N] int32 out: the drafts, then -1
 *
 * Limits: 0 <= N <= SPEC_MAX_T - 1, 1 <= n_min <= n_max <= SPEC_NGRAM_MAX.
 * Workspace: spec_ngram_propose_workspace(B, L).
 * ------------------------------------------------------------------------- */
#define SPEC_NGRAM_MAX 16

size_t spec_ngram_propose_workspace(int B, int L);

spec_status spec_ngram_propose(const int32_t* context, const int32_t* context_lens,
                               int32_t* num_drafts, int32_t* drafts,
                               int B, int L, int N, int n_min, int n_max,
                               void* workspace, size_t workspace_bytes, void* hip_stream);

/* ---------------------------------------------------------------------------
 * KV commit after acceptance (Primer §9.1: at the first divergence the engine
 * commits to the target's choice and drops the rest; glossary "Limites du
 * parallel decoding": tree attention keeps every branch's keys and values in
 * an enlarged cache, of which one branch survives verification).
 *
 * The verify pass found the T new positions' keys and values at rows
 * ctx..ctx+T-1 (see spec_verify_attention).  For every sequence b and KV head
 * g, with l = accept_len[b]:
 *
 *   K[b,g,ctx+i,:] <- K[b,g,ctx+path[b][i],:]   and the same for V, i = 0..l
 *   new_len[b] = ctx + l + 1
 *
 * i.e. the cache becomes the prefix followed by the accepted path, root first
 * (row ctx is the root, the last verified token).  Rows from new_len on are
 * left as they are.  The token emitted after the path (the target's own
 * choice, or the bonus token) has no key or value yet: the next pass computes
 * them.  A chain (path == NULL) already has its accepted positions in place:
 * only new_len is written, and k and v may then be NULL.
 *
 *   k, v        [B, Hkv, ctx+T, D]  dtype, modified in place; 16-byte aligned
 *   path        [B, T] int32 or NULL: node ids root..l then -1, as returned by
 *               spec_accept_tree (an entry outside [0, T) leaves row ctx+i as it is)
 *   accept_len  [B] int32: spec_accept_tree's accept_len, or spec_accept_chain's
 *               num_accepted (clamped to [0, T-1] on the device)
 *   new_len     [B] int32 out
 *
 * Limits: 1 <= T <= 64, D in {64, 128}, Hkv >= 1, ctx >= 0, (ctx + T)·D < 2^31.
 * No workspace.
 * ------------------------------------------------------------------------- */
spec_status spec_commit_kv(void* k, void* v, const int32_t* path, const int32_t* accept_len,
                           int32_t* new_len, int B, int T, int Hkv, int D, int ctx,
                           spec_dtype dtype, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
