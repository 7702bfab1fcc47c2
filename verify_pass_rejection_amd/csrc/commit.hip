// KV commit after acceptance: the accepted path's keys and values move to the
// front of the new positions, the cache length becomes prefix + path, and the
// other draft positions are dropped.
//
// "LLM Primer VI — Chapitre 9 — Décodage spéculatif", §9.1: at the first
// divergence the engine commits to the target's choice and throws the rest
// away.  "Parallel Decoding" glossary, "Limites du parallel decoding": tree
// attention keeps the keys and values of every branch in an enlarged cache;
// after verification one branch survives.
//
// One block per (sequence, KV head).  The kept rows are read into LDS before
// any is written, so the move is correct in place whatever the path (a root-
// to-leaf path only ever moves rows down, but a block-wide copy would race
// without the staging).  The length and the path are read together, then the
// K and V rows together: two round trips to memory.  16 bytes per thread and
// step.

#include "common.h"

namespace sv {

struct CommitArgs {
  uint8_t* k;                 // [B, Hkv, ctx+T, D] elements of esize bytes
  uint8_t* v;
  const int32_t* path;        // [B, T] node ids root..l then -1, or nullptr (chain)
  const int32_t* accept_len;  // [B]
  int32_t* new_len;           // [B]
  int B, T, Hkv, D, ctx, esize;
};

constexpr int kCommitThreads = 256;
constexpr int kCommitStage = 64 * 128 * 4;     // bytes per tensor: T <= 64 rows of D <= 128 fp32

__global__ __launch_bounds__(kCommitThreads) void commit_kv_kernel(CommitArgs a) {
  __shared__ uint4 stage[2][kCommitStage / 16];
  __shared__ int spath[64];
  const int u = blockIdx.x, b = u / a.Hkv, tid = threadIdx.x;
  // the length and the path entries in one round trip (T <= 64)
  const int len = a.accept_len[b];
  int pe = -1;
  if (a.path != nullptr && tid < a.T) pe = a.path[(size_t)b * a.T + tid];
  // accept_len outside [0, T-1] is clamped (memory safety; a precondition)
  const int l = min(max(len, 0), a.T - 1);
  if (u % a.Hkv == 0 && tid == 0) a.new_len[b] = a.ctx + l + 1;
  if (a.path == nullptr) return;               // a chain's accepted rows are in place
  if (tid < a.T) spath[tid] = (pe < 0 || pe >= a.T) ? tid : pe;   // invalid: row stays
  __syncthreads();
  const int row_bytes = a.D * a.esize;         // a multiple of 16 (D in {64, 128})
  const int rv = row_bytes / 16;               // 16-byte vectors per row
  const int n = (l + 1) * rv;
  const size_t off = ((size_t)u * (a.ctx + a.T) + a.ctx) * (size_t)row_bytes;
  uint8_t* const kb = a.k + off;
  uint8_t* const vb = a.v + off;
  // K and V rows of the path, together
  for (int idx = tid; idx < n; idx += kCommitThreads) {
    const int i = idx / rv, c = idx - i * rv;
    const size_t src = (size_t)spath[i] * row_bytes;
    const uint4 x = ((const uint4*)(kb + src))[c];
    const uint4 y = ((const uint4*)(vb + src))[c];
    stage[0][idx] = x;
    stage[1][idx] = y;
  }
  __syncthreads();
  for (int idx = tid; idx < n; idx += kCommitThreads) {
    const int i = idx / rv, c = idx - i * rv;
    ((uint4*)(kb + (size_t)i * row_bytes))[c] = stage[0][idx];
    ((uint4*)(vb + (size_t)i * row_bytes))[c] = stage[1][idx];
  }
}

hipError_t launch_commit(void* k, void* v, const int32_t* path, const int32_t* accept_len,
                         int32_t* new_len, int B, int T, int Hkv, int D, int ctx, int esize,
                         hipStream_t st) {
  CommitArgs a;
  a.k = (uint8_t*)k; a.v = (uint8_t*)v; a.path = path; a.accept_len = accept_len;
  a.new_len = new_len;
  a.B = B; a.T = T; a.Hkv = Hkv; a.D = D; a.ctx = ctx; a.esize = esize;
  commit_kv_kernel<<<B * Hkv, kCommitThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace sv
