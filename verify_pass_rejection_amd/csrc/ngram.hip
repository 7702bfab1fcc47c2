// n-gram (prompt-lookup) draft proposal: the drafts are the tokens that
// followed the most recent earlier occurrence of the context's last n tokens.
//
// "LLM Primer VI — Chapitre 9 — Décodage spéculatif", section "Pourquoi ce
// chapitre existe": n-gram and suffix drafting are among the draft algorithms;
// §9.3: the largest speedups come on highly repetitive loads.  "Parallel
// Decoding" glossary, "Parallel decoding en production": prompt lookup.
//
// For every candidate end e <= L-2 of an earlier occurrence, the match length
// l(e) is the number of tokens c[e], c[e-1], ... equal to c[L-1], c[L-2], ...
// (at most n_max, the occurrence starting at 0 or later).  The proposal comes
// from the largest key (min(l, n_max), e) with l >= n_min: the longest n-gram,
// then its most recent occurrence.
//
// Histories of up to 32768 tokens take one kernel, ngram_fused: one block per
// sequence holds the whole history in LDS (128 KB), every load in flight at
// once.  A key needs l >= n_min >= 1, so only the ends whose own token equals
// c[L-1] are extended backwards (a rare, divergent path on large
// vocabularies, and LDS reads only); a block maximum picks the key and the
// drafts are copied out of LDS.  One launch and one round trip to memory.
//
// Longer histories take two kernels:
//  ngram_scan     — grid (tiles, B), one 4096-position tile per block: the
//                   tile (and a 15-token halo) in LDS, l(e) for four
//                   positions per thread, the tile's largest key;
//  ngram_finalize — one wave per sequence: the largest key over the tiles,
//                   then the drafts c[e+1 .. min(e+N, L-1)].
// HBM-bound in principle: every token is read once (4 bytes), plus the halo.

#include "common.h"

namespace sv {

struct NgramArgs {
  const int32_t* ctx;      // [B, L]
  const int32_t* lens;     // [B] or nullptr (all L)
  int32_t* num;            // [B]
  int32_t* drafts;         // [B, N]
  uint64_t* part;          // [B, tiles] largest key per tile (0: none)
  int B, L, N, n_min, n_max, tiles;
};

constexpr int kNgThreads = 1024;
constexpr int kNgTile = 4096;                  // candidate ends per block
constexpr int kNgHalo = 15;                    // n_max <= 16

__device__ __forceinline__ int seq_len(const NgramArgs& a, int b) {
  return a.lens == nullptr ? a.L : min(max(a.lens[b], 0), a.L);
}

__global__ __launch_bounds__(kNgThreads) void ngram_scan_kernel(NgramArgs a) {
  __shared__ int tile[kNgTile + kNgHalo];
  __shared__ int suf[16];                      // suf[j] = c[L-1-j] (j < n_max)
  __shared__ uint64_t red[kNgThreads / kWave];
  const int t = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int L = seq_len(a, b);
  const int32_t* c = a.ctx + (size_t)b * a.L;
  const int e0 = t * kNgTile;
  // every load of the tile in flight at once, before this sequence's length
  // is known: indices clamped to the row, no branch around a load; entries
  // outside [0, L) are never compared
  constexpr int LOADS = (kNgTile + kNgHalo + kNgThreads - 1) / kNgThreads;
  int v[LOADS] = {};
  if (a.L >= 2) {                              // a kernel argument: no load to wait for
#pragma unroll
    for (int k = 0; k < LOADS; ++k) {
      const int idx = e0 - kNgHalo + tid + k * kNgThreads;
      v[k] = c[min(max(idx, 0), a.L - 1)];
    }
  }
  uint64_t best = 0;
  if (e0 <= L - 2) {                           // uniform: this tile holds candidate ends
    if (tid < a.n_max) suf[tid] = L - 1 - tid >= 0 ? c[L - 1 - tid] : 0;
#pragma unroll
    for (int k = 0; k < LOADS; ++k) {
      const int i = tid + k * kNgThreads;
      if (i < kNgTile + kNgHalo) tile[i] = v[k];
    }
    __syncthreads();
    int sj[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) sj[j] = suf[j & 15];
#pragma unroll
    for (int k = 0; k < kNgTile / kNgThreads; ++k) {
      const int e = e0 + k * kNgThreads + tid;
      // branch-free: bit j of m says c[e - j] == c[L - 1 - j] (j < n_max, e - j >= 0);
      // the match length is the run of ones from bit 0 (tile reads stay in range
      // for every j: e - j - e0 + 15 >= 0)
      uint32_t m = 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int tv = tile[e - j - e0 + kNgHalo];
        const bool eq = (j < a.n_max) & (e - j >= 0) & (tv == sj[j]);
        m |= (uint32_t)eq << j;
      }
      const int len = __builtin_ctz(~m);
      if (e <= L - 2 && len >= a.n_min) {
        const uint64_t key = ((uint64_t)len << 32) | (uint32_t)(e + 1);
        best = key > best ? key : best;
      }
    }
  }
  // block maximum of the keys
  best = wave_max(best);
  if ((tid & 63) == 0) red[tid >> 6] = best;
  __syncthreads();
  if (tid == 0) {
    uint64_t m = red[0];
    for (int w = 1; w < kNgThreads / kWave; ++w) m = red[w] > m ? red[w] : m;
    a.part[(size_t)b * a.tiles + t] = m;
  }
}

constexpr int kNgFusedMax = 32768;             // tokens one block holds in LDS

__global__ __launch_bounds__(kNgThreads) void ngram_fused_kernel(NgramArgs a) {
  constexpr int PER = kNgFusedMax / kNgThreads;
  __shared__ int row[kNgFusedMax];
  __shared__ uint64_t red[kNgThreads / kWave];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int32_t* c = a.ctx + (size_t)b * a.L;
  // the whole row, every load issued before anything waits (a.L is a kernel
  // argument; indices clamped into the row).  4-byte loads, 32 per thread:
  // 16-byte ones (8 per thread, rows aligned) made the call slower, 11.9 ->
  // 13.1 us on 64 histories of up to 32768 tokens.
  int v[PER];
  if (a.L >= 1) {
#pragma unroll
    for (int k = 0; k < PER; ++k) v[k] = c[min(tid + k * kNgThreads, a.L - 1)];
  }
  const int L = seq_len(a, b);
  if (a.L >= 1) {
#pragma unroll
    for (int k = 0; k < PER; ++k)
      if (tid + k * kNgThreads < a.L) row[tid + k * kNgThreads] = v[k];
  }
  __syncthreads();
  uint64_t best = 0;
  if (L >= 2) {                                // uniform
    const int s0 = row[L - 1];
#pragma unroll 4
    for (int k = 0; k < PER; ++k) {
      const int e = tid + k * kNgThreads;
      if (e <= L - 2 && row[e] == s0) {
        // extend backwards: c[e - j] against c[L - 1 - j], j < n_max, e - j >= 0
        int len = 1;
        while (len < a.n_max && e - len >= 0 && row[e - len] == row[L - 1 - len]) ++len;
        if (len >= a.n_min) {
          const uint64_t key = ((uint64_t)len << 32) | (uint32_t)(e + 1);
          best = key > best ? key : best;
        }
      }
    }
  }
  best = wave_max(best);
  if ((tid & 63) == 0) red[tid >> 6] = best;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kNgThreads / kWave; ++w) best = red[w] > best ? red[w] : best;
  const int e = best == 0 ? -1 : (int)(uint32_t)best - 1;
  const int n = e < 0 ? 0 : min(a.N, L - 1 - e);
  if (tid < a.N) a.drafts[(size_t)b * a.N + tid] = tid < n ? row[e + 1 + tid] : -1;
  if (tid == 0) a.num[b] = n;
}

__global__ __launch_bounds__(kWave) void ngram_finalize_kernel(NgramArgs a) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int L = seq_len(a, b);
  uint64_t best = 0;
  for (int t = lane; t < a.tiles; t += kWave) {
    const uint64_t k = a.part[(size_t)b * a.tiles + t];
    best = k > best ? k : best;
  }
  best = wave_max(best);
  const int e = best == 0 ? -1 : (int)(uint32_t)best - 1;
  const int n = e < 0 ? 0 : min(a.N, L - 1 - e);
  const int32_t* c = a.ctx + (size_t)b * a.L;
  for (int i = lane; i < a.N; i += kWave)
    a.drafts[(size_t)b * a.N + i] = i < n ? c[e + 1 + i] : -1;
  if (lane == 0) a.num[b] = n;
}

NgramPlan plan_ngram(int B, int L) {
  NgramPlan p{};
  p.tiles = L >= 2 ? (L - 2) / kNgTile + 1 : 1;
  p.total_bytes = align256((size_t)B * p.tiles * sizeof(uint64_t));
  return p;
}

hipError_t launch_ngram(const NgramPlan& p, const int32_t* ctx, const int32_t* lens,
                        int32_t* num, int32_t* drafts, int B, int L, int N, int n_min,
                        int n_max, void* workspace, hipStream_t st) {
  NgramArgs a;
  a.ctx = ctx; a.lens = lens; a.num = num; a.drafts = drafts;
  a.part = (uint64_t*)workspace;
  a.B = B; a.L = L; a.N = N; a.n_min = n_min; a.n_max = n_max; a.tiles = p.tiles;
  if (L <= kNgFusedMax) {
    ngram_fused_kernel<<<B, kNgThreads, 0, st>>>(a);
    return hipGetLastError();
  }
  ngram_scan_kernel<<<dim3(p.tiles, B), kNgThreads, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  ngram_finalize_kernel<<<B, kWave, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace sv
