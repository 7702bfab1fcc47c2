// Greedy acceptance of a draft tree.
//
// "Parallel Decoding" glossary, "L'attention en arbre : la brique commune": the
// root is the last verified token, every branch is a candidate continuation,
// and the longest accepted path becomes the generated sequence.  "LLM Primer
// VI — Chapitre 9 — Décodage spéculatif", §9.1: at the first divergence the
// engine commits to the target's own choice; §9.2: the target picks the best
// of several draft paths.
//
// Two kernels:
//  tree_argmax — every node's logit row is read once; per chunk the maximum
//                and its lowest index;
//  tree_walk   — one wave per sequence: merges the chunks into the target's
//                choice a_i at each node; every node then walks up its
//                parents: node i is accepted iff each node on its way to the
//                root carries its parent's choice; the deepest accepted node
//                (lowest id on ties, a wave reduction) ends the path; a_l
//                follows the path's tokens.

#include "common.h"

#include <limits.h>

namespace sv {

struct TreeArgs {
  const float* logits;     // [B, T, V]
  const int32_t* tokens;   // [B, T]
  const int32_t* parents;  // [B, T]
  int32_t* accept_len;     // [B]
  int32_t* path;           // [B, T]
  int32_t* out;            // [B, T]
  float* part_val;         // [B*T, nchunks]
  int32_t* part_idx;       // [B*T, nchunks]
  int B, T, V, nchunks;
};

// 512 threads over an 8192-logit chunk (four float4 loads per thread): 0.8 and
// 1.8 us faster than 256 threads on the 64-node and 42-node trees of 32000
// logits; 4096-logit chunks were slower.
constexpr int kArgThreads = 512;
constexpr int kArgChunk = 8192;

typedef float f32x4_nt __attribute__((ext_vector_type(4)));

// (v, i) is better than (bv, bi): larger value, or equal value and lower index.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}
// The best (value, index) over the wave, in every lane: lane pairs inside
// each row by DPP, then row pairs and halves by row swaps.
__device__ __forceinline__ void wave_best(float& bv, int& bi) {
  auto take = [&](float ov, int oi) { if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; } };
  take(dpp_f<kDppXor1>(bv), __builtin_amdgcn_mov_dpp(bi, kDppXor1, 0xf, 0xf, false));
  take(dpp_f<kDppXor2>(bv), __builtin_amdgcn_mov_dpp(bi, kDppXor2, 0xf, 0xf, false));
  take(dpp_f<kDppXor7>(bv), __builtin_amdgcn_mov_dpp(bi, kDppXor7, 0xf, 0xf, false));
  take(dpp_f<kDppXor15>(bv), __builtin_amdgcn_mov_dpp(bi, kDppXor15, 0xf, 0xf, false));
  float vlo, vhi, ilo, ihi;
  row_pair<false>(bv, vlo, vhi);
  row_pair<false>(__int_as_float(bi), ilo, ihi);
  bv = vlo; bi = __float_as_int(ilo);
  take(vhi, __float_as_int(ihi));
  row_pair<true>(bv, vlo, vhi);
  row_pair<true>(__int_as_float(bi), ilo, ihi);
  bv = vlo; bi = __float_as_int(ilo);
  take(vhi, __float_as_int(ihi));
}

template <int VEC>
__global__ __launch_bounds__(kArgThreads) void tree_argmax_kernel(TreeArgs a) {
  constexpr int ITER = kArgChunk / (kArgThreads * VEC);
  __shared__ float sv_[kArgThreads / kWave];
  __shared__ int si_[kArgThreads / kWave];
  const int ch = blockIdx.x, row = blockIdx.y;
  const float* z = a.logits + (size_t)row * a.V;
  const int begin = ch * kArgChunk;

  float v[ITER * VEC];
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int j = begin + (it * kArgThreads + threadIdx.x) * VEC;
    if constexpr (VEC == 4) {
      float4 x = {kNegInf, kNegInf, kNegInf, kNegInf};
      if (j < a.V) {                      // logits are read once: non-temporal
        const f32x4_nt y = __builtin_nontemporal_load((const f32x4_nt*)(z + j));
        x = make_float4(y[0], y[1], y[2], y[3]);
      }
      v[it * 4 + 0] = x.x; v[it * 4 + 1] = x.y; v[it * 4 + 2] = x.z; v[it * 4 + 3] = x.w;
    } else {
      v[it] = j < a.V ? z[j] : kNegInf;
    }
  }
  float bv = kNegInf;
  int bi = INT_MAX;
#pragma unroll
  for (int it = 0; it < ITER; ++it)
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const int j = begin + (it * kArgThreads + threadIdx.x) * VEC + e;
      if (j < a.V && better(v[it * VEC + e], j, bv, bi)) { bv = v[it * VEC + e]; bi = j; }
    }
  wave_best(bv, bi);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) { sv_[wave] = bv; si_[wave] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kArgThreads / kWave; ++w)
      if (better(sv_[w], si_[w], bv, bi)) { bv = sv_[w]; bi = si_[w]; }
    a.part_val[(size_t)row * a.nchunks + ch] = bv;
    a.part_idx[(size_t)row * a.nchunks + ch] = bi;
  }
}

// Rows of up to kWalkChunks chunks (V <= 65536) are merged from straight-line
// loads; a loop over the chunks waited for each chunk's pair of loads in turn.
constexpr int kWalkChunks = 8;

__global__ __launch_bounds__(64) void tree_walk_kernel(TreeArgs a) {
  __shared__ int choice[64], par[64], tok[64], path_nodes[64];
  __shared__ int s_best, s_depth;
  const int b = blockIdx.x, i = threadIdx.x, T = a.T;
  if (i < T) {
    const size_t row = (size_t)b * T + i;
    const int pa = a.parents[row], tk = a.tokens[row];
    const float* pv = a.part_val + row * a.nchunks;
    const int* pi = a.part_idx + row * a.nchunks;
    float bv;
    int bi;
    if (a.nchunks <= kWalkChunks) {
      // every load issued at once: chunks past the last re-read the last one,
      // which the merge leaves unchanged (equal value and index is not better)
      float v[kWalkChunks];
      int j[kWalkChunks];
#pragma unroll
      for (int c = 0; c < kWalkChunks; ++c) {
        const int cc = min(c, a.nchunks - 1);
        v[c] = pv[cc];
        j[c] = pi[cc];
      }
      bv = v[0];
      bi = j[0];
#pragma unroll
      for (int c = 1; c < kWalkChunks; ++c)
        if (better(v[c], j[c], bv, bi)) { bv = v[c]; bi = j[c]; }
    } else {
      bv = pv[0];
      bi = pi[0];
      for (int c = 1; c < a.nchunks; ++c)
        if (better(pv[c], pi[c], bv, bi)) { bv = pv[c]; bi = pi[c]; }
    }
    choice[i] = bi;
    par[i] = pa;
    tok[i] = tk;
  }
  __syncthreads();
  // Every node walks up to the root on its own: accepted iff each node on the
  // way carries its parent's choice; a parent that is not strictly smaller
  // (malformed input) ends the walk unaccepted.
  int depth = -1;                                // -1: not accepted
  if (i < T) {
    bool ok = true;
    int d = 0, n = i;
    while (n != 0) {
      const int p = par[n];
      if (p < 0 || p >= n) { ok = false; break; }
      ok = ok && tok[n] == choice[p];
      n = p;
      ++d;
    }
    if (ok) depth = d;
  }
  // Deepest accepted node, lowest id on ties (node 0 is always accepted).
  int best_d = depth, best_i = i;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int od = __shfl_xor(best_d, off), oi = __shfl_xor(best_i, off);
    if (od > best_d || (od == best_d && oi < best_i)) { best_d = od; best_i = oi; }
  }
  if (i == 0) {
    int n = best_i;
    for (int k = best_d; k >= 0; --k) { path_nodes[k] = n; n = par[n]; }
    s_best = best_i;
    s_depth = best_d;
  }
  __syncthreads();
  if (i < T) {
    const int d = s_depth;
    const size_t o = (size_t)b * T + i;
    a.path[o] = i <= d ? path_nodes[i] : -1;
    a.out[o] = i < d ? tok[path_nodes[i + 1]] : (i == d ? choice[s_best] : -1);
    if (i == 0) a.accept_len[b] = d;
  }
}

TreePlan plan_tree(int B, int T, int V) {
  TreePlan p{};
  p.chunk = kArgChunk;
  p.nchunks = (V + kArgChunk - 1) / kArgChunk;
  p.part_bytes = align256((size_t)B * T * p.nchunks * sizeof(float));
  p.total_bytes = 2 * p.part_bytes;
  return p;
}

hipError_t launch_tree(const TreePlan& p, const float* logits, const int32_t* tokens,
                       const int32_t* parents, int32_t* accept_len, int32_t* path,
                       int32_t* out, int B, int T, int V, void* workspace, hipStream_t st) {
  TreeArgs a;
  a.logits = logits; a.tokens = tokens; a.parents = parents;
  a.accept_len = accept_len; a.path = path; a.out = out;
  a.part_val = (float*)workspace;
  a.part_idx = (int32_t*)((char*)workspace + p.part_bytes);
  a.B = B; a.T = T; a.V = V; a.nchunks = p.nchunks;
  const bool vec4 = (V % 4 == 0) && ((uintptr_t)logits % 16 == 0);
  const dim3 g1(p.nchunks, B * T);
  if (vec4) tree_argmax_kernel<4><<<g1, kArgThreads, 0, st>>>(a);
  else tree_argmax_kernel<1><<<g1, kArgThreads, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  tree_walk_kernel<<<B, 64, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace sv
