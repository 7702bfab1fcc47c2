// Chain acceptance by rejection sampling.
//
// "LLM Primer VI — Chapitre 9 — Décodage spéculatif", §9.1: draft x drawn from
// q is kept with probability min(1, p(x)/q(x)); at the first draft that is not
// kept, the target's own token is drawn from the normalised positive part of
// p − q and the rest is dropped; this leaves the output distributed exactly as
// pure target sampling.  The pass gives N+1 target distributions, so when all
// N drafts are kept the last one supplies a bonus token.
//
// Three kernels (kernel boundaries order every step; no in-kernel signalling):
//  chain_stats  — one pass over every logit row (all B*(2N+1) rows), per chunk
//                 the row maximum and sum of 2^((z - max) log2(e)/tau);
//  chain_chunks — grid (group of draw chunks, sequence): every block first takes
//                 the sequence's decision (merges the chunk statistics into
//                 the row normalisers, runs the N ratio tests with two gathers
//                 a row, takes the first rejection k), then sums the weights
//                 of its chunks of the drawn row (the residual (p_k - q_k)+, or
//                 p_N); block 0 records the decision;
//  chain_select — one block per sequence: locates the chunk holding the
//                 inverse-CDF crossing from the chunk sums and re-scans that
//                 one chunk (if the residual is empty it first sums p_k's
//                 chunks itself).  Only the drawn row pair is read a second
//                 time.
//
// Every row's ratio test depends on that row alone, so computing all of them
// and then taking the first rejection gives the same result as the
// sequential walk.

#include <mutex>

#include "common.h"

namespace sv {

struct ChainArgs {
  const float* target;   // [B, N+1, V]
  const float* draft;    // [B, N, V]
  const int32_t* tokens; // [B, N]
  const float* u_acc;    // [B, N]
  const float* u_draw;   // [B, N+1]
  int32_t* num_acc;      // [B]
  int32_t* out;          // [B, N+1]
  float2* stats;         // [B, 2N+1, nchunks]: (row max, sum of 2^((z-max)c))
  float* csum;           // [B, 2, dchunks]: chunk sums of the residual and of p
  float4* decision;      // [B]: (k, p-row max, p-row log2 sum, unused) ...
  float4* decision_q;    // [B]: (q-row max, q-row log2 sum, unused, unused)
  int B, N, V, chunk, nchunks, dchunks;
  float c2;              // log2(e) / temperature
};

constexpr int kStatsThreads = 512;
constexpr int kStatsChunk = 16384;    // logits per stats block
constexpr int kDrawThreads = 1024;
constexpr int kDrawPer = 8;           // weights per thread per draw chunk
constexpr int kDrawChunk = kDrawThreads * kDrawPer;
// Draw chunks summed per chain_chunks block: one when a chunk per block still
// fits one wave of resident blocks (small batches are latency-bound: more
// blocks, shorter each), else five (about one block per CU, every load of the
// block in flight at once).
constexpr int kDrawCpbLarge = 5;
constexpr int kDrawCpbScalar = 3;     // the scalar-load path: five would spill
constexpr int kDrawResident = 512;    // 1024-thread blocks resident on 256 CUs

__device__ __forceinline__ const float* chain_row(const ChainArgs& a, int b, int rho) {
  return rho <= a.N ? a.target + ((size_t)b * (a.N + 1) + rho) * a.V
                    : a.draft + ((size_t)b * a.N + (rho - a.N - 1)) * a.V;
}

// The statistics pass reads every logit once; chain_chunks then reads the one
// drawn row of each sequence again.  When all the logits fit well inside the
// 256 MB last-level cache, ordinary loads leave the drawn rows there (0.9 of
// 20 us on a one-sequence chain of 11 rows of 128256); a larger stream takes
// non-temporal loads, which keep it at full rate (8 of 130 us on 64 x 17 rows
// of 152064).
constexpr size_t kCachedLogitBytes = size_t(128) << 20;

template <bool NT>
__device__ __forceinline__ float4 load_stream4(const float* p) {
  if constexpr (NT) {
    typedef float f32x4_nt __attribute__((ext_vector_type(4)));
    const f32x4_nt v = __builtin_nontemporal_load((const f32x4_nt*)p);
    return make_float4(v[0], v[1], v[2], v[3]);
  } else {
    return *(const float4*)p;
  }
}

__device__ __forceinline__ float4 load_draw4(const float* p) { return *(const float4*)p; }

// (m, s) pairs: s = sum 2^((z - m) c).
__device__ __forceinline__ void merge_ms(float& m, float& s, float m2, float s2, float c) {
  const float mx = fmaxf(m, m2);
  if (mx == kNegInf) return;
  s = s * fast_exp2((m - mx) * c) + s2 * fast_exp2((m2 - mx) * c);
  m = mx;
}
// (max, sum) over each row of 16 lanes, merged in a fixed order by DPP.
__device__ __forceinline__ void group16_merge_ms(float& m, float& s, float c) {
  merge_ms(m, s, dpp_f<kDppXor1>(m), dpp_f<kDppXor1>(s), c);
  merge_ms(m, s, dpp_f<kDppXor2>(m), dpp_f<kDppXor2>(s), c);
  merge_ms(m, s, dpp_f<kDppXor7>(m), dpp_f<kDppXor7>(s), c);
  merge_ms(m, s, dpp_f<kDppXor15>(m), dpp_f<kDppXor15>(s), c);
}
// (max, sum) over the wave: the rows of 16 first, then row pairs and halves
// by row swaps (lower first).
__device__ __forceinline__ void wave_merge_ms(float& m, float& s, float c) {
  group16_merge_ms(m, s, c);
  float m0, m1, s0, s1;
  row_pair<false>(m, m0, m1);
  row_pair<false>(s, s0, s1);
  m = m0; s = s0;
  merge_ms(m, s, m1, s1, c);
  row_pair<true>(m, m0, m1);
  row_pair<true>(s, s0, s1);
  m = m0; s = s0;
  merge_ms(m, s, m1, s1, c);
}

template <int VEC, bool NT>
__global__ __launch_bounds__(kStatsThreads) void chain_stats_kernel(ChainArgs a) {
  constexpr int ITER = kStatsChunk / (kStatsThreads * VEC);
  __shared__ float sm[kStatsThreads / kWave], ss[kStatsThreads / kWave];
  const int ch = blockIdx.x, row = blockIdx.y;
  const int rows = 2 * a.N + 1;
  const int b = row / rows, rho = row % rows;
  const float* z = chain_row(a, b, rho);
  const int begin = ch * kStatsChunk;

  float v[ITER * VEC];
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int j = begin + (it * kStatsThreads + threadIdx.x) * VEC;
    if constexpr (VEC == 4) {
      float4 x = {kNegInf, kNegInf, kNegInf, kNegInf};
      if (j < a.V) x = load_stream4<NT>(z + j);   // V % 4 == 0 on this path
      v[it * 4 + 0] = x.x; v[it * 4 + 1] = x.y; v[it * 4 + 2] = x.z; v[it * 4 + 3] = x.w;
    } else {
      v[it] = j < a.V ? z[j] : kNegInf;
    }
  }
  float m = v[0];
#pragma unroll
  for (int e = 1; e < ITER * VEC; ++e) m = fmaxf(m, v[e]);
  float s = 0.f;
  if (m != kNegInf) {
#pragma unroll
    for (int e = 0; e < ITER * VEC; ++e) s += fast_exp2((v[e] - m) * a.c2);
  }
  wave_merge_ms(m, s, a.c2);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) { sm[wave] = m; ss[wave] = s; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float M = sm[0], S = ss[0];
    for (int w = 1; w < kStatsThreads / kWave; ++w) merge_ms(M, S, sm[w], ss[w], a.c2);
    a.stats[(size_t)row * a.nchunks + ch] = make_float2(M, S);
  }
}

// The drawn row: weights (p - q)+ (RESID) or p alone.
struct DrawRow {
  const float* zp;
  const float* zq;   // read only when RESID
  float mp, lp;      // row max and log2 of the sum for p
  float mq, lq;
  float c;
};

template <bool RESID>
__device__ __forceinline__ float draw_w(const DrawRow& r, float xp, float xq) {
  const float p = fast_exp2((xp - r.mp) * r.c - r.lp);
  if constexpr (!RESID) return p;
  const float q = fast_exp2((xq - r.mq) * r.c - r.lq);
  return fmaxf(p - q, 0.f);
}

// Logits of this thread's kDrawPer tokens in draw chunk `chunk`.  Indices are
// clamped into the row so that every load is issued without a branch (a
// branch around each load makes the compiler wait for each one in turn); the
// weights of tokens past the row are zeroed by draw_weights_from.
template <int VEC, bool RESID>
__device__ __forceinline__ void draw_load(const DrawRow& r, int V, int chunk, float* xp,
                                          float* xq) {
  const int j0 = chunk * kDrawChunk + threadIdx.x * kDrawPer;
  if constexpr (VEC == 4) {
    static_assert(kDrawPer % 4 == 0, "whole float4 per thread");
#pragma unroll
    for (int i = 0; i < kDrawPer; i += 4) {
      const int j = min(j0 + i, V - 4);     // V % 4 == 0 on this path
      const float4 p4 = load_draw4(r.zp + j);
      xp[i] = p4.x; xp[i + 1] = p4.y; xp[i + 2] = p4.z; xp[i + 3] = p4.w;
      if constexpr (RESID) {
        const float4 q4 = load_draw4(r.zq + j);
        xq[i] = q4.x; xq[i + 1] = q4.y; xq[i + 2] = q4.z; xq[i + 3] = q4.w;
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < kDrawPer; ++e) {
      const int j = min(j0 + e, V - 1);
      xp[e] = r.zp[j];
      if constexpr (RESID) xq[e] = r.zq[j];
    }
  }
}

template <bool RESID>
__device__ __forceinline__ void draw_weights_from(const DrawRow& r, int V, int chunk,
                                                  const float* xp, const float* xq, float* w) {
  const int j0 = chunk * kDrawChunk + threadIdx.x * kDrawPer;
#pragma unroll
  for (int e = 0; e < kDrawPer; ++e) w[e] = (j0 + e < V) ? draw_w<RESID>(r, xp[e], xq[e]) : 0.f;
}

// The kDrawPer weights of this thread in draw chunk `chunk` (RESID or not is
// a block-uniform choice).
template <int VEC, bool RESID>
__device__ __forceinline__ void draw_weights(const DrawRow& r, int V, int chunk, float* w) {
  float xp[kDrawPer], xq[kDrawPer];
  draw_load<VEC, RESID>(r, V, chunk, xp, xq);
  draw_weights_from<RESID>(r, V, chunk, xp, xq, w);
}
template <int VEC>
__device__ __forceinline__ void draw_weights(const DrawRow& r, int V, int chunk, float* w) {
  if (r.zq != nullptr) draw_weights<VEC, true>(r, V, chunk, w);
  else draw_weights<VEC, false>(r, V, chunk, w);
}

// Running sums inside one draw chunk, in a fixed order: the thread's own
// weights left to right, thread offsets from an inclusive wave scan and a
// sequential scan of the wave totals.  prefix[e] is the running sum up to and
// including weight e of this thread; the chunk total is prefix[kDrawPer-1] of
// the last thread, so re-running the same scan reproduces it bit for bit.
__device__ __forceinline__ void chunk_scan(const float* w, float* prefix, float* wave_tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float local[kDrawPer];
  local[0] = w[0];
#pragma unroll
  for (int e = 1; e < kDrawPer; ++e) local[e] = local[e - 1] + w[e];
  const float incl = wave_scan(local[kDrawPer - 1]);
  const float excl = wave_prev(incl);
  __syncthreads();                               // wave_tot is free again
  if (lane == kWave - 1) wave_tot[wave] = incl;
  __syncthreads();
  // the wave's offset: the totals of the waves before it, added in wave order
  // (every read issued at once; adding 0 to the others changes no bit)
  float wo = 0.f;
#pragma unroll
  for (int i = 0; i < kDrawThreads / kWave; ++i) wo += i < wave ? wave_tot[i] : 0.f;
  const float off = wo + excl;
#pragma unroll
  for (int e = 0; e < kDrawPer; ++e) prefix[e] = off + local[e];
}

// The decision of sequence b, taken by a whole block of NT threads: merges the
// chunk statistics into the row normalisers (row_m: max, row_l: log2 of the
// sum; 16 lanes per row when a row has at most 16 chunks, else a wave with
// lane-strided partial merges, then DPP and row-swap merges in a fixed
// order), runs the N ratio tests (keep x_i iff u < p_i(x_i)/q_i(x_i))
// and returns k, the first rejection (N if none), to every thread.
template <int NT>
__device__ __forceinline__ int chain_decision(const ChainArgs& a, int b, float* row_m,
                                              float* row_l, int* s_k) {
  const int tid = threadIdx.x, N = a.N, rows = 2 * N + 1;
  const int lane = tid & 63, wave = tid >> 6;
  // The drafted tokens' logits are gathered first so that their latency
  // overlaps the merge of the chunk statistics.
  int x = -1;
  float zp = 0.f, zq = 0.f;
  if (tid < N) {
    x = a.tokens[(size_t)b * N + tid];
    if (x >= 0 && x < a.V) {
      zp = a.target[((size_t)b * (N + 1) + tid) * a.V + x];
      zq = a.draft[((size_t)b * N + tid) * a.V + x];
    }
  }
  if (a.nchunks <= 16) {
    // 16 lanes per row, every row in one pass (up to 64 rows): lanes past the
    // row's chunks hold (-inf, 0), which every merge step passes through
    // exactly, so the result is that of a merge over the whole wave
    const int l16 = tid & 15;
    for (int r = tid >> 4; r < rows; r += NT / 16) {
      const float2* st = a.stats + ((size_t)b * rows + r) * a.nchunks;
      float M = kNegInf, S = 0.f;
      if (l16 < a.nchunks) merge_ms(M, S, st[l16].x, st[l16].y, a.c2);
      group16_merge_ms(M, S, a.c2);
      if (l16 == 0) { row_m[r] = M; row_l[r] = log2f(S); }
    }
  } else {
    for (int r = wave; r < rows; r += NT / kWave) {
      const float2* st = a.stats + ((size_t)b * rows + r) * a.nchunks;
      float M = kNegInf, S = 0.f;
      for (int i = lane; i < a.nchunks; i += kWave) merge_ms(M, S, st[i].x, st[i].y, a.c2);
      wave_merge_ms(M, S, a.c2);
      if (lane == 0) { row_m[r] = M; row_l[r] = log2f(S); }
    }
  }
  __syncthreads();
  // The N <= 63 ratio tests sit in wave 0: k is its first failing lane.
  if (wave == 0) {
    bool ok = true;
    if (tid < N) {
      ok = false;
      if (x >= 0 && x < a.V) {
        const float lp = (zp - row_m[tid]) * a.c2 - row_l[tid];
        const float lq = (zq - row_m[N + 1 + tid]) * a.c2 - row_l[N + 1 + tid];
        const float r = exp2f(lp - lq);   // q = 0: +inf when p > 0; NaN (reject) when both 0
        ok = a.u_acc[(size_t)b * N + tid] < r;
      }
    }
    const uint64_t rej = __ballot(!ok);
    if (tid == 0) *s_k = rej ? __builtin_ctzll(rej) : N;
  }
  __syncthreads();
  return *s_k;
}

// The drawn row's weights for sequence b, from the decision record.
// Both records are loaded whatever k is, so that neither load waits for the
// other.
__device__ __forceinline__ void draw_rows(const ChainArgs& a, int b, int& k, DrawRow& dp,
                                          DrawRow& dr) {
  const float4 dec = a.decision[b];
  const float4 dq = a.decision_q[b];
  k = __float_as_int(dec.x);
  dp.zp = a.target + ((size_t)b * (a.N + 1) + k) * a.V;
  dp.mp = dec.y;
  dp.lp = dec.z;
  dp.c = a.c2;
  dp.zq = nullptr;
  dp.mq = dp.lq = 0.f;
  dr = dp;
  if (k < a.N) {
    dr.zq = a.draft + ((size_t)b * a.N + k) * a.V;
    dr.mq = dq.x;
    dr.lq = dq.y;
  }
}

// Chunk sums of draw chunks [c0, c0 + CPB) of the drawn row: every load
// first, then the scans of all the chunks with one barrier between their wave
// scans and their totals (chunks past the row are not written).  A chunk's
// total is what chunk_scan gives the last thread, with the same additions in
// the same order, so chain_select's re-scan reproduces it bit for bit.
// wave_tot holds CPB × (waves per block) floats.
template <int VEC, int CPB, bool RESID>
__device__ __forceinline__ void chunk_sums(const ChainArgs& a, const DrawRow& r, int b, int c0,
                                           float* wave_tot) {
  constexpr int NW = kDrawThreads / kWave;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float xp[CPB][kDrawPer], xq[CPB][kDrawPer];
#pragma unroll
  for (int cc = 0; cc < CPB; ++cc) draw_load<VEC, RESID>(r, a.V, c0 + cc, xp[cc], xq[cc]);
  float last[CPB], excl[CPB];
#pragma unroll
  for (int cc = 0; cc < CPB; ++cc) {
    last[cc] = excl[cc] = 0.f;
    if (c0 + cc >= a.dchunks) continue;          // block-uniform
    float w[kDrawPer];
    draw_weights_from<RESID>(r, a.V, c0 + cc, xp[cc], xq[cc], w);
    float l = w[0];
#pragma unroll
    for (int e = 1; e < kDrawPer; ++e) l = l + w[e];
    const float incl = wave_scan(l);
    const float ex = wave_prev(incl);
    last[cc] = l;
    excl[cc] = ex;
    if (lane == kWave - 1) wave_tot[cc * NW + wave] = incl;
  }
  __syncthreads();
  if (threadIdx.x == kDrawThreads - 1) {
#pragma unroll
    for (int cc = 0; cc < CPB; ++cc) {
      if (c0 + cc >= a.dchunks) continue;
      float wo = 0.f;
#pragma unroll
      for (int i = 0; i < NW - 1; ++i) wo += wave_tot[cc * NW + i];
      a.csum[(size_t)b * 2 * a.dchunks + c0 + cc] = (wo + excl[cc]) + last[cc];
    }
  }
}

// Every block of a sequence takes the decision itself (the statistics are
// small), so that no launch sits between the statistics and the draw, and
// then sums CPB chunks of the drawn row; block 0 records the decision for
// chain_select.
template <int VEC, int CPB>
__global__ __launch_bounds__(kDrawThreads) void chain_chunks_kernel(ChainArgs a) {
  __shared__ float wave_tot[CPB * (kDrawThreads / kWave)];
  __shared__ float row_m[128], row_l[128];
  __shared__ int s_k;
  const int c = blockIdx.x, b = blockIdx.y, N = a.N;
  const int k = chain_decision<kDrawThreads>(a, b, row_m, row_l, &s_k);
  DrawRow dr;
  dr.zp = a.target + ((size_t)b * (N + 1) + k) * a.V;
  dr.mp = row_m[k];
  dr.lp = row_l[k];
  dr.c = a.c2;
  dr.zq = nullptr;
  dr.mq = dr.lq = 0.f;
  if (k < N) {
    dr.zq = a.draft + ((size_t)b * N + k) * a.V;
    dr.mq = row_m[N + 1 + k];
    dr.lq = row_l[N + 1 + k];
  }
  if (c == 0 && threadIdx.x == 0) {
    a.decision[b] = make_float4(__int_as_float(k), row_m[k], row_l[k], 0.f);
    a.decision_q[b] = make_float4(dr.mq, dr.lq, 0.f, 0.f);
  }
  if (k < N) chunk_sums<VEC, CPB, true>(a, dr, b, c * CPB, wave_tot);
  else chunk_sums<VEC, CPB, false>(a, dr, b, c * CPB, wave_tot);
}

template <int VEC>
__global__ __launch_bounds__(kDrawThreads) void chain_select_kernel(ChainArgs a) {
  __shared__ float wave_tot[kDrawThreads / kWave];
  __shared__ int wave_hit[kDrawThreads / kWave];
  __shared__ int s_chunk;
  __shared__ float s_carry, s_target, s_total;
  const int b = blockIdx.x, tid = threadIdx.x, N = a.N, nch = a.dchunks;
  const int lane = tid & 63, wave = tid >> 6;
  // The sequence's draw uniforms, its decision records and the chunk sums
  // are independent loads, issued together; u is picked once k is known.
  __shared__ float u_l[64];                // N + 1 <= 64, checked on the host
  if (tid <= N) u_l[tid] = a.u_draw[(size_t)b * (N + 1) + tid];
  int k;
  DrawRow dp, dr;
  draw_rows(a, b, k, dp, dr);
  float* cs = a.csum + (size_t)b * 2 * nch;
  __shared__ float cs_l[kDrawThreads];
  const bool in_lds = nch <= kDrawThreads;
  if (in_lds && tid < nch) cs_l[tid] = cs[tid];           // one parallel load
  __syncthreads();
  const float u = u_l[k];

  // The chunk holding the crossing of u·total, over the chunk sums row[0..nch),
  // found by wave 0.  The additions run in chunk order, as one thread would
  // take them: with nch <= 64 lane i holds chunk i's sum, the running total
  // passes from lane to lane through readlane (register to register), and
  // the first lane whose prefix plus own sum passes the target is the chunk.
  auto locate = [&](const float* row) {
    if (nch <= kWave) {
      const float ri = lane < nch ? row[min(lane, nch - 1)] : 0.f;   // clamped: in bounds
      float acc = 0.f, run = 0.f;                 // acc: the prefix before this lane's chunk
      for (int j = 0; j < nch; ++j) {             // nch is wave-uniform
        if (lane == j) acc = run;
        run += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ri), j));
      }
      const float total = run;
      const float target = u * total;
      const uint64_t cross = __ballot(lane < nch && acc + ri > target);
      const uint64_t mass = __ballot(lane < nch && ri > 0.f);
      // rounding left no crossing: the last chunk with mass
      const int cstar = cross ? __builtin_ctzll(cross) : mass ? 63 - __builtin_clzll(mass) : -1;
      // without a crossing the prefix is the whole total, as in the serial scan
      const float carry =
          cross ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), cstar)) : total;
      if (lane == 0) {
        s_total = total;
        s_chunk = cstar;
        s_carry = carry;
        s_target = target;
      }
    } else if (lane == 0) {
      float total = 0.f;
      for (int i = 0; i < nch; ++i) total += row[i];
      const float target = u * total;
      float acc = 0.f;
      int cstar = -1;
      for (int i = 0; i < nch; ++i) {
        if (acc + row[i] > target) { cstar = i; break; }
        acc += row[i];
      }
      if (cstar < 0)                  // rounding left no crossing: last chunk with mass
        for (int i = nch - 1; i >= 0; --i)
          if (row[i] > 0.f) { cstar = i; break; }
      s_total = total;
      s_chunk = cstar;
      s_carry = acc;
      s_target = target;
    }
  };
  if (wave == 0) locate(in_lds ? cs_l : cs);
  __syncthreads();
  int use = 0;
  if (k < N && s_total == 0.f) {
    // Empty residual at a rejection (possible only through rounding): the
    // chunk sums of p_k, computed here with the same scan.
    use = 1;
    for (int c = 0; c < nch; ++c) {
      float w[kDrawPer], pre[kDrawPer];
      draw_weights<VEC>(dp, a.V, c, w);
      chunk_scan(w, pre, wave_tot);
      if (tid == kDrawThreads - 1) cs[nch + c] = pre[kDrawPer - 1];
      __syncthreads();
    }
    __threadfence_block();
    __syncthreads();
    if (wave == 0) locate(cs + nch);
    __syncthreads();
  }

  // The crossing inside chunk s_chunk: the first weight whose running sum
  // exceeds u * total (or the last positive weight if rounding left none).
  const int cstar = s_chunk;
  int y = -1;
  if (cstar >= 0) {
    const float* row = (use == 0 && in_lds) ? cs_l : cs + (size_t)use * nch;
    const float carry = s_carry, target = s_target;
    const bool last_mass = !(carry + row[cstar] > target);
    float w[kDrawPer], pre[kDrawPer];
    draw_weights<VEC>(use ? dp : dr, a.V, cstar, w);
    chunk_scan(w, pre, wave_tot);
    int pick = -1;
    if (!last_mass) {
#pragma unroll
      for (int e = kDrawPer - 1; e >= 0; --e)
        if (carry + pre[e] > target) pick = e;
    } else {
#pragma unroll
      for (int e = 0; e < kDrawPer; ++e)
        if (w[e] > 0.f) pick = e;
    }
    const int tok = pick < 0 ? -1 : cstar * kDrawChunk + tid * kDrawPer + pick;
    const uint64_t ballot = __ballot(pick >= 0);
    int src = 0;
    if (ballot) src = last_mass ? 63 - __builtin_clzll(ballot) : __builtin_ctzll(ballot);
    const int wtok = __builtin_amdgcn_readlane(tok, src);   // src: wave-uniform
    if (lane == 0) wave_hit[wave] = ballot ? wtok : -1;
    __syncthreads();
    // every wave: the first (or, for the last positive weight, the last) wave
    // with a hit, from one ballot over the wave results
    const int h = lane < kDrawThreads / kWave ? wave_hit[lane] : -1;
    const uint64_t hits = __ballot(h >= 0);
    if (hits)
      y = __builtin_amdgcn_readlane(h, last_mass ? 63 - __builtin_clzll(hits) : __builtin_ctzll(hits));
  }

  // Emit x_0..x_{k-1}, y, then -1.
  if (tid <= N) {
    int v = -1;
    if (tid < k) v = a.tokens[(size_t)b * N + tid];
    else if (tid == k) v = y;
    a.out[(size_t)b * (N + 1) + tid] = v;
  }
  if (tid == 0) a.num_acc[b] = k;
}

ChainPlan plan_chain(int B, int N, int V) {
  ChainPlan p{};
  p.rows_per_seq = 2 * N + 1;
  p.chunk = kStatsChunk;
  p.nchunks = (V + kStatsChunk - 1) / kStatsChunk;
  p.dchunks = (V + kDrawChunk - 1) / kDrawChunk;
  p.cpb = (size_t)B * p.dchunks <= kDrawResident ? 1 : kDrawCpbLarge;
  p.stats_bytes = align256((size_t)B * p.rows_per_seq * p.nchunks * sizeof(float2));
  p.csum_bytes = align256((size_t)B * 2 * p.dchunks * sizeof(float));
  p.decision_bytes = align256((size_t)B * 2 * sizeof(float4));
  p.total_bytes = p.stats_bytes + p.csum_bytes + p.decision_bytes;
  return p;
}

hipError_t launch_chain(const ChainPlan& p, const float* target, const float* draft,
                        const int32_t* tokens, const float* u_acc, const float* u_draw,
                        float temperature, int32_t* num_acc, int32_t* out, int B, int N, int V,
                        void* workspace, hipStream_t st) {
  ChainArgs a;
  a.target = target; a.draft = draft; a.tokens = tokens; a.u_acc = u_acc; a.u_draw = u_draw;
  a.num_acc = num_acc; a.out = out;
  a.stats = (float2*)workspace;
  a.csum = (float*)((char*)workspace + p.stats_bytes);
  a.decision = (float4*)((char*)workspace + p.stats_bytes + p.csum_bytes);
  a.decision_q = a.decision + B;
  a.B = B; a.N = N; a.V = V; a.chunk = p.chunk; a.nchunks = p.nchunks; a.dchunks = p.dchunks;
  a.c2 = kLog2e / temperature;
  const bool vec4 = (V % 4 == 0) && ((uintptr_t)target % 16 == 0) &&
                    (N == 0 || (uintptr_t)draft % 16 == 0);
  const dim3 g1(p.nchunks, B * p.rows_per_seq);
  const bool stream = (size_t)B * p.rows_per_seq * V * sizeof(float) > kCachedLogitBytes;
  if (vec4 && stream) chain_stats_kernel<4, true><<<g1, kStatsThreads, 0, st>>>(a);
  else if (vec4) chain_stats_kernel<4, false><<<g1, kStatsThreads, 0, st>>>(a);
  else chain_stats_kernel<1, false><<<g1, kStatsThreads, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int cpb = p.cpb == 1 ? 1 : vec4 ? kDrawCpbLarge : kDrawCpbScalar;
  const dim3 g2((p.dchunks + cpb - 1) / cpb, B);
  if (cpb == 1) {
    if (vec4) chain_chunks_kernel<4, 1><<<g2, kDrawThreads, 0, st>>>(a);
    else chain_chunks_kernel<1, 1><<<g2, kDrawThreads, 0, st>>>(a);
  } else {
    if (vec4) chain_chunks_kernel<4, kDrawCpbLarge><<<g2, kDrawThreads, 0, st>>>(a);
    else chain_chunks_kernel<1, kDrawCpbScalar><<<g2, kDrawThreads, 0, st>>>(a);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (vec4) chain_select_kernel<4><<<B, kDrawThreads, 0, st>>>(a);
  else chain_select_kernel<1><<<B, kDrawThreads, 0, st>>>(a);
  return hipGetLastError();
}

// ---- scratch of the allocation-free entry point --------------------------------
// spec_accept_chain_noalloc runs the kernels above with their workspace in
// this array.  Each GPU the library runs on holds its own copy until the
// process ends, and every call on that GPU shares it.  Nothing in it needs
// clearing: every kernel writes what it later reads within one call.  Host
// code never passes the array's name to a kernel (on the host it is only a
// stand-in for the symbol); chain_scratch gives its device address.
static __device__ __align__(256) unsigned char scratch[kChainScratchBytes];

// The device address of the scratch array on the GPU that runs `st` (the
// current device for the null stream), looked up once per device with that
// device current and kept.
hipError_t chain_scratch(hipStream_t st, void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxScratchDevices] = {};
  int dev = 0;
  hipError_t e = st != nullptr ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t back = hipSetDevice(cur);
      if (e == hipSuccess) e = back;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace sv
