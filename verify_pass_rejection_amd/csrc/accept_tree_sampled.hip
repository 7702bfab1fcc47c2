// Sampled (non-greedy) acceptance of a draft tree.
//
// "LLM Primer VI — Chapitre 9 — Décodage spéculatif", §9.1: a draft x is kept
// with probability min(1, p(x)/q(x)); otherwise the committed token is drawn
// from the normalised (p − q)+, which keeps the output distributed as the
// target's own sampling.  §9.2: the target picks among several draft paths (an
// EAGLE-2 tree).  A node's children are several candidates for the same
// position, drawn independently from that node's draft distribution q; they
// are tried in increasing id order, each against the residual that the
// rejections before it leave; when none is kept (or the node is a leaf) the
// token is drawn from that residual.
//
// Two kernels:
//  stree_stats — the whole chip, once over the logits: per 8192-logit chunk
//                of every target row, and of the draft row of every node with
//                children, the maximum and Σ 2^((z − max)·log2e/τ);
//  stree_walk  — one block per sequence (1024 threads for V <= 32768, else
//                512).  It merges the chunk statistics of every node and
//                gathers, for every node, p and q of its parent at its own
//                token, so a ratio test is a few LDS reads.  A node's rows are read only when a rejection
//                there needs the residual mass, or for the final draw: after j
//                rejections the residual is (p − c_j q)+ / Z_j, with c_0 = 0,
//                Z_0 = 1, c_{j+1} = c_j + Z_j and Z_{j+1} = Σ_v (p(v) −
//                c_{j+1} q(v))+ (one pass per rejection).  For V <= 32768 the
//                rows, once read, stay on chip while the node is visited: the
//                target row in registers (up to 32 tokens per thread), the
//                draft row in LDS, thread t holding the float4 groups t,
//                t + 1024, ... (coalesced loads).  The draw then takes the
//                block totals of the 4096-token segments to find the segment
//                holding the crossing, one block scan inside it to find the
//                thread, and that thread's four tokens to find the token.
//                For larger V the rows are streamed: each thread sums a
//                contiguous chunk, a block scan gives every chunk its
//                starting mass, each thread looks for the crossing in its own
//                chunk and a block minimum picks the token.
// Every reduction runs in a fixed order and leaves the same value in every
// thread, so the walk's control flow is uniform without broadcasts.
//
// Precision: the probabilities a ratio test reads come from the hardware exp2
// on an exact float64 argument split (2^a = 2^n · 2^f, n integer, |f| ≤ 1/2),
// within about 2 ulp of float32; the row sums (normalisers, residual masses,
// the draw) take float32 arguments (e_bulk); every sum, ratio and comparison
// is float64.

#include "common.h"

// Products are rounded before they are subtracted: with q = p (identical rows)
// the residual p − c q must cancel to exactly zero, which a fused multiply-add
// of an unrounded c·q against the rounded p does not give.
#pragma clang fp contract(off)

namespace sv {

struct STreeArgs {
  const float* target;     // [B, T, V]
  const float* draft;      // [B, T, V]
  const int32_t* tokens;   // [B, T]
  const int32_t* parents;  // [B, T]
  const float* u_accept;   // [B, T]
  const float* u_draw;     // [B, T]
  int32_t* accept_len;     // [B]
  int32_t* path;           // [B, T]
  int32_t* out;            // [B, T]
  float* part_m;           // [2, B*T, nchunks] chunk maxima (target rows, then draft rows)
  double* part_s;          // [2, B*T, nchunks] chunk sums
  float2* gz;              // [B*T] node i: target and draft logit of its parent at its token
  int B, T, V, nchunks;
  double k2;               // log2(e) / temperature
  float k2f;               // the same, rounded to float32
};

typedef float f32x4_t __attribute__((ext_vector_type(4)));
// Word 3 of a raw buffer resource on gfx9-family parts: 32-bit data format,
// no swizzle; with stride 0 a read past num_records returns 0.
constexpr int kBufferWord3 = 0x00020000;

constexpr int kSTThreads = 512;                // statistics; the streaming walk
constexpr int kSTWaves = kSTThreads / kWave;
constexpr int kSTWalkCached = 1024;            // the walk with rows on chip (V <= 32768)
constexpr int kSTMergeChunks = 8;              // rows of up to 8 chunks: straight-line merge
constexpr int kSTChunk = 8192;                 // logits per statistics block

// 2^a for a <= 0 (0 below the double range, or for z = -inf); branch-free.
__device__ __forceinline__ double exp2_split(double a) {
  const double ac = fmax(a, -1020.0);          // also maps -inf to a finite value
  const double n = rint(ac);
  const float f = (float)(ac - n);
  const double r = ldexp((double)__builtin_amdgcn_exp2f(f), (int)n);
  return a > -1020.0 ? r : 0.0;
}

// e(v) = 2^((z(v) − m)·k2) for the tokens a ratio test reads: float64
// argument, float32 result (exact but below float32's range: 2^f is a float32
// and 2^n a power of two), within about 2 ulp.
__device__ __forceinline__ double e_of(float z, float m, double k2) {
  return (double)(float)exp2_split(((double)z - m) * k2);
}
// The same for the sums over a whole row (normalisers, residual masses, the
// draw): float32 argument and hardware exp2.  The argument's rounding adds
// |a|·2^-24 (relative) to a term 2^a; a term with |a| >= 16 is below 2^-16 of
// the row's largest, so the mass-weighted error of a sum stays below about
// 1e-6 for V <= 2^20.
__device__ __forceinline__ float e_bulk(float z, float m, float k2f) {
  return __builtin_amdgcn_exp2f((z - m) * k2f);
}

// Block reductions: fixed order, the same result in every thread.
template <int NW>
__device__ __forceinline__ double block_sum(double x, double* red) {
  x = wave_sum(x);
  __syncthreads();                       // red is free again
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int w = 0; w < NW; ++w) s += red[w];
  return s;
}
template <int NW>
__device__ __forceinline__ float block_max(float x, float* redf) {
  x = wave_max(x);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) redf[threadIdx.x >> 6] = x;
  __syncthreads();
  float m = redf[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) m = fmaxf(m, redf[w]);
  return m;
}
template <int NW>
__device__ __forceinline__ int block_min(int x, int* redi) {
  x = wave_min(x);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) redi[threadIdx.x >> 6] = x;
  __syncthreads();
  int m = redi[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) m = min(m, redi[w]);
  return m;
}

// Marks cached row registers as rewritten, so that values derived from them
// (float64 conversions, products) are recomputed in the pass that follows
// instead of being kept alive across passes: the row already takes CH
// registers, its float64 image would take 2·CH more.
template <int N>
__device__ __forceinline__ void launder(float (&r)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(r[i]));
}

// ---------------------------------------------------------------------------
// stree_stats: block (chunk, row): that chunk of the node's target row and,
// when the node has children, of its draft row (no other draft row is ever
// used).  Whether it has children is read (one parent per thread, a block OR)
// while the target chunk's loads are in flight.  The two chunks' maxima are
// reduced side by side, then their sums, so a node with children costs one
// pair of barriers per reduction, as a leaf does.  A child whose token falls
// in the chunk copies its parent's two logits at that token into gz, so that
// the walk reads them with its other set-up loads instead of gathering them
// after the parents arrive.  16-byte loads when VEC, with indices clamped into
// the row, so every load is issued before the first use.  Ordinary (cached)
// loads: the walk reads the rows of the visited nodes again right after this
// pass, and finds them in the last-level cache.
// ---------------------------------------------------------------------------
template <bool VEC>
__global__ __launch_bounds__(kSTThreads) void stree_stats_kernel(STreeArgs a) {
  __shared__ double red[2 * kSTWaves];
  __shared__ float redf[2 * kSTWaves];
  const int ch = blockIdx.x, row = blockIdx.y;
  const int b = row / a.T, node = row % a.T;
  const int begin = ch * kSTChunk, end = min(a.V, begin + kSTChunk);
  constexpr int PER = kSTChunk / kSTThreads;
  auto load = [&](const float* z, float (&x)[PER]) __attribute__((always_inline)) {
    if constexpr (VEC) {                         // V % 4 == 0: a group is wholly in or out
#pragma unroll
      for (int k = 0; k < PER / 4; ++k) {
        const int v = begin + (k * kSTThreads + threadIdx.x) * 4;
        const f32x4_t y = *(const f32x4_t*)(z + min(v, a.V - 4));
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * k + e] = v < end ? y[e] : -__builtin_huge_valf();
      }
    } else {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int v = begin + i * kSTThreads + threadIdx.x;
        const float y = z[min(v, a.V - 1)];
        x[i] = v < end ? y : -__builtin_huge_valf();
      }
    }
  };
  // the chunk's maximum and Σ e: groups of four terms in float32 (at most 3
  // roundings), groups in float64; a chunk of -inf logits (a masked
  // vocabulary range) has no mass: its maximum stays -inf and its sum 0,
  // which the walk's merge weighs 0
  auto local_max = [&](const float (&x)[PER]) __attribute__((always_inline)) {
    float mx = x[0];
#pragma unroll
    for (int i = 1; i < PER; ++i) mx = fmaxf(mx, x[i]);
    return mx;
  };
  auto local_sum = [&](const float (&x)[PER], float mx) __attribute__((always_inline)) {
    double s = 0.0;
    if (mx != -__builtin_huge_valf()) {
#pragma unroll
      for (int i = 0; i < PER; i += 4)
        s += (double)((e_bulk(x[i], mx, a.k2f) + e_bulk(x[i + 1], mx, a.k2f)) +
                      (e_bulk(x[i + 2], mx, a.k2f) + e_bulk(x[i + 3], mx, a.k2f)));
    }
    return s;
  };
  auto store = [&](int kind, float mx, double s) __attribute__((always_inline)) {
    if (threadIdx.x == 0) {
      const size_t o = ((size_t)kind * a.B * a.T + row) * a.nchunks + ch;
      a.part_m[o] = mx;
      a.part_s[o] = s;
    }
  };
  // Block reductions of one value, or of the target and draft chunks' values
  // side by side (one pair of barriers for both; each value is reduced in the
  // same order either way).
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  auto block_max2 = [&](float& u, float& v) __attribute__((always_inline)) {
    u = wave_max(u);
    v = wave_max(v);
    __syncthreads();
    if (lane == 0) { redf[wave] = u; redf[kSTWaves + wave] = v; }
    __syncthreads();
    u = redf[0];
    v = redf[kSTWaves];
#pragma unroll
    for (int w = 1; w < kSTWaves; ++w) { u = fmaxf(u, redf[w]); v = fmaxf(v, redf[kSTWaves + w]); }
  };
  auto block_sum2 = [&](double& u, double& v) __attribute__((always_inline)) {
    u = wave_sum(u);
    v = wave_sum(v);
    __syncthreads();
    if (lane == 0) { red[wave] = u; red[kSTWaves + wave] = v; }
    __syncthreads();
    double su = 0.0, sv = 0.0;
#pragma unroll
    for (int w = 0; w < kSTWaves; ++w) { su += red[w]; sv += red[kSTWaves + w]; }
    u = su;
    v = sv;
  };
  float x[PER], y[PER];
  load(a.target + (size_t)row * a.V, x);
  const int i = threadIdx.x;
  const size_t ci = (size_t)b * a.T + min(i, a.T - 1);
  const int ipar = a.parents[ci], itok = a.tokens[ci];
  const bool mine = i > node && i < a.T && ipar == node;
  if (mine && itok >= begin && itok < end) {
    const size_t r = (size_t)row * a.V + itok;
    a.gz[ci] = make_float2(a.target[r], a.draft[r]);
  }
  const bool kids = __syncthreads_or(mine);    // uniform
  if (kids) {
    // both chunks: maxima side by side, then sums side by side
    load(a.draft + (size_t)row * a.V, y);
    float mx = local_max(x), my = local_max(y);
    block_max2(mx, my);
    double sx = local_sum(x, mx), sy = local_sum(y, my);
    block_sum2(sx, sy);
    store(0, mx, sx);
    store(1, my, sy);
  } else {
    float mx = local_max(x);
    mx = block_max<kSTWaves>(mx, redf);
    double sx = local_sum(x, mx);
    sx = block_sum<kSTWaves>(sx, red);
    store(0, mx, sx);
  }
}

// ---------------------------------------------------------------------------
// stree_walk, NT threads.  CH > 0: V <= NT·CH, a visited node's rows are read
// once, one row at a time with every load in flight (buffer loads; 16 bytes
// each when VEC), into registers (target) and LDS (draft: group k of this
// thread, elements 4k .. 4k + 3, at float4 k·NT + tid, read with 16-byte LDS
// reads); element i = 4k + e is token 4·(tid + NT·k) + e.  CH = 0: any V, every pass streams the rows from memory.
// With the rows on chip, 1024 threads (32 tokens each at V = 32768) halve
// each thread's share of the residual passes, the draw's sums and the
// exponentials against 512 threads (64 tokens each): call 57.4 -> 55.3 us
// (eagle2 tree), 95.1 -> 91.5 us (medusa tree).
// ---------------------------------------------------------------------------
template <int CH, bool VEC, int NT>
__global__ __launch_bounds__(NT) void stree_walk_kernel(STreeArgs a) {
  constexpr int NW = NT / kWave;
  constexpr bool CACHED = CH > 0;
  __shared__ int spar[64], stok[64], spath[65], shas[64];
  __shared__ float sua[64];
  __shared__ float nm_p[64], nm_q[64];       // every node's row maxima
  __shared__ double ni_p[64], ni_q[64];      // and 1 / Σ e
  __shared__ double ge_p[64], ge_q[64];      // e of node i's token in its parent's rows
  __shared__ __attribute__((aligned(16))) float lq[CACHED ? CH * NT : 4];
  __shared__ double red2[CACHED ? (CH / 4) * NW : 1];   // segment totals per wave
  __shared__ double segS[CACHED ? CH / 4 : 1];                 // and per block
  __shared__ double red[NW];
  __shared__ int redi[NW];

  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int T = a.T, V = a.V;
  const double k2 = a.k2;
  // Set-up loads, all issued at once before the first barrier: the node's
  // parent, token, uniform and the two logits of its parent at its token,
  // which the statistics pass copied (threads 0..T-1; an entry is written for
  // exactly the nodes that use it below); every chunk statistic of the target
  // row (threads 0..T-1) or draft row (threads 64..64+T-1) of node tid % 64,
  // the latter also for childless nodes, whose entries are never written and
  // never used.
  int pa0 = -1, x0 = -1;
  float ua0 = 0.f;
  float2 gz = make_float2(0.f, 0.f);
  if (tid < T) {
    pa0 = a.parents[(size_t)b * T + tid];
    x0 = a.tokens[(size_t)b * T + tid];
    ua0 = a.u_accept[(size_t)b * T + tid];
    gz = a.gz[(size_t)b * T + tid];
  }
  float pm[kSTMergeChunks];
  double ps[kSTMergeChunks];
  if ((tid & 63) < T && tid < 128 && a.nchunks <= kSTMergeChunks) {
    const size_t base0 = ((size_t)(tid >> 6) * a.B * T + (size_t)b * T + (tid & 63)) * a.nchunks;
#pragma unroll
    for (int c = 0; c < kSTMergeChunks; ++c) {
      const int cc = min(c, a.nchunks - 1);     // past the last chunk: re-read it, not summed
      pm[c] = a.part_m[base0 + cc];
      ps[c] = a.part_s[base0 + cc];
    }
  }
  const bool gth = tid < T && tid >= 1 && pa0 >= 0 && pa0 < tid && x0 >= 0 && x0 < V;
  if (tid < 64) shas[tid] = 0;
  __syncthreads();
  if (tid < T) {
    const int pa = pa0;
    spar[tid] = pa;
    stok[tid] = x0;
    sua[tid] = ua0;
    if (tid >= 1 && pa >= 0 && pa < tid) shas[pa] = 1;     // pa has a child
  }
  __syncthreads();
  // Merge the chunk statistics of every row (target rows by threads 0..T-1,
  // draft rows by 64..64+T-1); a draft row without statistics is never used.
  if ((tid & 63) < T && tid < 128) {
    const int kind = tid >> 6, node = tid & 63;
    const size_t base = ((size_t)kind * a.B * T + (size_t)b * T + node) * a.nchunks;
    const bool has_row = kind == 0 || shas[node] != 0;
    float m = 0.f;
    double inv = 1.0;
    if (has_row) {
      double s = 0.0;
      if (a.nchunks <= kSTMergeChunks) {
        m = pm[0];
#pragma unroll
        for (int c = 1; c < kSTMergeChunks; ++c) m = fmaxf(m, pm[c]);
#pragma unroll
        for (int c = 0; c < kSTMergeChunks; ++c)
          if (c < a.nchunks) s += ps[c] * exp2_split(((double)pm[c] - m) * k2);
      } else {
        m = a.part_m[base];
        for (int c = 1; c < a.nchunks; ++c) m = fmaxf(m, a.part_m[base + c]);
        for (int c = 0; c < a.nchunks; ++c)
          s += a.part_s[base + c] * exp2_split(((double)a.part_m[base + c] - m) * k2);
      }
      inv = 1.0 / s;
    }
    if (kind == 0) { nm_p[node] = m; ni_p[node] = inv; }
    else { nm_q[node] = m; ni_q[node] = inv; }
  }
  __syncthreads();
  // e at every node's own token in its parent's target and draft rows.
  if (tid < T) {
    ge_p[tid] = gth ? e_of(gz.x, nm_p[pa0], k2) : 0.0;
    ge_q[tid] = gth ? e_of(gz.y, nm_q[pa0], k2) : 0.0;
  }
  __syncthreads();
  // lane i of every wave stands for node i: the same masks in every wave
  const int my_par = lane < T ? spar[lane] : -1;
  const bool my_ok = lane >= 1 && lane < T && my_par >= 0 && my_par < lane;

  // Streaming: this thread's tokens j0 .. j1 - 1 (ascending, contiguous).
  const int chs = (V + NT - 1) / NT;
  const int j0 = min(V, tid * chs), j1 = min(V, j0 + chs);
  // Cached: element i = 4k + e of this thread is token 4·(tid + NT·k) + e, so
  // that a wave's float4 loads cover 1 KB of consecutive tokens; segment k
  // (elements 4k .. 4k + 3 of every thread) is tokens 4·NT·k .. 4·NT·(k+1) − 1.
  auto tok = [&](int i) -> int { return 4 * (tid + NT * (i >> 2)) + (i & 3); };

  float rp[CACHED ? CH : 1];
  // The draft row in LDS: group k (elements 4k .. 4k + 3) of this thread at
  // float4 k·NT + tid, so a wave's groups are 1 KB contiguous, as one
  // direct-to-LDS load writes them, and are read with 16-byte LDS reads.
  typedef __attribute__((address_space(3))) f32x4_t lds_f4;
  auto q4 = [&](int k) -> lds_f4& { return ((lds_f4*)lq)[k * NT + tid]; };
  int n = 0, depth = 0;
  if (tid == 0) spath[0] = 0;
  double c = 0.0, Z = 1.0;
  const float* zt = nullptr;
  const float* zq = nullptr;
  float mp = 0.f, mq = 0.f;
  double ip = 1.0, iq = 1.0;
  float ipf = 1.f, iqf = 1.f, cf = 0.f;

  // Reads the current node's rows as e values (cached path); the draft row
  // only when `both`.
  auto load_rows = [&](bool both_in) {
    if constexpr (CACHED) {
      // wave-uniform: one branch around the draft row's loads and
      // exponentials, not one per token
      const bool both = __builtin_amdgcn_readfirstlane((int)both_in) != 0;
      // Buffer loads: the row's base in SGPRs, the lane's offset in one VGPR
      // and each segment's offset in an SGPR (global loads would need an
      // address pair per segment); reads past the row return 0 and are
      // replaced by -inf below.
      const __amdgpu_buffer_rsrc_t rt = __builtin_amdgcn_make_buffer_rsrc(
          (void*)zt, (short)0, V * (int)sizeof(float), kBufferWord3);
      const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
          (void*)zq, (short)0, V * (int)sizeof(float), kBufferWord3);
      // A whole row into d: every load issued before the first use.  With 16-
      // byte loads the loaded groups pass through one empty asm statement that
      // takes them all, so the compiler cannot interleave a group's use with the
      // next group's load (at the 128-register limit it did, leaving one load in
      // flight at a time).
      auto load_row = [&](__amdgpu_buffer_rsrc_t r, float (&d)[CH]) __attribute__((always_inline)) {
        if constexpr (VEC) {                      // V % 4 == 0: a group is wholly in or out
          f32x4_t x[CH / 4];
#pragma unroll
          for (int k = 0; k < CH / 4; ++k)
            // cast the whole vector: a bit cast of one element of it reads element 0
            x[k] = __builtin_bit_cast(
                f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, 16 * tid, NT * 16 * k, 0));
          static_assert(CH == 16 || CH == 32, "row groups per thread");
          if constexpr (CH == 16) {
            asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]));
          } else {
            asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]),
                         "+v"(x[5]), "+v"(x[6]), "+v"(x[7]));
          }
#pragma unroll
          for (int k = 0; k < CH / 4; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e) d[4 * k + e] = x[k][e];
        } else {
#pragma unroll
          for (int k = 0; k < CH / 4; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              d[4 * k + e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                           r, 16 * tid + 4 * e, NT * 16 * k, 0));
        }
#pragma unroll
        for (int i = 0; i < CH; ++i)
          if (tok(i) >= V) d[i] = -__builtin_huge_valf();
      };
      // One row at a time, all of its loads in flight: with both rows' loads
      // outstanding together the compiler ran out of registers and waited for
      // each draft-row load before issuing the next (walk 38.9 -> 46.7 us on
      // the eagle2 tree, 64 tokens per thread).  The rows are kept normalised,
      // p = e·(1/Z_p) and q = e·(1/Z_q) in float32 (the products every pass
      // and the draw would otherwise form again); the draft row is formed in
      // registers and stored to LDS once.
      load_row(rt, rp);
#pragma unroll
      for (int i = 0; i < CH; ++i) rp[i] = e_bulk(rp[i], mp, a.k2f) * ipf;
      if (both) {
        float y[CH];
        load_row(rq, y);
#pragma unroll
        for (int k = 0; k < CH / 4; ++k) {
          f32x4_t q;
#pragma unroll
          for (int e = 0; e < 4; ++e) q[e] = e_bulk(y[4 * k + e], mq, a.k2f) * iqf;
          q4(k) = q;
        }
      }
    }
  };
  // residual weight (p − c q)+ of element i (cached: float32 terms of the
  // normalised rows; q = p and c = 1 still cancel exactly) or of token v
  // (streaming)
  // the four weights of group k (cached path)
  auto res4 = [&](int k, float (&r)[4]) {
    const f32x4_t q = q4(k);
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = fmaxf(rp[4 * k + e] - cf * q[e], 0.f);
  };
  auto res_s = [&](int v) -> double {
    return fmax((double)e_bulk(zt[v], mp, a.k2f) * ip -
                c * ((double)e_bulk(zq[v], mq, a.k2f) * iq), 0.0);
  };

  bool loaded = false;
  while (true) {
    const uint64_t kids = __ballot(my_ok && my_par == n);
    zt = a.target + ((size_t)b * T + n) * V;
    zq = a.draft + ((size_t)b * T + n) * V;
    mp = nm_p[n]; ip = ni_p[n]; mq = nm_q[n]; iq = ni_q[n];
    ipf = (float)ip; iqf = (float)iq;
    loaded = false;
    c = 0.0;
    Z = 1.0;
    int kept = -1;
    for (uint64_t k = kids; k != 0; k &= k - 1) {
      const int ch = __builtin_ctzll(k);
      const int x = stok[ch];
      double r = 0.0;
      if (x >= 0 && x < V) {
        const double px = ge_p[ch] * ip, qx = ge_q[ch] * iq;
        const double w = fmax(px - c * qx, 0.0);
        r = qx > 0.0 ? w / (Z * qx) : (w > 0.0 ? __builtin_huge_val() : 0.0);
      }
      if ((double)sua[ch] < r) {
        kept = ch;
        break;
      }
      // rejected: the residual moves on to (p − (c + Z) q)+
      c += Z;
      double s = 0.0;
      if constexpr (CACHED) {
        if (!loaded) { load_rows(true); loaded = true; }
        launder(rp);
        cf = (float)c;
        // groups of four terms in float32, groups in float64
#pragma unroll
        for (int k = 0; k < CH / 4; ++k) {
          float r[4];
          res4(k, r);
          s += (double)((r[0] + r[1]) + (r[2] + r[3]));
        }
      } else {
        for (int v = tid; v < V; v += NT) s += res_s(v);
      }
      Z = block_sum<NW>(s, red);
      if (!(Z > 0.0)) { c = 0.0; Z = 1.0; }    // an empty residual falls back to p
    }
    if (kept < 0) break;
    ++depth;
    if (tid == 0) spath[depth] = kept;
    n = kept;
  }

  // Draw from w = (p − c q)+ (p itself when c = 0) with u_draw[b][n]: the
  // first token with positive weight whose running mass exceeds u·(total).
  if constexpr (CACHED) {
    if (!loaded) load_rows(c != 0.0);            // only c != 0 needs the draft row
  }
  cf = (float)c;
  const double u = (double)a.u_draw[(size_t)b * T + n];
  // c = 0 (p itself) or not: one wave-uniform branch for the whole draw
  const bool pure = __builtin_amdgcn_readfirstlane((int)(c == 0.0)) != 0;

  // Cached rows: the block totals of the 4·NT-token segments locate the
  // segment holding the crossing; one block scan inside it locates the
  // thread, and that thread's four tokens the token.
  auto draw_cached = [&](auto pure_tag) -> int {
    constexpr bool P = decltype(pure_tag)::value;
    constexpr int K = CACHED ? CH / 4 : 1;
    // The weights, once, in place of the row (which the walk no longer needs):
    // the segment sums, the scan and the search below read them from registers.
    if constexpr (!P) {
#pragma unroll
      for (int k = 0; k < CH / 4; ++k) {
        float r[4];
        res4(k, r);
#pragma unroll
        for (int e = 0; e < 4; ++e) rp[4 * k + e] = r[e];
      }
    }
    auto w = [&](int i) -> double { return (double)rp[i]; };
    auto quad = [&](int k) -> double {          // this thread's four tokens of segment k
      return ((w(4 * k) + w(4 * k + 1)) + w(4 * k + 2)) + w(4 * k + 3);
    };
    // The wave's total of every segment: K sums per lane, halved at each step
    // (a lane keeps half of the segments and adds its partner's share of
    // them: partners lane ^ 32, lane ^ 16, lane ^ 8), then a sum over the
    // 64 / K lanes left holding the same segment: lane L ends with segment
    // L / (64 / K).  Lane exchanges by row swaps and DPP, not LDS.
    constexpr int LOGK = K == 8 ? 3 : K == 4 ? 2 : K == 2 ? 1 : 0;
    static_assert((1 << LOGK) == K && K <= 8, "segments per lane");
    launder(rp);
    double v[K];
#pragma unroll
    for (int k = 0; k < K; ++k) v[k] = quad(k);
    if constexpr (LOGK >= 1) {
#pragma unroll
      for (int j = 0; j < K / 2; ++j) v[j] = swap_sum<true>(v[j], v[j + K / 2]);
    }
    if constexpr (LOGK >= 2) {
#pragma unroll
      for (int j = 0; j < K / 4; ++j) v[j] = swap_sum<false>(v[j], v[j + K / 4]);
    }
    if constexpr (LOGK >= 3) {
      const bool up = (lane & 8) != 0;
      const double keep = up ? v[1] : v[0], send = up ? v[0] : v[1];
      v[0] = keep + dpp_d<kDppXor8>(send);
    }
    if constexpr (64 / K >= 2) v[0] += dpp_d<kDppXor1>(v[0]);
    if constexpr (64 / K >= 4) v[0] += dpp_d<kDppXor2>(v[0]);
    if constexpr (64 / K >= 8) v[0] += dpp_d<kDppXor7>(v[0]);
    if constexpr (64 / K >= 16) v[0] += dpp_d<kDppXor15>(v[0]);
    if ((lane & (64 / K - 1)) == 0) red2[(tid >> 6) * K + lane / (64 / K)] = v[0];
    __syncthreads();
    if (tid < K) {                               // segment totals: the waves in order
      double t = 0.0;
#pragma unroll
      for (int w8 = 0; w8 < NW; ++w8) t += red2[w8 * K + tid];
      segS[tid] = t;
    }
    __syncthreads();
    double total = 0.0;
#pragma unroll
    for (int k = 0; k < K; ++k) total += segS[k];
    const double thr = u * total;
    int ks = -1;
    double pre = 0.0, pks = 0.0;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const double t = segS[k];
      if (ks < 0 && pre + t > thr) { ks = k; pks = pre; }
      pre += t;
    }
    ks = __builtin_amdgcn_readfirstlane(ks);
    if (ks < 0) return V;                        // a zero total: nothing to draw
    launder(rp);
    double mine = 0.0;
#pragma unroll
    for (int k = 0; k < K; ++k)
      if (k == ks) mine = quad(k);
    // exclusive scan of the threads' sums in segment ks: the wave, then the waves
    const double inc = wave_scan(mine);
    double ex = wave_prev(inc);
    if (lane == 63) red[tid >> 6] = inc;         // red's last readers are behind the barriers above
    __syncthreads();
    for (int w8 = 0; w8 < (tid >> 6); ++w8) ex += red[w8];
    launder(rp);
    double run = pks + ex;
    int cand = V, last = -1;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      if (k != ks) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double wi = w(4 * k + e);
        run += wi;
        if (cand == V && wi > 0.0 && run > thr) cand = tok(4 * k + e);
        if (wi > 0.0) last = tok(4 * k + e);
      }
    }
    int y = block_min<NW>(cand, redi);
    // Rounding can leave the scan's end of segment ks at or below thr although
    // the segment totals put the crossing inside it: then it is the segment's
    // last token with positive weight.
    if (y >= V) {
      const int lastpos = -block_min<NW>(-last, redi);
      y = lastpos >= 0 ? lastpos : V;
    }
    return y;
  };

  // Streaming: each thread sums its contiguous chunk, a block scan gives every
  // chunk its starting mass, each thread looks for the crossing in its own
  // chunk and a block minimum picks the token.
  auto draw_stream = [&](auto pure_tag) -> int {
    constexpr bool P = decltype(pure_tag)::value;
    auto w = [&](int v) -> double {
      return P ? (double)e_bulk(zt[v], mp, a.k2f) * ip : res_s(v);
    };
    double cs = 0.0;
    for (int v = j0; v < j1; ++v) cs += w(v);
    const double inc = wave_scan(cs);
    double ex = wave_prev(inc);
    __syncthreads();
    if (lane == 63) red[tid >> 6] = inc;
    __syncthreads();
    double base = 0.0;
    for (int v = 0; v < (tid >> 6); ++v) base += red[v];
    double total = 0.0;
#pragma unroll
    for (int v = 0; v < NW; ++v) total += red[v];
    ex += base;
    const double thr = u * total;
    // this chunk's first token with positive weight whose running mass passes thr
    int cand = V;
    double run = ex;
    for (int v = j0; v < j1; ++v) {
      const double wi = w(v);
      run += wi;
      if (wi > 0.0 && run > thr) { cand = v; break; }
    }
    return block_min<NW>(cand, redi);
  };

  int y;
  if constexpr (CACHED) y = pure ? draw_cached(std::true_type{}) : draw_cached(std::false_type{});
  else y = pure ? draw_stream(std::true_type{}) : draw_stream(std::false_type{});
  if (y >= V) y = V - 1;                      // nothing to draw (a zero total)

  __syncthreads();
  for (int i = tid; i < T; i += NT) {
    const size_t o = (size_t)b * T + i;
    a.path[o] = i <= depth ? spath[i] : -1;
    a.out[o] = i < depth ? stok[spath[i + 1]] : (i == depth ? y : -1);
  }
  if (tid == 0) a.accept_len[b] = depth;
}

STreePlan plan_tree_sampled(int B, int T, int V) {
  STreePlan p{};
  p.nchunks = (V + kSTChunk - 1) / kSTChunk;
  const size_t parts = (size_t)2 * B * T * p.nchunks;
  p.s_bytes = align256(parts * sizeof(double));
  p.m_bytes = align256(parts * sizeof(float));
  p.g_bytes = align256((size_t)B * T * sizeof(float2));
  p.total_bytes = p.s_bytes + p.m_bytes + p.g_bytes;
  return p;
}

hipError_t launch_tree_sampled(const STreePlan& p, const float* target, const float* draft,
                               const int32_t* tokens, const int32_t* parents,
                               const float* u_accept, const float* u_draw, float temperature,
                               int32_t* accept_len, int32_t* path, int32_t* out, int B, int T,
                               int V, void* workspace, hipStream_t st) {
  STreeArgs a;
  a.target = target; a.draft = draft; a.tokens = tokens; a.parents = parents;
  a.u_accept = u_accept; a.u_draw = u_draw;
  a.accept_len = accept_len; a.path = path; a.out = out;
  a.part_s = (double*)workspace;
  a.part_m = (float*)((char*)workspace + p.s_bytes);
  a.gz = (float2*)((char*)workspace + p.s_bytes + p.m_bytes);
  a.B = B; a.T = T; a.V = V; a.nchunks = p.nchunks;
  a.k2 = 1.4426950408889634 / (double)temperature;
  a.k2f = (float)a.k2;
  const bool vec = V % 4 == 0 && ((uintptr_t)target | (uintptr_t)draft) % 16 == 0;
  if (vec) stree_stats_kernel<true><<<dim3(p.nchunks, B * T), kSTThreads, 0, st>>>(a);
  else stree_stats_kernel<false><<<dim3(p.nchunks, B * T), kSTThreads, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid(B);
  constexpr int NT = kSTWalkCached;
  if (V <= NT * 16) {
    if (vec) stree_walk_kernel<16, true, NT><<<grid, NT, 0, st>>>(a);
    else stree_walk_kernel<16, false, NT><<<grid, NT, 0, st>>>(a);
  } else if (V <= NT * 32) {
    if (vec) stree_walk_kernel<32, true, NT><<<grid, NT, 0, st>>>(a);
    else stree_walk_kernel<32, false, NT><<<grid, NT, 0, st>>>(a);
  } else {
    stree_walk_kernel<0, false, kSTThreads><<<grid, kSTThreads, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace sv
