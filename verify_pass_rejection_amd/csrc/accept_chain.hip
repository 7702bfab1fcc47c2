// Chain acceptance by rejection sampling.
//
// "LLM Primer VI — Chapitre 9 — Décodage spéculatif", §9.1: draft x drawn from
// q is kept with probability min(1, p(x)/q(x)); at the first draft that is not
// kept, the target's own token is drawn from the normalised positive part of
// p − q and the rest is dropped; this leaves the output distributed exactly as
// pure target sampling.  The pass gives N+1 target distributions, so when all
// N drafts are kept the last one supplies a bonus token.
//
// Two kernels:
//  chain_stats  — one pass over every logit row (all B*(2N+1) rows), per chunk
//                 the row maximum and sum of 2^((z - max) log2(e)/tau);
//  chain_draw   — one block per sequence: merges the chunk statistics into
//                 each row's normaliser, runs the N ratio tests (two gathers a
//                 row), takes the first rejection k, then draws the committed
//                 token from row k only (the residual (p_k - q_k)+, or p_N):
//                 a first sweep computes chunk sums of the weights, a second
//                 re-scans the one chunk holding the crossing.  Only the drawn
//                 row pair is read a second time.
//
// Every row's ratio test depends on that row alone, so computing all of them
// and then taking the first rejection gives the same result as the
// sequential walk.

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
  int B, N, V, chunk, nchunks;
  float c2;              // log2(e) / temperature
};

constexpr int kStatsThreads = 256;
constexpr int kStatsChunk = 8192;     // logits per stats block
constexpr int kDrawThreads = 1024;
constexpr int kDrawPer = 4;           // weights per thread per draw chunk
constexpr int kDrawChunk = kDrawThreads * kDrawPer;
constexpr int kMaxDrawChunks = (1 << 24) / kDrawChunk;

__device__ __forceinline__ const float* chain_row(const ChainArgs& a, int b, int rho) {
  return rho <= a.N ? a.target + ((size_t)b * (a.N + 1) + rho) * a.V
                    : a.draft + ((size_t)b * a.N + (rho - a.N - 1)) * a.V;
}

// (m, s) pairs: s = sum 2^((z - m) c).
__device__ __forceinline__ void merge_ms(float& m, float& s, float m2, float s2, float c) {
  const float mx = fmaxf(m, m2);
  if (mx == kNegInf) return;
  s = s * fast_exp2((m - mx) * c) + s2 * fast_exp2((m2 - mx) * c);
  m = mx;
}

template <int VEC>
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
      if (j < a.V) x = *(const float4*)(z + j);   // V % 4 == 0 on this path
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
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(s, off);
    merge_ms(m, s, m2, s2, a.c2);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) { sm[wave] = m; ss[wave] = s; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float M = sm[0], S = ss[0];
    for (int w = 1; w < kStatsThreads / kWave; ++w) merge_ms(M, S, sm[w], ss[w], a.c2);
    a.stats[(size_t)row * a.nchunks + ch] = make_float2(M, S);
  }
}

// Weights of the drawn row: residual (p - q)+ or p alone.
struct DrawRow {
  const float* zp;
  const float* zq;   // nullptr: weights are p
  float mp, lp;      // row max and log2 of the sum for p
  float mq, lq;
  float c;
  __device__ __forceinline__ float w(float xp, float xq) const {
    const float p = fast_exp2((xp - mp) * c - lp);
    if (zq == nullptr) return p;
    const float q = fast_exp2((xq - mq) * c - lq);
    return fmaxf(p - q, 0.f);
  }
};

// Loads the kDrawPer weights of this thread in draw chunk `chunk`.
template <int VEC>
__device__ __forceinline__ void draw_weights(const DrawRow& r, int V, int chunk, float* w) {
  const int j0 = chunk * kDrawChunk + threadIdx.x * kDrawPer;
  float xp[kDrawPer], xq[kDrawPer];
  if constexpr (VEC == 4) {
    float4 p4 = {kNegInf, kNegInf, kNegInf, kNegInf}, q4 = p4;
    if (j0 < V) {
      p4 = *(const float4*)(r.zp + j0);
      if (r.zq) q4 = *(const float4*)(r.zq + j0);
    }
    xp[0] = p4.x; xp[1] = p4.y; xp[2] = p4.z; xp[3] = p4.w;
    xq[0] = q4.x; xq[1] = q4.y; xq[2] = q4.z; xq[3] = q4.w;
  } else {
#pragma unroll
    for (int e = 0; e < kDrawPer; ++e) {
      const int j = j0 + e;
      xp[e] = j < V ? r.zp[j] : kNegInf;
      xq[e] = (j < V && r.zq) ? r.zq[j] : kNegInf;
    }
  }
#pragma unroll
  for (int e = 0; e < kDrawPer; ++e) w[e] = (j0 + e < V) ? r.w(xp[e], xq[e]) : 0.f;
}

// Running sums inside one draw chunk, in a fixed order: the thread's own
// weights left to right, thread offsets from an inclusive wave scan and a
// sequential scan of the wave totals.  prefix[e] is the running sum up to and
// including weight e of this thread; the chunk total is prefix[kDrawPer-1] of
// the last thread, so re-running the same scan reproduces it bit for bit.
__device__ __forceinline__ void chunk_scan(const float* w, float* prefix, float* wave_tot,
                                           float* wave_off) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float local[kDrawPer];
  local[0] = w[0];
#pragma unroll
  for (int e = 1; e < kDrawPer; ++e) local[e] = local[e - 1] + w[e];
  float incl = local[kDrawPer - 1];
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const float y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  float excl = __shfl_up(incl, 1);
  if (lane == 0) excl = 0.f;
  if (lane == kWave - 1) wave_tot[wave] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    float acc = 0.f;
    for (int i = 0; i < kDrawThreads / kWave; ++i) { wave_off[i] = acc; acc += wave_tot[i]; }
  }
  __syncthreads();
  const float off = wave_off[wave] + excl;
#pragma unroll
  for (int e = 0; e < kDrawPer; ++e) prefix[e] = off + local[e];
}

template <int VEC>
__global__ __launch_bounds__(kDrawThreads) void chain_draw_kernel(ChainArgs a) {
  __shared__ float row_m[128], row_l[128];     // per row: max, log2(sum)
  __shared__ float ratio_ok[64];
  __shared__ float csum[kMaxDrawChunks];
  __shared__ float wave_tot[kDrawThreads / kWave], wave_off[kDrawThreads / kWave];
  __shared__ int wave_hit[kDrawThreads / kWave];
  __shared__ int s_k, s_chunk, s_y;
  __shared__ float s_carry, s_target;
  __shared__ int s_mode;

  const int b = blockIdx.x, tid = threadIdx.x;
  const int N = a.N, rows = 2 * N + 1;
  const int lane = tid & 63, wave = tid >> 6;

  // 1. Row normalisers from the chunk statistics (fixed chunk order).
  if (tid < rows) {
    const float2* st = a.stats + ((size_t)b * rows + tid) * a.nchunks;
    float M = st[0].x, S = st[0].y;
    for (int c = 1; c < a.nchunks; ++c) merge_ms(M, S, st[c].x, st[c].y, a.c2);
    row_m[tid] = M;
    row_l[tid] = log2f(S);
  }
  __syncthreads();

  // 2. Ratio tests: keep x_i iff u < p_i(x_i)/q_i(x_i).
  if (tid < N) {
    const int x = a.tokens[(size_t)b * N + tid];
    bool keep = false;
    if (x >= 0 && x < a.V) {
      const float zp = a.target[((size_t)b * (N + 1) + tid) * a.V + x];
      const float zq = a.draft[((size_t)b * N + tid) * a.V + x];
      const float lp = (zp - row_m[tid]) * a.c2 - row_l[tid];
      const float lq = (zq - row_m[N + 1 + tid]) * a.c2 - row_l[N + 1 + tid];
      const float r = exp2f(lp - lq);   // q = 0: +inf when p > 0; NaN (reject) when both 0
      keep = a.u_acc[(size_t)b * N + tid] < r;
    }
    ratio_ok[tid] = keep ? 1.f : 0.f;
  }
  __syncthreads();
  if (tid == 0) {
    int k = N;
    for (int i = 0; i < N; ++i)
      if (ratio_ok[i] == 0.f) { k = i; break; }
    s_k = k;
    s_mode = k < N ? 1 : 0;
  }
  __syncthreads();
  const int k = s_k;
  const int nch = (a.V + kDrawChunk - 1) / kDrawChunk;
  const float u = a.u_draw[(size_t)b * (N + 1) + k];

  for (int attempt = 0; attempt < 2; ++attempt) {
    DrawRow dr;
    dr.zp = a.target + ((size_t)b * (N + 1) + k) * a.V;
    dr.mp = row_m[k];
    dr.lp = row_l[k];
    dr.c = a.c2;
    dr.zq = nullptr;
    dr.mq = dr.lq = 0.f;
    if (s_mode == 1) {
      dr.zq = a.draft + ((size_t)b * N + k) * a.V;
      dr.mq = row_m[N + 1 + k];
      dr.lq = row_l[N + 1 + k];
    }

    // 3. Chunk sums of the weights.
    float w[kDrawPer], pre[kDrawPer];
    for (int c = 0; c < nch; ++c) {
      draw_weights<VEC>(dr, a.V, c, w);
      chunk_scan(w, pre, wave_tot, wave_off);
      if (tid == kDrawThreads - 1) csum[c] = pre[kDrawPer - 1];
    }
    __syncthreads();
    if (tid == 0) {
      float total = 0.f;
      for (int c = 0; c < nch; ++c) total += csum[c];
      s_chunk = -2;
      if (total == 0.f && s_mode == 1) {
        s_mode = 0;            // empty residual: fall back to p_k
      } else {
        const float target = u * total;
        float acc = 0.f;
        s_chunk = -1;
        for (int c = 0; c < nch; ++c) {
          if (acc + csum[c] > target) { s_chunk = c; break; }
          acc += csum[c];
        }
        s_carry = acc;
        s_target = target;
        if (s_chunk < 0) {      // rounding left no crossing: last chunk with mass
          for (int c = nch - 1; c >= 0; --c)
            if (csum[c] > 0.f) { s_chunk = c; break; }
        }
      }
    }
    __syncthreads();
    if (s_chunk == -2) continue;   // retry with p_k

    // 4. Locate the crossing inside chunk c: the first weight whose running
    //    sum exceeds u*total (or, if rounding left no crossing, the last
    //    positive weight of the last chunk with mass).
    const int c = s_chunk;
    if (c < 0) {                    // no mass at all (a row of -inf): no token
      if (tid == 0) s_y = -1;
      __syncthreads();
      break;
    }
    const bool last_mass = !(s_carry + csum[c] > s_target);
    draw_weights<VEC>(dr, a.V, c, w);
    chunk_scan(w, pre, wave_tot, wave_off);
    int pick = -1;
    if (!last_mass) {
#pragma unroll
      for (int e = kDrawPer - 1; e >= 0; --e)
        if (s_carry + pre[e] > s_target) pick = e;
    } else {
#pragma unroll
      for (int e = 0; e < kDrawPer; ++e)
        if (w[e] > 0.f) pick = e;
    }
    const int tok = pick < 0 ? -1 : c * kDrawChunk + tid * kDrawPer + pick;
    const uint64_t ballot = __ballot(pick >= 0);
    int src = 0;
    if (ballot) src = last_mass ? 63 - __builtin_clzll(ballot) : __builtin_ctzll(ballot);
    const int wtok = __shfl(tok, src);
    if (lane == 0) wave_hit[wave] = ballot ? wtok : -1;
    __syncthreads();
    if (tid == 0) {
      int y = -1;
      if (!last_mass) {
        for (int i = 0; i < kDrawThreads / kWave; ++i)
          if (wave_hit[i] >= 0) { y = wave_hit[i]; break; }
      } else {
        for (int i = kDrawThreads / kWave - 1; i >= 0; --i)
          if (wave_hit[i] >= 0) { y = wave_hit[i]; break; }
      }
      s_y = y;
    }
    __syncthreads();
    break;
  }

  // 5. Emit x_0..x_{k-1}, y, then -1.
  if (tid <= N) {
    int v = -1;
    if (tid < k) v = a.tokens[(size_t)b * N + tid];
    else if (tid == k) v = s_y;
    a.out[(size_t)b * (N + 1) + tid] = v;
  }
  if (tid == 0) a.num_acc[b] = k;
}

ChainPlan plan_chain(int B, int N, int V) {
  ChainPlan p{};
  p.rows_per_seq = 2 * N + 1;
  p.chunk = kStatsChunk;
  p.nchunks = (V + kStatsChunk - 1) / kStatsChunk;
  p.stats_bytes = align256((size_t)B * p.rows_per_seq * p.nchunks * sizeof(float2));
  p.total_bytes = p.stats_bytes;
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
  a.B = B; a.N = N; a.V = V; a.chunk = p.chunk; a.nchunks = p.nchunks;
  a.c2 = kLog2e / temperature;
  const bool vec4 = (V % 4 == 0) && ((uintptr_t)target % 16 == 0) &&
                    (N == 0 || (uintptr_t)draft % 16 == 0);
  const dim3 g1(p.nchunks, B * p.rows_per_seq);
  if (vec4) chain_stats_kernel<4><<<g1, kStatsThreads, 0, st>>>(a);
  else chain_stats_kernel<1><<<g1, kStatsThreads, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (vec4) chain_draw_kernel<4><<<B, kDrawThreads, 0, st>>>(a);
  else chain_draw_kernel<1><<<B, kDrawThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace sv
