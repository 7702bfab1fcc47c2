// Verify attention for the N+1 chain positions or the T tree nodes of a draft,
// against the KV cache of the accepted prefix plus the draft positions.
//
// "LLM Primer VI — Chapitre 9 — Décodage spéculatif", §9.1: the target's pass
// over prefix + N candidates is parallel over positions and yields a next-token
// distribution at each of the N+1 positions; §9.2: an EAGLE-2 draft tree is
// verified in one attention pass under a custom mask.  "Parallel Decoding"
// glossary, "L'attention en arbre : la brique commune": the root is the last
// verified token and the mask encodes the tree.
//
// Design (gfx950):
//  * split-K over the key axis: block (split s, unit u = b*Hkv + g) streams its
//    key range once for all R = G*T grouped rows that share KV head g, keeps an
//    online softmax per row and writes an unnormalised partial (o, m, l);
//    attn_combine merges the splits with a log-sum-exp;
//  * the tree mask is the ancestor-or-self bitmask of each query position,
//    one u64 per row held in registers: key ctx + t is visible to row i iff
//    bit t of mask(i) is set; prefix keys are visible to every row;
//  * fp32 inputs: VALU kernel, 16-byte loads, one key row spread over D/4
//    lanes, scores reduced across those lanes;
//  * bf16: MFMA kernel (v_mfma_f32_16x16x32_bf16), whatever R (a part-empty
//    row tile costs matrix work only; the pass is bound by the K/V stream).
//    Scores are computed transposed, S^T = K Q^T, and the output as
//    O^T += V^T P^T, so the probabilities produced by the first product are
//    already in the operand layout of the second: no cross-lane shuffle of P.
//    A loader wave streams K and V into an LDS ring with direct-to-LDS loads;
//    the V operand, which needs four consecutive keys per lane, is read with
//    the gfx950 transposing LDS load (ds_read_tr16_b64).
//
// Scores are kept in the log2 domain (scale * log2(e) folded in) and
// exponentiated with the hardware exp2.

#include <type_traits>

#include "common.h"

namespace sv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

struct AttnArgs {
  const void* q;           // [B, T, Hq, D]
  const void* k;           // [B, Hkv, L, D], or the page pool of a paged cache
  const void* v;           // [B, Hkv, L, D], or the page pool of a paged cache
  const int32_t* parents;  // [B, T] or nullptr (chain)
  float* out;              // [B, T, Hq, D]
  float* part_o;           // [units, S, R, D]  unnormalised partial outputs
  float* part_ml;          // [units, S, R, 2]  (running max in log2 units, sum)
  int B, T, Hq, Hkv, G, D, ctx, L, R, S, chunk;
  float scale_log2;        // softmax scale * log2(e)
  // Paged cache (the PAGED kernels only): position i of sequence b is row
  // i % page_size of page block_table[b][i / page_size]; ctx is then the
  // largest prefix and L = ctx + T the largest sequence.
  const int32_t* block_table;    // [B, max_blocks]
  const int32_t* ctx_lens;       // [B] prefix lengths, or nullptr (all ctx)
  int page_shift, max_blocks, num_pages;
  int64_t page_stride, head_stride, row_stride;   // elements
};

// Prefix length of sequence b: its own in a paged cache (clamped to
// [0, ctx], so a bad length cannot reach past the planned key range).
template <bool PAGED>
__device__ __forceinline__ int seq_ctx(const AttnArgs& a, int b) {
  if constexpr (PAGED) {
    if (a.ctx_lens != nullptr) return min(max(a.ctx_lens[b], 0), a.ctx);
  }
  return a.ctx;
}

// Element offset of row `key` of KV head g in page `page` of the pool (page
// ids outside the pool are clamped into it: wrong but in-bounds data).
__device__ __forceinline__ size_t paged_row(const AttnArgs& a, int page, int g, int key) {
  page = min(max(page, 0), a.num_pages - 1);
  return (size_t)page * a.page_stride + (size_t)g * a.head_stride +
         (size_t)(key & ((1 << a.page_shift) - 1)) * a.row_stride;
}

// Ancestor-or-self masks of the T query positions of sequence b, into LDS.
// Each position walks up its parents (a chain needs no walk).  A parent that
// is not strictly smaller than its child ends the walk, so malformed input
// cannot loop or index out of range.
__device__ __forceinline__ void build_masks(const AttnArgs& a, int b, int* par,
                                            uint64_t* masks) {
  const int t = threadIdx.x;
  if (a.parents != nullptr && t < a.T) par[t] = a.parents[(size_t)b * a.T + t];
  __syncthreads();
  if (t < a.T) {
    uint64_t m;
    if (a.parents == nullptr) {
      m = (t == 63) ? ~0ull : ((2ull << t) - 1ull);
    } else {
      m = 0;
      int n = t;
      while (true) {
        m |= 1ull << n;
        const int p = par[n];
        if (p < 0 || p >= n) break;
        n = p;
      }
    }
    masks[t] = m;
  }
  __syncthreads();
}

__device__ __forceinline__ bool tail_visible(uint64_t mask, int key, int ctx) {
  return key < ctx || ((mask >> (key - ctx)) & 1ull);
}

// Lambdas of the kernels are always inlined: an out-of-line call inside the
// key loop would make the compiler drain every outstanding load at its return.
#define SV_INLINE __attribute__((always_inline))

// Marks registers as used here, so the compiler waits for their loads once,
// before a loop, instead of re-checking (and draining newer loads) inside it.
__device__ __forceinline__ void settle(const u32x4_t& v) { asm volatile("" ::"v"(v)); }

// Lazy rescaling: the running reference max is kept until a new score exceeds
// it by 2^8 (in log2 units); the final ratio is unchanged by the choice.
constexpr float kRescaleLog2 = 8.f;

// Merge two online-softmax states (m in log2 units).
__device__ __forceinline__ void merge_state(float& m, float& l, float m2, float l2,
                                            float* o, const float* o2, int n) {
  const float mx = fmaxf(m, m2);
  if (mx == kNegInf) return;
  const float a1 = fast_exp2(m - mx), a2 = fast_exp2(m2 - mx);
  l = l * a1 + l2 * a2;
  for (int e = 0; e < n; ++e) o[e] = o[e] * a1 + o2[e] * a2;
  m = mx;
}

// ---------------------------------------------------------------------------
// VALU kernel (fp32 inputs): 4 independent waves per block; grid (S, B*Hkv,
// ceil(R / RMAX)).  A key row is spread over LPK lanes (one 16-byte load
// each); partial scores are summed across the LPK lanes with a DPP butterfly,
// which leaves the bit-identical total in every lane of the group.  Each lane
// group keeps its own online-softmax state over its keys; the groups and the
// waves are merged at the end.
// ---------------------------------------------------------------------------
// Sum over aligned groups of LPK lanes (LPK in {8, 16, 32}); every lane of a
// group ends with the same bits (each step adds a commuted pair).
template <int LPK>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp_f<kDppXor1>(v);                           // quad_perm [1,0,3,2]
  v += dpp_f<kDppXor2>(v);                           // quad_perm [2,3,0,1]
  v += dpp_f<kDppXor7>(v);                           // row_half_mirror: quads of each 8
  if constexpr (LPK >= 16) v += dpp_f<kDppXor15>(v); // row_mirror: halves of each 16
  if constexpr (LPK >= 32) {                         // row pairs: 32-lane halves
    float lo, hi;
    row_pair<false>(v, lo, hi);
    v = lo + hi;
  }
  return v;
}
template <int LPK>
__device__ __forceinline__ float group_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppXor7>(v));
  if constexpr (LPK >= 16) v = fmaxf(v, dpp_f<kDppXor15>(v));
  if constexpr (LPK >= 32) {
    float lo, hi;
    row_pair<false>(v, lo, hi);
    v = fmaxf(lo, hi);
  }
  return v;
}

template <int D, int RMAX, bool PAGED>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(1)))
void attn_valu_kernel(AttnArgs a) {
  constexpr int EPL = 4;                      // fp32 elements per lane per 16-byte load
  constexpr int LPK = D / EPL;                // lanes sharing one key row
  constexpr int KPS = kWave / LPK;            // keys per wave step
  constexpr int U = 4;                        // key steps per iteration
  constexpr int KPI = KPS * U;                // keys per wave iteration
  static_assert(LPK >= 8 && LPK <= 32, "layout");

  __shared__ int par[64];
  __shared__ uint64_t masks[64];
  __shared__ float red_o[4][RMAX][D];
  __shared__ float red_ml[4][RMAX][2];

  const int s = blockIdx.x, u = blockIdx.y, rc = blockIdx.z;
  const int b = u / a.Hkv, g = u % a.Hkv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ks = lane / LPK, dp = lane % LPK;
  const int r0 = rc * RMAX;
  const int nr = min(RMAX, a.R - r0);

  build_masks(a, b, par, masks);

  // Query rows (fp32 bits).
  u32x4_t qw[RMAX];
  uint64_t mrow[RMAX];
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    qw[r] = (u32x4_t){0, 0, 0, 0};
    mrow[r] = 0;
    if (r < nr) {
      const int row = r0 + r, t = row / a.G, h = g * a.G + row % a.G;
      qw[r] = *(const u32x4_t*)((const float*)a.q + (((size_t)b * a.T + t) * a.Hq + h) * D +
                                dp * EPL);
      mrow[r] = masks[t];
    }
  }
  // Q stays in registers for the whole key loop: wait for it here.
#pragma unroll
  for (int r = 0; r < RMAX; ++r) settle(qw[r]);

  // This block's keys, cut into 4 contiguous per-wave ranges (a split past
  // the end of a shorter paged sequence has none).
  const int ctx = seq_ctx<PAGED>(a, b), L = ctx + a.T;
  const int kb = s * a.chunk, ke = max(kb, min(L, kb + a.chunk));
  const int per = ((ke - kb + 3) / 4 + KPI - 1) / KPI * KPI;
  const int wb = kb + wave * per, we = min(ke, wb + per);
  const int clean_end = min(ctx, we);
  const float c = a.scale_log2;

  float m[RMAX], l[RMAX], o[RMAX][EPL];
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    m[r] = kNegInf;
    l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[r][e] = 0.f;
  }

  const size_t unit_off = PAGED ? 0 : (size_t)u * a.L * D;
  const float* kp = (const float*)a.k + unit_off + dp * EPL;
  const float* vp = (const float*)a.v + unit_off + dp * EPL;
  const int32_t* bt = a.block_table + (PAGED ? (size_t)b * a.max_blocks : 0);
  const int last = L - 1;

  u32x4_t kw[U], vw[U];
  auto load = [&](int key0) {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int key = min(key0 + j * KPS + ks, last);
      size_t off;
      if constexpr (PAGED) off = paged_row(a, bt[key >> a.page_shift], g, key);
      else off = (uint32_t)(key * D);
      kw[j] = *(const u32x4_t*)(kp + off);
      vw[j] = *(const u32x4_t*)(vp + off);
    }
  };
  if (wb < we) load(wb);
  for (int key0 = wb; key0 < we; key0 += KPI) {
    u32x4_t kcur[U], vcur[U];
#pragma unroll
    for (int j = 0; j < U; ++j) { kcur[j] = kw[j]; vcur[j] = vw[j]; }
    if (key0 + KPI < we) load(key0 + KPI);       // next keys in flight

    float vf[U][EPL];
#pragma unroll
    for (int j = 0; j < U; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) vf[j][e] = __uint_as_float(vcur[j][e]);
    const bool clean = key0 + KPI <= clean_end;
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
      if (r >= nr) break;
      float sc[U];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc = fmaf(__uint_as_float(qw[r][e]), __uint_as_float(kcur[j][e]), acc);
        sc[j] = group_sum<LPK>(acc);
        if (!clean) {
          const int key = key0 + j * KPS + ks;
          if (!(key < we && tail_visible(mrow[r], key, ctx))) sc[j] = kNegInf;
        }
      }
      float mt = sc[0];
#pragma unroll
      for (int j = 1; j < U; ++j) mt = fmaxf(mt, sc[j]);
      mt *= c;
      const bool bump = mt > m[r] + kRescaleLog2;
      if (__any(bump)) {
        // lanes that keep their reference (possibly -inf) must not compute -inf - -inf
        const float alpha = bump ? fast_exp2(m[r] - mt) : 1.f;
        if (bump) m[r] = mt;
        l[r] *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[r][e] *= alpha;
      }
      const float msafe = (m[r] == kNegInf) ? 0.f : m[r];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const float p = fast_exp2(fmaf(sc[j], c, -msafe));
        l[r] += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[r][e] = fmaf(p, vf[j][e], o[r][e]);
      }
    }
  }

  // Merge the KPS key slots of the wave (lanes with equal dp hold equal d's).
#pragma unroll
  for (int off = LPK; off < kWave; off <<= 1) {
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
      const float m2 = __shfl_xor(m[r], off), l2 = __shfl_xor(l[r], off);
      float o2[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) o2[e] = __shfl_xor(o[r][e], off);
      merge_state(m[r], l[r], m2, l2, o[r], o2, EPL);
    }
  }
  // Merge the four waves through LDS.
  if (ks == 0) {
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) red_o[wave][r][dp * EPL + e] = o[r][e];
      if (dp == 0) { red_ml[wave][r][0] = m[r]; red_ml[wave][r][1] = l[r]; }
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < nr * D; idx += 256) {
    const int r = idx / D, d = idx % D;
    float mm = red_ml[0][r][0], ll = red_ml[0][r][1], oo = red_o[0][r][d];
    for (int w = 1; w < 4; ++w) merge_state(mm, ll, red_ml[w][r][0], red_ml[w][r][1], &oo,
                                            &red_o[w][r][d], 1);
    const size_t prow = ((size_t)u * a.S + s) * a.R + (r0 + r);
    a.part_o[prow * D + d] = oo;
    if (d == 0) { a.part_ml[prow * 2] = mm; a.part_ml[prow * 2 + 1] = ll; }
  }
}

// ---------------------------------------------------------------------------
// MFMA kernel (bf16): a block of W waves shares each 32-key K/V tile in LDS;
// wave w owns RT row tiles of 16 grouped rows.  Grid (S, B*Hkv, row chunks).
//
// Products per 32-key tile and row tile (v_mfma_f32_16x16x32_bf16):
//   S^T[key][row]  = K[key][:] . Q[row][:]    A = K fragment (ds_read_b128),
//                                             B = Q fragment (registers);
//   O^T[d][row]   += V^T[d][key] . P[row][key] A = V fragment (two
//                                             ds_read_tr16_b64), B = P (registers).
// The accumulator layout of S^T (lane l: row l%16, keys 4(l/16)+r of each
// 16-key half) is the B-operand layout of P when the contraction runs over
// the tile's keys in the order pv_key(): so P never leaves its lanes.
// ---------------------------------------------------------------------------
constexpr int kMfmaKeys = 32;      // keys per tile (the contraction depth of P.V)

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Key (0..31) of the tile that contraction position 8g + e (g = lane/16) stands
// for: positions 0..3 of a lane group are keys 4g..4g+3 (first 16-key half),
// positions 4..7 are keys 16+4g..16+4g+3 (second half).
__device__ __forceinline__ int pv_key(int g, int e) {
  return (e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4));
}

// Reductions over the four 16-lane groups of a wave (lanes l, l^16, l^32,
// l^48), every lane receiving the result.  The gfx950 lane-swap instructions
// exchange rows 1,3 with rows 0,2 of a second register (permlane16) and the
// upper with the lower half (permlane32); combining each pair gives the
// xor-16 / xor-32 partner without going through LDS.
__device__ __forceinline__ float group4_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float group4_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Loading.  The block is W compute waves plus one loader wave.  The loader
// streams the block's key range through a ring of P LDS slots of one 32-key
// K/V tile each with direct-to-LDS loads (global_load_lds, 16 bytes per lane
// written straight into LDS), keeping AHEAD tiles in flight without holding
// them in registers.  It waits for its own loads (s_waitcnt vmcnt) and joins
// the block barrier: after barrier j, tile j is complete in slot j % P and a
// slot no wave reads any more is refilled with tile j + AHEAD.  The compute
// waves issue no global loads inside the key loop.  The loads are written as
// inline assembly so that the compiler does not order LDS reads after them.
//
// Slot layout.  A direct-to-LDS load writes 1 KB contiguous (lane L at +16L),
// here a group of KG = 512/D key rows.  Inside a group the 16-byte chunks are
// placed by chunk_pos() so that the V fragment reads (ds_read_tr16_b64) are
// free of bank conflicts and the K fragment reads (ds_read_b128) spread over
// all banks; groups are padded to GSK / GSV bytes.
//   D = 128 (4 rows x 16 chunks): chunk c of row j at 4c + j;
//   D = 64  (8 rows x 8 chunks):  16(c/2) + 8(j/4) + ((4(c%2) + j%4) ^ 4(j/4)).
template <int D>
struct MfmaLayout {
  static constexpr int KT = kMfmaKeys;
  static constexpr int KG = 512 / D;              // key rows per 1 KB group
  static constexpr int NG = KT / KG;              // groups per tile and tensor
  static constexpr int GSK = D == 128 ? 1088 : 1152;
  static constexpr int GSV = 1152;
  static constexpr int KHALF = NG * GSK;
  static constexpr int SLOT = KHALF + NG * GSV;
  static constexpr int NIT = 2 * NG;              // 1 KB loads per tile (K and V)
  __host__ __device__ static constexpr int chunk_pos(int j, int c) {
    return D == 128 ? 4 * c + j
                    : 16 * (c >> 1) + 8 * (j >> 2) + ((4 * (c & 1) + (j & 3)) ^ (4 * (j >> 2)));
  }
};

// Ring depth: four slots (72 KB at D = 128) keep two blocks per CU resident
// for one-row-tile kernels; five or six for the larger ones (one block per CU).  The
// loader's outstanding loads, (AHEAD - 1) * NIT, must fit the 6-bit vmcnt.
template <int D, int RT>
struct MfmaRing {
  // LAG: with two compute waves per SIMD (more than four compute waves), the
  // upper waves run half a tile behind (see the key loop), which keeps the
  // previous tile's slot in use until the next barrier.  Measured: medusa
  // tree (three row tiles) 104.8 -> 97.8 us; eagle2 tree (two row tiles)
  // 94.8 -> 91.8 us once the softmax had shed its per-tile row reduction
  // (before that, two-row-tile kernels were slower lagged).
  static constexpr bool LAG = RT >= 2;
  static constexpr int P = RT == 1 ? 4 : LAG ? 6 : 5;
  static constexpr int AHEAD_MAX = 63 / MfmaLayout<D>::NIT + 1;   // (AHEAD-1)*NIT < 64
  static constexpr int AHEAD = (LAG ? P - 2 : P - 1) < AHEAD_MAX ? (LAG ? P - 2 : P - 1)
                                                                 : AHEAD_MAX;
  static_assert((AHEAD - 1) * MfmaLayout<D>::NIT < 64, "vmcnt range");
};

// One direct load of 16 bytes per lane into LDS at byte offset lds (wave-
// uniform; lane L writes lds + 16L).  M0 carries the LDS address; the nop
// covers the M0-write to LDS-DMA hazard.  K and V are read once: the loads
// are non-temporal.
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(g), "{m0}"(lds) : "memory");
}
// The same with 4 bytes per lane (lane L writes lds + 4L): page ids.
__device__ __forceinline__ void lds_dma4(const void* g, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Wait until at most `rem` (<= MAXR, wave-uniform) tiles of C loads each are
// still outstanding (this wave's loads only).
template <int C, int MAXR>
__device__ __forceinline__ void wait_tiles(int rem) {
  if constexpr (MAXR == 0) {
    wait_vm<0>();
  } else {
    if (rem >= MAXR) wait_vm<MAXR * C>();
    else wait_tiles<C, MAXR - 1>(rem);
  }
}
// Block barrier for the ring: LDS reads done, then s_barrier.  The memory
// clobber keeps every LDS access on its side of the barrier.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int D, int RT, int W, bool PAGED>
__global__ __launch_bounds__(64 * (W + 1))
void attn_mfma_kernel(AttnArgs a) {
  using LY = MfmaLayout<D>;
  using RG = MfmaRing<D, RT>;
  constexpr int KT = kMfmaKeys;
  constexpr int P = RG::P;
  constexpr int DT = D / 16;
  constexpr int KK = D / 32;

  __shared__ __attribute__((aligned(1024))) uint8_t ring[P * LY::SLOT];
  __shared__ int par[64];
  __shared__ uint64_t masks[64];
  __shared__ int ptab[PAGED ? P * 64 : 1];    // paged: page ids of the tiles in flight

  const int s = blockIdx.x, u = blockIdx.y, rc = blockIdx.z;
  const int b = u / a.Hkv, gk = u % a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
  const int l16 = lane & 15, g4 = lane >> 4;

  build_masks(a, b, par, masks);

  // a split past the end of a shorter paged sequence has no tiles
  const int ctx = seq_ctx<PAGED>(a, b), L = ctx + a.T;
  const int kb = s * a.chunk, ke = max(kb, min(L, kb + a.chunk));
  const int ntiles = (ke - kb + KT - 1) / KT;
  const size_t unit_off = PAGED ? 0 : (size_t)u * L * D;
  const uint16_t* kg = (const uint16_t*)a.k + unit_off;
  const uint16_t* vg = (const uint16_t*)a.v + unit_off;

  if (wave == W) {
    // ---- loader wave: this lane's key row within a group and 16-byte chunk ----
    int lj, lc;
    if constexpr (D == 128) {
      lj = lane & 3; lc = lane >> 2;
    } else {
      const int sg = (lane >> 3) & 1, x = (lane & 7) ^ (4 * sg);
      lj = 4 * sg + (x & 3); lc = 2 * (lane >> 4) + (x >> 2);
    }
    const uint32_t ring_lds =
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)ring;
    // Paged: the ids of the (up to 32) pages under tile t are loaded, 64 at a
    // time, into ptab[t % P] by the issue of tile t - AHEAD, as one more load
    // of that issue, so the in-order wait for a tile also covers them.  Every
    // issue loads them (clamped ids past the end) to keep NIT + 1 loads per tile.
    const int32_t* bt = a.block_table + (PAGED ? (size_t)b * a.max_blocks : 0);
    const int last_blk = PAGED ? (L - 1) >> a.page_shift : 0;
    const uint32_t ptab_lds =
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) int*)ptab;
    auto fetch_pages = [&](int t) SV_INLINE {
      const int idx = min(((kb + t * KT) >> a.page_shift) + lane, last_blk);
      lds_dma4(bt + idx, ptab_lds + (uint32_t)((t % P) * 256));
    };
    auto issue = [&](int t) SV_INLINE {
      const int key0 = kb + t * KT + lj;
      const uint32_t slot = ring_lds + (uint32_t)((t % P) * LY::SLOT);
#pragma unroll
      for (int g = 0; g < LY::NG; ++g) {
        // keys past the end re-read the last row (finite data, masked later)
        const int key = min(key0 + g * LY::KG, L - 1);
        const uint32_t off = (uint32_t)key * D + 8 * lc;
        lds_dma16(kg + off, slot + g * LY::GSK);
        lds_dma16(vg + off, slot + LY::KHALF + g * LY::GSV);
      }
    };
    // Paged: every offset of a tile is computed (page ids read from LDS) before
    // its first load is issued, so that the reads share one wait.
    auto paged_offsets = [&](int t, size_t (&off)[LY::NG]) SV_INLINE {
      const int key0 = kb + t * KT + lj;
      const int first = (kb + t * KT) >> a.page_shift;
#pragma unroll
      for (int g = 0; g < LY::NG; ++g) {
        const int key = min(key0 + g * LY::KG, L - 1);
        off[g] = paged_row(a, ptab[(t % P) * 64 + (key >> a.page_shift) - first], gk, key) +
                 8 * lc;
      }
    };
    auto paged_issue = [&](int t, const size_t (&off)[LY::NG]) SV_INLINE {
      const uint32_t slot = ring_lds + (uint32_t)((t % P) * LY::SLOT);
#pragma unroll
      for (int g = 0; g < LY::NG; ++g) {
        lds_dma16(kg + off[g], slot + g * LY::GSK);
        lds_dma16(vg + off[g], slot + LY::KHALF + g * LY::GSV);
      }
      fetch_pages(t + RG::AHEAD);
    };
    // After barrier j the slot refilled with tile j + AHEAD is that of tile
    // j - 1 (j - 2 with LAG: lagging waves still read tile j - 1).
    const int pre = min(RG::AHEAD, ntiles);
    if constexpr (PAGED) {
      constexpr int C = LY::NIT + 1;                  // loads per issue
      static_assert((RG::AHEAD - 1) * C < 64, "vmcnt range");
      for (int t = 0; t < pre; ++t) fetch_pages(t);
      wait_vm<0>();
      for (int t = 0; t < pre; ++t) {
        size_t off[LY::NG];
        paged_offsets(t, off);
        paged_issue(t, off);
      }
      for (int j = 0; j < ntiles; ++j) {
        wait_tiles<C, RG::AHEAD - 1>(min(ntiles - 1 - j, RG::AHEAD - 1));
        // the page ids of tile j + AHEAD came with tile j: read them while
        // the compute waves reach the barrier
        const bool more = j + RG::AHEAD < ntiles;
        size_t off[LY::NG];
        if (more) paged_offsets(j + RG::AHEAD, off);
        ring_barrier();
        if (more) paged_issue(j + RG::AHEAD, off);
      }
    } else {
      for (int t = 0; t < pre; ++t) issue(t);
      for (int j = 0; j < ntiles; ++j) {
        wait_tiles<LY::NIT, RG::AHEAD - 1>(min(ntiles - 1 - j, RG::AHEAD - 1));
        ring_barrier();
        if (j + RG::AHEAD < ntiles) issue(j + RG::AHEAD);
      }
    }
    return;
  }

  // ---- Q fragments (registers for the whole key loop) ----
  const int tile0 = (rc * W + wave) * RT;
  bf16x8_t qf[RT][KK];
  uint64_t mrow[RT];
  bool live[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = (tile0 + rt) * 16 + l16;
    live[rt] = (tile0 + rt) * 16 < a.R;
    mrow[rt] = 0;
    const u32x4_t z = {0, 0, 0, 0};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[rt][kk] = __builtin_bit_cast(bf16x8_t, z);
    if (row < a.R) {
      const int t = row / a.G, h = gk * a.G + row % a.G;
      const uint16_t* qp = (const uint16_t*)a.q + (((size_t)b * a.T + t) * a.Hq + h) * D;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        qf[rt][kk] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(qp + 32 * kk + 8 * g4));
      mrow[rt] = masks[t];
    }
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) settle(__builtin_bit_cast(u32x4_t, qf[rt][kk]));

  f32x4_t acc[RT][DT];
  float m[RT], m8[RT], lsum[RT];      // m8 = m + kRescaleLog2, the raising threshold
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m[rt] = kNegInf;
    m8[rt] = kNegInf;
    lsum[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[rt][dt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  }

  // LDS byte offsets of this lane's fragments within a slot.
  //  K: row 16*sub + l16, chunk 4*kk + g4      -> kofs + sub*KSUB + kk*KKS
  //  V: keys pv_key(g4, l16/4) and pv_key(g4, 4 + l16/4), bf16 columns
  //     16*dt + 4*(l16%4) .. +3 (chunk 2*dt + (l16/2)%2, half l16%2)
  //                                            -> vofs0/vofs1 + dt*VDT
  int kofs, vofs0, vofs1;
  constexpr int KSUB = (16 / LY::KG) * LY::GSK;
  constexpr int KKS = 16 * (LY::chunk_pos(0, 4) - LY::chunk_pos(0, 0));
  constexpr int VDT = 16 * (LY::chunk_pos(0, 2) - LY::chunk_pos(0, 0));
  {
    const int kr = l16;                                   // row within the 16-row half
    kofs = (kr / LY::KG) * LY::GSK + 16 * LY::chunk_pos(kr % LY::KG, g4);
    const int vk0 = pv_key(g4, l16 >> 2), vk1 = pv_key(g4, 4 + (l16 >> 2));
    const int vc = (l16 >> 1) & 1;                        // chunk 0 or 1 of the dt pair
    vofs0 = LY::KHALF + (vk0 / LY::KG) * LY::GSV + 16 * LY::chunk_pos(vk0 % LY::KG, vc) +
            8 * (l16 & 1);
    vofs1 = LY::KHALF + (vk1 / LY::KG) * LY::GSV + 16 * LY::chunk_pos(vk1 % LY::KG, vc) +
            8 * (l16 & 1);
  }

  const float c = a.scale_log2;
  // tiles [0, nclean) lie wholly inside the prefix: every key visible, no mask
  const int clean_end = min(ctx, ke);
  const int nclean = clean_end > kb ? (clean_end - kb) / KT : 0;
  typedef __attribute__((address_space(3))) const uint8_t lds_u8;
  lds_u8* const ring3 = (lds_u8*)ring;
  // The slot offset goes through readfirstlane: an opaque wave-uniform value,
  // so that every fragment address is one base plus an immediate offset.
  auto slot_of = [&](int t) SV_INLINE -> lds_u8* {
    return ring3 + __builtin_amdgcn_readfirstlane((t % P) * LY::SLOT);
  };

  // S^T for a tile's two 16-key halves.
  auto qk = [&](lds_u8* slot, f32x4_t (&st)[RT][2]) SV_INLINE {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) st[rt][0] = st[rt][1] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const bf16x8_t kf = __builtin_bit_cast(
            bf16x8_t, *(__attribute__((address_space(3))) const u32x4_t*)(slot + kofs + sub * KSUB +
                                                                           kk * KKS));
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)   // a dead tile (zero Q) computes harmless values
          st[rt][sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[rt][kk], st[rt][sub],
                                                               0, 0, 0);
      }
    }
  };

  // Online softmax of one tile, in log2 units with a lazily raised reference
  // max m, in two parts.  smax: masks the scores in place (tiles that reach
  // past the prefix), raises m where the tile's max exceeds it by 2^8 and
  // rescales the accumulators of those rows (rare).  sexp: probabilities as
  // bf16 in the B-operand layout of P.V (pf), their rounded sum into lsum.
  //
  // A row's m is raised only where the tile's row max, scaled, exceeds
  // m8 = m + kRescaleLog2.  The scaled row max exceeds m8 exactly when some
  // lane's own scaled max does (max commutes with the positive scale), so the
  // cross-lane row reduction runs only when some lane of the wave passes that
  // check: m evolves exactly as with a reduction on every tile, at 6 instead
  // of 18 vector instructions per row tile.
  auto smax = [&](auto clean_tag, f32x4_t (&st)[RT][2], int base) SV_INLINE {
    constexpr bool CLEAN = decltype(clean_tag)::value;
    float lm[RT];
    bool hit = false;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      if constexpr (!CLEAN) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int key = base + (e < 4 ? 4 * g4 + e : 16 + 4 * g4 + e - 4);
          if (!(key < ke && tail_visible(mrow[rt], key, ctx))) st[rt][e >> 2][e & 3] = kNegInf;
        }
      }
      const f32x4_t x0 = st[rt][0], x1 = st[rt][1];
      lm[rt] = fmaxf(fmaxf(fmaxf(x0[0], x0[1]), fmaxf(x0[2], x0[3])),
                     fmaxf(fmaxf(x1[0], x1[1]), fmaxf(x1[2], x1[3])));
      hit |= lm[rt] * c > m8[rt];
    }
    if (__any(hit)) {
      float mold[RT];
      bool raised = false;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const float mt = group4_max(lm[rt]) * c;   // scale > 0: max commutes with scaling
        mold[rt] = m[rt];
        if (mt > m8[rt]) { m[rt] = mt; m8[rt] = mt + kRescaleLog2; }
        raised |= m[rt] != mold[rt];
      }
      if (__any(raised)) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          // unchanged rows (possibly still -inf) keep factor 1; mold = -inf gives 0
          const float alpha = m[rt] == mold[rt] ? 1.f : fast_exp2(mold[rt] - m[rt]);
          lsum[rt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) acc[rt][dt] *= alpha;
        }
      }
    }
  };
  const bf16x2_t ones = {(__bf16)1.f, (__bf16)1.f};
  auto sexp = [&](auto clean_tag, const f32x4_t (&st)[RT][2], bf16x8_t (&pf)[RT]) SV_INLINE {
    constexpr bool CLEAN = decltype(clean_tag)::value;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      // a tile without visible keys leaves m = -inf: subtract 0 then (p = 0)
      const float msub = CLEAN ? m[rt] : (m[rt] == kNegInf ? 0.f : m[rt]);
      const f32x4_t x0 = st[rt][0], x1 = st[rt][1];
      const float sc[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      bf16x2_t pk[4];
      float sum = lsum[rt];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float p0 = fast_exp2(fmaf(sc[e], c, -msub));
        const float p1 = fast_exp2(fmaf(sc[e + 1], c, -msub));
        pk[e / 2] = __builtin_convertvector((f32x2_t){p0, p1}, bf16x2_t);
        sum = __builtin_amdgcn_fdot2_f32_bf16(pk[e / 2], ones, sum, false);
      }
      lsum[rt] = sum;
      pf[rt] = __builtin_shufflevector(__builtin_shufflevector(pk[0], pk[1], 0, 1, 2, 3),
                                       __builtin_shufflevector(pk[2], pk[3], 0, 1, 2, 3),
                                       0, 1, 2, 3, 4, 5, 6, 7);
    }
  };

  // O^T += V^T P^T.
  auto pv = [&](lds_u8* slot, const bf16x8_t (&pf)[RT]) SV_INLINE {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4_t*)(slot + vofs0 + dt * VDT));
      const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4_t*)(slot + vofs1 + dt * VDT));
      const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3,
                                                                               4, 5, 6, 7));
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        acc[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[rt], acc[rt][dt], 0, 0, 0);
    }
  };

  const std::integral_constant<bool, true> kClean;
  const std::integral_constant<bool, false> kMasked;
  auto step = [&](auto clean_tag, int it) SV_INLINE {
    ring_barrier();                             // tile it has landed in its slot
    f32x4_t st[RT][2];
    bf16x8_t pf[RT];
    qk(slot_of(it), st);
    smax(clean_tag, st, kb + it * KT);
    sexp(clean_tag, st, pf);
    pv(slot_of(it), pf);
  };
  // Waves 0-3 and 4-7 share the four SIMDs (waves are placed round-robin).
  // With LAG the upper waves apply P.V of the previous tile right after each
  // barrier and the current tile's P.V after the next one: while a lower wave
  // exponentiates, its partner computes scores, and the reverse.
  auto step_lag = [&](auto clean_tag, int it, bf16x8_t (&pprev)[RT]) SV_INLINE {
    ring_barrier();
    if (it > 0) pv(slot_of(it - 1), pprev);
    f32x4_t st[RT][2];
    qk(slot_of(it), st);
    smax(clean_tag, st, kb + it * KT);
    sexp(clean_tag, st, pprev);
  };
  int it = 0;
  if (RG::LAG && wave >= 4) {
    bf16x8_t pprev[RT];
    for (; it < ntiles && it < nclean; ++it) step_lag(kClean, it, pprev);
    for (; it < ntiles; ++it) step_lag(kMasked, it, pprev);
    if (ntiles > 0) pv(slot_of(ntiles - 1), pprev);   // the loader has stopped: slot intact
  } else {
    for (; it < ntiles && it < nclean; ++it) step(kClean, it);
    for (; it < ntiles; ++it) step(kMasked, it);
  }

  // Row sums over the four lane groups (every lane of a row gets the total).
  float lt[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) lt[rt] = group4_sum(lsum[rt]);

  // Lane holds O^T[16dt + 4g4 + r][row l16]: the final output when the block
  // saw every key (one split), else an unnormalised partial (o, m, l).
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = (tile0 + rt) * 16 + l16;
    if (!live[rt] || row >= a.R) continue;
    if (a.S == 1) {
      const int t = row / a.G, h = gk * a.G + row % a.G;
      float* op = a.out + (((size_t)b * a.T + t) * a.Hq + h) * D + 4 * g4;
      const float inv = 1.f / lt[rt];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) *(f32x4_t*)(op + 16 * dt) = acc[rt][dt] * inv;
    } else {
      const size_t prow = ((size_t)u * a.S + s) * a.R + row;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *(f32x4_t*)(a.part_o + prow * D + 16 * dt + 4 * g4) = acc[rt][dt];
      if (g4 == 0) { a.part_ml[prow * 2] = m[rt]; a.part_ml[prow * 2 + 1] = lt[rt]; }
    }
  }
}

// ---------------------------------------------------------------------------
// Split combine: log-sum-exp merge of the S partials of each row.  A block
// of 256 threads takes 1024/D rows of one unit, D/4 threads per row, each
// thread a float4 of the output; the split weights 2^(m_s - max) are computed
// once per row into LDS.  Grid (ceil(R / rows per block), units).
// ---------------------------------------------------------------------------
constexpr int kCombineThreads = 256;
constexpr int kCombineMaxS = 512;            // >= every split count the planner makes

template <int D>
__global__ __launch_bounds__(kCombineThreads) void attn_combine_kernel(AttnArgs a) {
  constexpr int GL = D / 4;                  // threads per row
  constexpr int RPB = kCombineThreads / GL;  // rows per block
  __shared__ float wsh[RPB][kCombineMaxS];
  const int u = blockIdx.y, tid = threadIdx.x;
  const int r = tid / GL, g = tid % GL;
  const int row = blockIdx.x * RPB + r;
  const bool live = row < a.R;
  const int S = a.S;
  const size_t base = (size_t)u * S * a.R + row;   // partial index of split 0

  // Row max over the splits (group of GL lanes, aligned within a wave).
  float mx = kNegInf;
  if (live)
    for (int sp = g; sp < S; sp += GL) mx = fmaxf(mx, a.part_ml[(base + (size_t)sp * a.R) * 2]);
  mx = group_max<GL>(mx);
  // Split weights into LDS and the weighted sum of the row sums.
  float den = 0.f;
  if (live)
    for (int sp = g; sp < S; sp += GL) {
      const size_t pi = base + (size_t)sp * a.R;
      const float ms = a.part_ml[pi * 2];
      const float w = ms == kNegInf ? 0.f : fast_exp2(ms - mx);
      wsh[r][sp] = w;
      den = fmaf(w, a.part_ml[pi * 2 + 1], den);
    }
  den = group_sum<GL>(den);
  __syncthreads();
  if (!live) return;
  f32x4_t num = {0.f, 0.f, 0.f, 0.f};
  const float* po = a.part_o + base * D + 4 * g;
  const size_t stride = (size_t)a.R * D;
#pragma unroll 4
  for (int sp = 0; sp < S; ++sp) num += wsh[r][sp] * *(const f32x4_t*)(po + sp * stride);
  const int b = u / a.Hkv, gk = u % a.Hkv;
  const int t = row / a.G, h = gk * a.G + row % a.G;
  *(f32x4_t*)(a.out + (((size_t)b * a.T + t) * a.Hq + h) * D + 4 * g) = num / den;
}

// ---------------------------------------------------------------------------
// Host-side dispatch.
// ---------------------------------------------------------------------------
template <int D, int RT, bool PG>
static void launch_mfma_w(const AttnPlan& p, const AttnArgs& a, hipStream_t st, dim3 grid) {
  switch (p.waves) {
    // W compute waves + the loader wave
    case 1: attn_mfma_kernel<D, RT, 1, PG><<<grid, 128, 0, st>>>(a); break;
    case 2: attn_mfma_kernel<D, RT, 2, PG><<<grid, 192, 0, st>>>(a); break;
    case 3: attn_mfma_kernel<D, RT, 3, PG><<<grid, 256, 0, st>>>(a); break;
    case 4: attn_mfma_kernel<D, RT, 4, PG><<<grid, 320, 0, st>>>(a); break;
    case 5: attn_mfma_kernel<D, RT, 5, PG><<<grid, 384, 0, st>>>(a); break;
    case 6: attn_mfma_kernel<D, RT, 6, PG><<<grid, 448, 0, st>>>(a); break;
    case 7: attn_mfma_kernel<D, RT, 7, PG><<<grid, 512, 0, st>>>(a); break;
    default:
      // three row tiles need more than the 168 registers that 9 waves per CU allow
      if constexpr (RT < 3) attn_mfma_kernel<D, RT, 8, PG><<<grid, 576, 0, st>>>(a);
      break;
  }
}

template <int D, bool PG>
static void launch_mfma(const AttnPlan& p, const AttnArgs& a, hipStream_t st, dim3 grid) {
  switch (p.rt) {
    case 1: launch_mfma_w<D, 1, PG>(p, a, st, grid); break;
    case 2: launch_mfma_w<D, 2, PG>(p, a, st, grid); break;
    default: launch_mfma_w<D, 3, PG>(p, a, st, grid); break;
  }
}

template <int D, bool PG>
static void launch_valu(const AttnPlan& p, const AttnArgs& a, hipStream_t st, dim3 grid) {
  switch (p.rmax) {
    case 1: attn_valu_kernel<D, 1, PG><<<grid, 256, 0, st>>>(a); break;
    case 2: attn_valu_kernel<D, 2, PG><<<grid, 256, 0, st>>>(a); break;
    case 4: attn_valu_kernel<D, 4, PG><<<grid, 256, 0, st>>>(a); break;
    default: attn_valu_kernel<D, 8, PG><<<grid, 256, 0, st>>>(a); break;
  }
}

template <bool PG>
static void launch_main(const AttnPlan& p, const AttnArgs& a, hipStream_t st, dim3 grid) {
  if (p.mfma) {
    if (a.D == 64) launch_mfma<64, PG>(p, a, st, grid);
    else launch_mfma<128, PG>(p, a, st, grid);
  } else {
    if (a.D == 64) launch_valu<64, PG>(p, a, st, grid);
    else launch_valu<128, PG>(p, a, st, grid);
  }
}

// Splits and tiles for a problem; a pure function of the shape so that the
// workspace query and the launch always agree.  The block targets aim at one
// full wave of resident blocks on the 256 CUs: the MFMA kernel's LDS ring
// admits two blocks per CU with one row tile per wave, one block otherwise.
constexpr int kMfmaBlocksRT1 = 512;   // one row tile per wave: two blocks per CU
constexpr int kMfmaBlocks = 256;      // larger row tiles: one block per CU
constexpr int kValuBlocks = 512;
constexpr int kMinChunk = 256;        // fewest keys per split
AttnPlan plan_attention(int B, int T, int Hq, int Hkv, int D, int ctx, int bf16) {
  AttnPlan p{};
  const int G = Hq / Hkv, R = G * T, L = ctx + T, units = B * Hkv;
  p.rows = R;
  // bf16 always takes the MFMA kernel (fewer than 16 rows leave part of the
  // one row tile empty: the pass is bound by the K/V stream, not the matrix
  // unit); fp32 inputs take the VALU kernel.
  p.mfma = bf16;
  int tile, blocks_target;
  if (p.mfma) {
    const int tiles = (R + 15) / 16;
    // one to three 16-row tiles per wave, at most 8 compute waves (7 with three
    // tiles each); the rest in row chunks
    p.rt = tiles <= 8 ? 1 : tiles <= 16 ? 2 : 3;
    const int max_waves = p.rt == 3 ? 7 : 8;
    int waves = (tiles + p.rt - 1) / p.rt;
    p.row_chunks = (waves + max_waves - 1) / max_waves;
    p.waves = (waves + p.row_chunks - 1) / p.row_chunks;
    tile = kMfmaKeys;
    blocks_target = p.rt == 1 ? kMfmaBlocksRT1 : kMfmaBlocks;
  } else {
    const int rr = R < 8 ? R : 8;
    p.rmax = rr <= 1 ? 1 : rr <= 2 ? 2 : rr <= 4 ? 4 : 8;
    p.waves = 4;
    p.row_chunks = (R + p.rmax - 1) / p.rmax;
    tile = 64;
    blocks_target = kValuBlocks;
  }
  const int min_chunk = kMinChunk;
  int S = (blocks_target + units * p.row_chunks - 1) / (units * p.row_chunks);
  if (S > kCombineMaxS) S = kCombineMaxS;
  const int s_max = (L + min_chunk - 1) / min_chunk;
  if (S > s_max) S = s_max;
  if (S < 1) S = 1;
  int chunk = (L + S - 1) / S;
  chunk = (chunk + tile - 1) / tile * tile;
  S = (L + chunk - 1) / chunk;
  p.splits = S;
  p.chunk = chunk;
  p.part_o_bytes = align256((size_t)units * S * R * D * sizeof(float));
  p.part_ml_bytes = align256((size_t)units * S * R * 2 * sizeof(float));
  p.total_bytes = p.part_o_bytes + p.part_ml_bytes;
  return p;
}

hipError_t launch_attention(const AttnPlan& p, const void* q, const void* k, const void* v,
                            const int32_t* parents, float* out, int B, int T, int Hq, int Hkv,
                            int D, int ctx, int bf16, float scale, void* workspace,
                            hipStream_t st, const PagedKV* paged) {
  AttnArgs a{};
  a.q = q; a.k = k; a.v = v; a.parents = parents; a.out = out;
  a.part_o = (float*)workspace;
  a.part_ml = (float*)((char*)workspace + p.part_o_bytes);
  a.B = B; a.T = T; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv; a.D = D; a.ctx = ctx;
  a.L = ctx + T; a.R = p.rows; a.S = p.splits; a.chunk = p.chunk;
  a.scale_log2 = scale * kLog2e;
  (void)bf16;
  const dim3 grid(p.splits, B * Hkv, p.row_chunks);
  if (paged != nullptr) {
    const int64_t ps = paged->page_size;
    a.block_table = paged->block_table;
    a.ctx_lens = paged->ctx_lens;
    a.page_shift = __builtin_ctz((unsigned)paged->page_size);
    a.max_blocks = paged->max_blocks;
    a.num_pages = paged->num_pages;
    a.page_stride = ps * Hkv * D;
    if (paged->position_major) {     // [pages, page_size, Hkv, D]
      a.head_stride = D; a.row_stride = (int64_t)Hkv * D;
    } else {                         // [pages, Hkv, page_size, D]
      a.head_stride = ps * D; a.row_stride = D;
    }
    launch_main<true>(p, a, st, grid);
  } else {
    launch_main<false>(p, a, st, grid);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || (p.mfma && p.splits == 1)) return e;
  const int rpb = kCombineThreads / (D / 4);
  const dim3 gc((p.rows + rpb - 1) / rpb, B * Hkv);
  if (D == 64) attn_combine_kernel<64><<<gc, kCombineThreads, 0, st>>>(a);
  else attn_combine_kernel<128><<<gc, kCombineThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace sv
