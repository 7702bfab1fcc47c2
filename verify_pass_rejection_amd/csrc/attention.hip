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
//  * R < 16 (or fp32 inputs): VALU kernel, 16-byte loads, one key row spread
//    over D*sizeof/16 lanes, scores reduced across those lanes;
//  * bf16 with R >= 16: MFMA kernel (v_mfma_f32_16x16x32_bf16).  Scores are
//    computed transposed, S^T = K Q^T, and the output as O^T += V^T P^T, so the
//    probabilities produced by the first product are already in the operand
//    layout of the second: no cross-lane shuffle of P.  K and V are staged in
//    LDS row-major; the V operand, which needs four consecutive keys per lane,
//    is read with the gfx950 transposing LDS load (ds_read_tr16_b64).
//
// Scores are kept in the log2 domain (scale * log2(e) folded in) and
// exponentiated with the hardware exp2.

#include "common.h"

namespace sv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

struct AttnArgs {
  const void* q;           // [B, T, Hq, D]
  const void* k;           // [B, Hkv, L, D]
  const void* v;           // [B, Hkv, L, D]
  const int32_t* parents;  // [B, T] or nullptr (chain)
  float* out;              // [B, T, Hq, D]
  float* part_o;           // [units, S, R, D]  unnormalised partial outputs
  float* part_ml;          // [units, S, R, 2]  (running max in log2 units, sum)
  int B, T, Hq, Hkv, G, D, ctx, L, R, S, chunk;
  float scale_log2;        // softmax scale * log2(e)
};

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

#ifndef SV_SETTLE_MFMA
#define SV_SETTLE_MFMA 1
#endif
#ifndef SV_MFMA_WAVES_PER_EU
#define SV_MFMA_WAVES_PER_EU 4
#endif
#ifndef SV_SETTLE_VALU
#define SV_SETTLE_VALU 1
#endif
#ifndef SV_VALU_WAVES_PER_EU
#define SV_VALU_WAVES_PER_EU 1
#endif

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
// VALU kernel: 4 independent waves per block; grid (S, B*Hkv, ceil(R / RMAX)).
// A key row is spread over LPK lanes (one 16-byte load each); bf16 scores use
// v_dot2_f32_bf16 and are summed across the LPK lanes with a DPP butterfly,
// which leaves the bit-identical total in every lane of the group.  Each lane
// group keeps its own online-softmax state over its keys; the groups and the
// waves are merged at the end.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of LPK lanes (LPK in {8, 16, 32}); every lane of a
// group ends with the same bits (each step adds a commuted pair).
template <int LPK>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp_f<0xB1>(v);     // quad_perm [1,0,3,2]: lane ^ 1
  v += dpp_f<0x4E>(v);     // quad_perm [2,3,0,1]: lane ^ 2
  v += dpp_f<0x141>(v);    // row_half_mirror: quad 0 <-> quad 1 of each 8
  if constexpr (LPK >= 16) v += dpp_f<0x140>(v);   // row_mirror: halves of each 16
  if constexpr (LPK >= 32) v += __shfl_xor(v, 16);
  return v;
}

template <typename TIn, int D, int RMAX>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(RMAX <= 4 ? SV_VALU_WAVES_PER_EU : 1)))
void attn_valu_kernel(AttnArgs a) {
  constexpr bool BF = sizeof(TIn) == 2;
  constexpr int EPL = 16 / (int)sizeof(TIn);  // elements per lane per 16-byte load
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

  // Query rows: raw bf16 pairs (dot2 operands) or fp32 values.
  u32x4_t qw[RMAX];
  uint64_t mrow[RMAX];
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    qw[r] = (u32x4_t){0, 0, 0, 0};
    mrow[r] = 0;
    if (r < nr) {
      const int row = r0 + r, t = row / a.G, h = g * a.G + row % a.G;
      qw[r] = *(const u32x4_t*)((const TIn*)a.q + (((size_t)b * a.T + t) * a.Hq + h) * D +
                                dp * EPL);
      mrow[r] = masks[t];
    }
  }
  // Q stays in registers for the whole key loop: wait for it here.
#if SV_SETTLE_VALU
#pragma unroll
  for (int r = 0; r < RMAX; ++r) settle(qw[r]);
#endif

  // This block's keys, cut into 4 contiguous per-wave ranges.
  const int kb = s * a.chunk, ke = min(a.L, kb + a.chunk);
  const int per = ((ke - kb + 3) / 4 + KPI - 1) / KPI * KPI;
  const int wb = kb + wave * per, we = min(ke, wb + per);
  const int clean_end = min(a.ctx, we);
  const float c = a.scale_log2;

  float m[RMAX], l[RMAX], o[RMAX][EPL];
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    m[r] = kNegInf;
    l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[r][e] = 0.f;
  }

  const size_t unit_off = (size_t)u * a.L * D;
  const TIn* kp = (const TIn*)a.k + unit_off + dp * EPL;
  const TIn* vp = (const TIn*)a.v + unit_off + dp * EPL;
  const int last = a.L - 1;

  u32x4_t kw[U], vw[U];
  auto load = [&](int key0) {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const uint32_t off = (uint32_t)(min(key0 + j * KPS + ks, last) * D);
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
    for (int j = 0; j < U; ++j) {
      if constexpr (BF) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vf[j][2 * e] = bf16_lo(vcur[j][e]);
          vf[j][2 * e + 1] = bf16_hi(vcur[j][e]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) vf[j][e] = __uint_as_float(vcur[j][e]);
      }
    }
    const bool clean = key0 + KPI <= clean_end;
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
      if (r >= nr) break;
      float sc[U];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        float acc = 0.f;
        if constexpr (BF) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // copy the vector elements out first: a bit_cast of an ext-vector
            // element expression reads element 0 whatever the index
            const uint32_t qe = qw[r][e], ke2 = kcur[j][e];
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, qe),
                                                  __builtin_bit_cast(bf16x2v_t, ke2), acc,
                                                  false);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc = fmaf(__uint_as_float(qw[r][e]), __uint_as_float(kcur[j][e]), acc);
        }
        sc[j] = group_sum<LPK>(acc);
        if (!clean) {
          const int key = key0 + j * KPS + ks;
          if (!(key < we && tail_visible(mrow[r], key, a.ctx))) sc[j] = kNegInf;
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

// One row tile per wave: ask for the occupancy that keeps two blocks per CU
// resident (measured: 1.39 ms vs 1.50 ms on the 64 x 32768 batch).  Larger
// row tiles need their registers (forcing occupancy there spills).
template <int D, int RT, int W, int KS>
__global__ __launch_bounds__(64 * W * KS)
__attribute__((amdgpu_waves_per_eu(RT == 1 ? SV_MFMA_WAVES_PER_EU : 1)))
void attn_mfma_kernel(AttnArgs a) {
  constexpr int KT = kMfmaKeys;
  constexpr int KSTR = D + 8;        // bf16 per K row in LDS (+16 B: conflict-free b128 reads)
  constexpr int VSTR = D + 16;       // bf16 per V row in LDS (+32 B: conflict-free tr16 reads)
  constexpr int DT = D / 16;
  constexpr int KK = D / 32;
  constexpr int CPR = D / 8;         // 16-byte chunks per key row
  constexpr int NCH = KT * CPR;      // chunks per tile and tensor
  constexpr int NPT = (NCH + 64 * W - 1) / (64 * W);
  constexpr int TILE_BYTES = KT * (KSTR + VSTR) * 2;
  static_assert(KS == 1 || KS == 2, "key streams per block");
  // stream 1's final state goes through LDS: W waves x RT tiles x DT f32x4 x 64 lanes, + (m, l)
  static_assert(KS == 1 || W * RT * (DT * 64 * 16 + 64 * 8) <= KS * TILE_BYTES, "merge buffer");

  // Per key stream: a K tile and a V tile.  The buffer is reused at the end
  // to hand stream 1's state to stream 0.
  __shared__ __attribute__((aligned(16))) uint8_t tiles[KS * TILE_BYTES];
  __shared__ int par[64];
  __shared__ uint64_t masks[64];

  const int s = blockIdx.x, u = blockIdx.y, rc = blockIdx.z;
  const int b = u / a.Hkv, gk = u % a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
  const int ks = wave / W, wr = wave % W;                       // key stream, row wave
  const int stid = tid - ks * 64 * W;                           // thread within the stream
  const int l16 = lane & 15, g4 = lane >> 4;
  const int tile0 = (rc * W + wr) * RT;
  uint16_t* Ks = (uint16_t*)(tiles + ks * TILE_BYTES);
  uint16_t* Vs = Ks + KT * KSTR;

  build_masks(a, b, par, masks);

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
  // Q stays in registers for the whole key loop: wait for it here.
#if SV_SETTLE_MFMA
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) settle(__builtin_bit_cast(u32x4_t, qf[rt][kk]));
#endif

  f32x4_t acc[RT][DT];
  float m[RT], lpart[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m[rt] = kNegInf;
    lpart[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[rt][dt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  }

  // The block's keys [kb, ke) are cut into KS contiguous, tile-aligned parts.
  const int kb = s * a.chunk, ke = min(a.L, kb + a.chunk);
  const int ntiles = (ke - kb + KT - 1) / KT;
  const int tps = (ntiles + KS - 1) / KS;                       // tiles per stream
  const int sb = min(ke, kb + ks * tps * KT), se = min(ke, sb + tps * KT);
  const size_t unit_off = (size_t)u * a.L * D;
  const uint16_t* kg = (const uint16_t*)a.k + unit_off;
  const uint16_t* vg = (const uint16_t*)a.v + unit_off;
  const float c = a.scale_log2;
  const int clean_end = min(a.ctx, se);   // tiles ending here need no mask

  // Register staging: chunk i*64W + stid of the tile, 16 lanes per key row.
  // Keys past the end are clamped to the last row (finite data, masked later).
  u32x4_t kreg[NPT], vreg[NPT];
  auto load_tile = [&](int base) {
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int ch = i * 64 * W + stid;
      if (NCH % (64 * W) == 0 || (i * W + wr) * 64 < NCH) {   // uniform per wave
        const int key = min(base + ch / CPR, a.L - 1);
        const uint32_t off = (uint32_t)(key * D + 8 * (ch % CPR));
        kreg[i] = *(const u32x4_t*)(kg + off);
        vreg[i] = *(const u32x4_t*)(vg + off);
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int ch = i * 64 * W + stid;
      if (NCH % (64 * W) == 0 || (i * W + wr) * 64 < NCH) {
        const int kr = ch / CPR, kc = ch % CPR;
        *(u32x4_t*)(Ks + kr * KSTR + 8 * kc) = kreg[i];
        *(u32x4_t*)(Vs + kr * VSTR + 8 * kc) = vreg[i];
      }
    }
  };

  // Transposed-read addresses of this lane for V fragment halves: lane j of a
  // 16-lane group points at V[key(j/4)][16dt + 4(j%4) .. +4]; the hardware
  // hands lane i the four keys' values at d = 16dt + i.
  const int vkey0 = pv_key(g4, l16 >> 2), vkey1 = pv_key(g4, 4 + (l16 >> 2));
  const int vcol = 4 * (l16 & 3);

  if (sb < se) load_tile(sb);
  // Every stream runs tps iterations so that all waves meet at each barrier.
  for (int it = 0; it < tps; ++it) {
    const int base = sb + it * KT;
    const bool active = base < se;                              // uniform per stream
    __syncthreads();
    if (active) store_tile();
    __syncthreads();
    if (!active) continue;
    if (base + KT < se) load_tile(base + KT);

    // S^T for the tile's two 16-key halves.
    f32x4_t st[RT][2];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) st[rt][0] = st[rt][1] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const bf16x8_t kf = __builtin_bit_cast(
            bf16x8_t, *(const u32x4_t*)(Ks + (16 * sub + l16) * KSTR + 32 * kk + 8 * g4));
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)   // a dead tile (zero Q) computes harmless values
          st[rt][sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[rt][kk], st[rt][sub],
                                                               0, 0, 0);
      }
    }

    // Online softmax in log2 units with a lazily refreshed reference max.
    const bool clean = base + KT <= clean_end;
    bf16x8_t pf[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float sc[8];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[4 * sub + r] = st[rt][sub][r];
      if (!clean) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int key = base + (e < 4 ? 4 * g4 + e : 16 + 4 * g4 + e - 4);
          if (!(key < se && tail_visible(mrow[rt], key, a.ctx))) sc[e] = kNegInf;
        }
      }
      float mt = sc[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mt = fmaxf(mt, sc[e]);
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      mt *= c;                                  // scale > 0: max commutes with scaling
      const bool bump = mt > m[rt] + kRescaleLog2;
      if (__any(bump)) {
        // lanes that keep their reference (possibly -inf) must not compute -inf - -inf
        const float alpha = bump ? fast_exp2(m[rt] - mt) : 1.f;   // m = -inf: 0
        if (bump) m[rt] = mt;
        lpart[rt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[rt][dt] *= alpha;
      }
      const float msafe = (m[rt] == kNegInf) ? 0.f : m[rt];
      float ps = 0.f;
      bf16x2_t pk[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float p0 = fast_exp2(fmaf(sc[e], c, -msafe));
        const float p1 = fast_exp2(fmaf(sc[e + 1], c, -msafe));
        ps += p0 + p1;
        pk[e / 2] = __builtin_convertvector((f32x2_t){p0, p1}, bf16x2_t);
      }
      lpart[rt] += ps;
      pf[rt] = __builtin_shufflevector(__builtin_shufflevector(pk[0], pk[1], 0, 1, 2, 3),
                                       __builtin_shufflevector(pk[2], pk[3], 0, 1, 2, 3),
                                       0, 1, 2, 3, 4, 5, 6, 7);
    }

    // O^T += V^T P^T.
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4_t*)(Vs + vkey0 * VSTR + 16 * dt + vcol));
      const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4_t*)(Vs + vkey1 * VSTR + 16 * dt + vcol));
      const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3,
                                                                               4, 5, 6, 7));
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        acc[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[rt], acc[rt][dt], 0, 0, 0);
    }
  }

  // Row sums over the four lane groups (every lane of a row gets the total).
  float lt[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    lt[rt] = lpart[rt];
    lt[rt] += __shfl_xor(lt[rt], 16);
    lt[rt] += __shfl_xor(lt[rt], 32);
  }

  if constexpr (KS == 2) {
    // Stream 1 hands its state to stream 0 through LDS (same row wave, same
    // lane, same layout), and stream 0 merges the two.
    __syncthreads();
    f32x4_t* xo = (f32x4_t*)tiles;
    float* xm = (float*)(tiles + W * RT * DT * 64 * 16);
    if (ks == 1) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) xo[((wr * RT + rt) * DT + dt) * 64 + lane] = acc[rt][dt];
        xm[((wr * RT + rt) * 64 + lane) * 2] = m[rt];
        xm[((wr * RT + rt) * 64 + lane) * 2 + 1] = lt[rt];
      }
    }
    __syncthreads();
    if (ks == 1) return;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float m2 = xm[((wr * RT + rt) * 64 + lane) * 2];
      const float l2 = xm[((wr * RT + rt) * 64 + lane) * 2 + 1];
      const float mx = fmaxf(m[rt], m2);
      if (mx == kNegInf) continue;
      const float a1 = fast_exp2(m[rt] - mx), a2 = fast_exp2(m2 - mx);
      lt[rt] = lt[rt] * a1 + l2 * a2;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        acc[rt][dt] = acc[rt][dt] * a1 + xo[((wr * RT + rt) * DT + dt) * 64 + lane] * a2;
      m[rt] = mx;
    }
  }

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
// Split combine: block per (row, unit), one thread per d.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(128) void attn_combine_kernel(AttnArgs a) {
  const int row = blockIdx.x, u = blockIdx.y, d = threadIdx.x;
  const int b = u / a.Hkv, gk = u % a.Hkv;
  const int t = row / a.G, h = gk * a.G + row % a.G;
  const size_t base = (size_t)u * a.S * a.R + row;
  float mx = kNegInf;
  for (int s = 0; s < a.S; ++s) mx = fmaxf(mx, a.part_ml[(base + (size_t)s * a.R) * 2]);
  float num = 0.f, den = 0.f;
  for (int s = 0; s < a.S; ++s) {
    const size_t p = base + (size_t)s * a.R;
    const float ms = a.part_ml[p * 2];
    if (ms == kNegInf) continue;
    const float w = fast_exp2(ms - mx);
    den = fmaf(w, a.part_ml[p * 2 + 1], den);
    num = fmaf(w, a.part_o[p * a.D + d], num);
  }
  a.out[(((size_t)b * a.T + t) * a.Hq + h) * a.D + d] = num / den;
}

// ---------------------------------------------------------------------------
// Host-side dispatch.
// ---------------------------------------------------------------------------
template <int D, int RT>
static void launch_mfma_w(const AttnPlan& p, const AttnArgs& a, hipStream_t st, dim3 grid) {
  switch (p.waves) {
    case 1: attn_mfma_kernel<D, RT, 1, 1><<<grid, 64, 0, st>>>(a); break;
    case 2: attn_mfma_kernel<D, RT, 2, 1><<<grid, 128, 0, st>>>(a); break;
    case 3: attn_mfma_kernel<D, RT, 3, 1><<<grid, 192, 0, st>>>(a); break;
    case 4: attn_mfma_kernel<D, RT, 4, 1><<<grid, 256, 0, st>>>(a); break;
    case 5: attn_mfma_kernel<D, RT, 5, 1><<<grid, 320, 0, st>>>(a); break;
    case 6: attn_mfma_kernel<D, RT, 6, 1><<<grid, 384, 0, st>>>(a); break;
    case 7: attn_mfma_kernel<D, RT, 7, 1><<<grid, 448, 0, st>>>(a); break;
    default: attn_mfma_kernel<D, RT, 8, 1><<<grid, 512, 0, st>>>(a); break;
  }
}

template <int D, int KS>
static void launch_mfma_rt(const AttnPlan& p, const AttnArgs& a, hipStream_t st, dim3 grid) {
  switch (p.rt) {
    case 1: launch_mfma_w<D, 1>(p, a, st, grid); break;
    case 2: launch_mfma_w<D, 2>(p, a, st, grid); break;
    default: launch_mfma_w<D, 3>(p, a, st, grid); break;
  }
}

template <int D>
static void launch_mfma(const AttnPlan& p, const AttnArgs& a, hipStream_t st, dim3 grid) {
  // two key streams are planned only with one row tile per wave and <= 4 row waves
  if (p.kstreams == 2) {
    switch (p.waves) {
      case 1: attn_mfma_kernel<D, 1, 1, 2><<<grid, 128, 0, st>>>(a); break;
      case 2: attn_mfma_kernel<D, 1, 2, 2><<<grid, 256, 0, st>>>(a); break;
      case 3: attn_mfma_kernel<D, 1, 3, 2><<<grid, 384, 0, st>>>(a); break;
      default: attn_mfma_kernel<D, 1, 4, 2><<<grid, 512, 0, st>>>(a); break;
    }
  } else {
    launch_mfma_rt<D, 1>(p, a, st, grid);
  }
}

template <typename TIn, int D>
static void launch_valu(const AttnPlan& p, const AttnArgs& a, hipStream_t st, dim3 grid) {
  switch (p.rmax) {
    case 1: attn_valu_kernel<TIn, D, 1><<<grid, 256, 0, st>>>(a); break;
    case 2: attn_valu_kernel<TIn, D, 2><<<grid, 256, 0, st>>>(a); break;
    case 4: attn_valu_kernel<TIn, D, 4><<<grid, 256, 0, st>>>(a); break;
    default: attn_valu_kernel<TIn, D, 8><<<grid, 256, 0, st>>>(a); break;
  }
}

// Splits and tiles for a problem; a pure function of the shape so that the
// workspace query and the launch always agree.  The block targets aim at one
// full wave of resident blocks on the 256 CUs.
#ifndef SV_MFMA_BLOCKS
#define SV_MFMA_BLOCKS 1024
#endif
#ifndef SV_VALU_BLOCKS
#define SV_VALU_BLOCKS 512
#endif
#ifndef SV_MIN_CHUNK
#define SV_MIN_CHUNK 256
#endif
#ifndef SV_FUSE_UNITS
#define SV_FUSE_UNITS 512
#endif
AttnPlan plan_attention(int B, int T, int Hq, int Hkv, int D, int ctx, int bf16) {
  AttnPlan p{};
  const int G = Hq / Hkv, R = G * T, L = ctx + T, units = B * Hkv;
  p.rows = R;
  p.mfma = bf16 && R >= 16;
  int tile, blocks_target;
  if (p.mfma) {
    const int tiles = (R + 15) / 16;
    // one to three 16-row tiles per wave, at most 8 waves; the rest in row chunks
    p.rt = tiles <= 8 ? 1 : tiles <= 16 ? 2 : 3;
    int waves = (tiles + p.rt - 1) / p.rt;
    p.row_chunks = (waves + 7) / 8;
    p.waves = (waves + p.row_chunks - 1) / p.row_chunks;
    // With enough (sequence, KV head) units to fill the chip, one block holds
    // two key streams and merges them itself: one launch, no partials.
    p.kstreams = 1;
    if (p.waves <= 4 && units * p.row_chunks >= SV_FUSE_UNITS) p.kstreams = 2;
    tile = kMfmaKeys;
    blocks_target = SV_MFMA_BLOCKS;
  } else {
    const int rr = R < 8 ? R : 8;
    p.rmax = rr <= 1 ? 1 : rr <= 2 ? 2 : rr <= 4 ? 4 : 8;
    p.waves = 4;
    p.row_chunks = (R + p.rmax - 1) / p.rmax;
    tile = 64;
    blocks_target = SV_VALU_BLOCKS;
  }
  const int min_chunk = SV_MIN_CHUNK;
  int S = (blocks_target + units * p.row_chunks - 1) / (units * p.row_chunks);
  if (p.mfma && p.kstreams == 2) S = 1;
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
                            hipStream_t st) {
  AttnArgs a;
  a.q = q; a.k = k; a.v = v; a.parents = parents; a.out = out;
  a.part_o = (float*)workspace;
  a.part_ml = (float*)((char*)workspace + p.part_o_bytes);
  a.B = B; a.T = T; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv; a.D = D; a.ctx = ctx;
  a.L = ctx + T; a.R = p.rows; a.S = p.splits; a.chunk = p.chunk;
  a.scale_log2 = scale * kLog2e;
  const dim3 grid(p.splits, B * Hkv, p.row_chunks);
  if (p.mfma) {
    if (D == 64) launch_mfma<64>(p, a, st, grid);
    else launch_mfma<128>(p, a, st, grid);
  } else if (bf16) {
    if (D == 64) launch_valu<uint16_t, 64>(p, a, st, grid);
    else launch_valu<uint16_t, 128>(p, a, st, grid);
  } else {
    if (D == 64) launch_valu<float, 64>(p, a, st, grid);
    else launch_valu<float, 128>(p, a, st, grid);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || (p.mfma && p.splits == 1)) return e;
  attn_combine_kernel<<<dim3(p.rows, B * Hkv), D, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace sv
