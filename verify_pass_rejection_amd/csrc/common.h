// Device helpers and launch-plan structures shared by the verify-step kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

namespace sv {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// ---- bf16 <-> fp32 ---------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even fp32 -> bf16 for finite values (probabilities here).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// ---- lane exchanges without LDS (64-lane waves) -----------------------------
// DPP inside a row of 16 lanes: quad_perm [1,0,3,2] (lane ^ 1), [2,3,0,1]
// (lane ^ 2), row_half_mirror (lane ^ 7 within 8), row_mirror (lane ^ 15),
// row_ror:8 (lane ^ 8); row_shr:n shifts by n inside the row, row_bcast:15 /
// row_bcast:31 broadcast lane 15 of a row to the next / lane 31 to rows 2
// and 3, wave_shr:1 shifts the whole wave by one lane.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppXor7 = 0x141, kDppXor15 = 0x140;
constexpr int kDppXor8 = 0x128, kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114;
constexpr int kDppShr8 = 0x118, kDppBcast15 = 0x142, kDppBcast31 = 0x143, kDppWaveShr1 = 0x138;

// The value of the lane that DPP control C names.
template <int C>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), C, 0xf, 0xf, false));
}
template <int C>
__device__ __forceinline__ double dpp_d(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)u, C, 0xf, 0xf, false);
  const uint32_t hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), C, 0xf, 0xf, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
// The same, with 0 where there is no source lane (shifted in from outside the
// row or the wave, or a row that row mask R leaves out).
template <int C, int R = 0xf>
__device__ __forceinline__ float dpp_f0(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), C, R, 0xf, true));
}
template <int C, int R = 0xf>
__device__ __forceinline__ double dpp_d0(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, C, R, 0xf, true);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), C, R, 0xf, true);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// gfx950 row swaps: permlane16 exchanges rows 1, 3 of its first operand with
// rows 0, 2 of its second, permlane32 the upper half of the first with the
// lower half of the second.  row_pair: for every lane, the value of x in the
// lower and in the upper row (half, P32) of the lane's pair of rows (halves).
template <bool P32>
__device__ __forceinline__ void row_pair(float x, float& lo, float& hi) {
  const auto r = P32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                        false, false)
                     : __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                        false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}
// swap_sum(a, b): a[l] + a[l ^ 16] (a[l] + a[l ^ 32] for P32) in lanes whose
// bit 4 (bit 5) is clear, b[l] + b[l ^ 16] (b[l] + b[l ^ 32]) in the others.
template <bool P32>
__device__ __forceinline__ double swap_sum(double a, double b) {
  const uint64_t ua = __builtin_bit_cast(uint64_t, a), ub = __builtin_bit_cast(uint64_t, b);
  const uint32_t alo = (uint32_t)ua, ahi = (uint32_t)(ua >> 32);
  const uint32_t blo = (uint32_t)ub, bhi = (uint32_t)(ub >> 32);
  const auto rl = P32 ? __builtin_amdgcn_permlane32_swap(alo, blo, false, false)
                      : __builtin_amdgcn_permlane16_swap(alo, blo, false, false);
  const auto rh = P32 ? __builtin_amdgcn_permlane32_swap(ahi, bhi, false, false)
                      : __builtin_amdgcn_permlane16_swap(ahi, bhi, false, false);
  const double x = __builtin_bit_cast(double, ((uint64_t)(uint32_t)rh[0] << 32) | (uint32_t)rl[0]);
  const double y = __builtin_bit_cast(double, ((uint64_t)(uint32_t)rh[1] << 32) | (uint32_t)rl[1]);
  return x + y;
}

// Sum over the wave, the same value in every lane (every step adds one pair of
// lanes' values, which both lanes of the pair then hold).
__device__ __forceinline__ double wave_sum(double x) {
  x += dpp_d<kDppXor1>(x);
  x += dpp_d<kDppXor2>(x);
  x += dpp_d<kDppXor7>(x);
  x += dpp_d<kDppXor15>(x);
  x = swap_sum<false>(x, x);
  return swap_sum<true>(x, x);
}
// Maximum over the wave, in every lane.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f<kDppXor1>(x));
  x = fmaxf(x, dpp_f<kDppXor2>(x));
  x = fmaxf(x, dpp_f<kDppXor7>(x));
  x = fmaxf(x, dpp_f<kDppXor15>(x));
  float lo, hi;
  row_pair<false>(x, lo, hi);
  x = fmaxf(lo, hi);
  row_pair<true>(x, lo, hi);
  return fmaxf(lo, hi);
}
// Maximum of unsigned 64-bit keys over the wave, in every lane.
__device__ __forceinline__ uint64_t wave_max(uint64_t x) {
  auto step = [](uint64_t v, uint64_t y) { return y > v ? y : v; };
  auto dpp = [](uint64_t v, auto c) {
    constexpr int C = decltype(c)::value;
    const uint32_t lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)v, C, 0xf, 0xf, false);
    const uint32_t hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), C, 0xf, 0xf, false);
    return ((uint64_t)hi << 32) | lo;
  };
  x = step(x, dpp(x, std::integral_constant<int, kDppXor1>{}));
  x = step(x, dpp(x, std::integral_constant<int, kDppXor2>{}));
  x = step(x, dpp(x, std::integral_constant<int, kDppXor7>{}));
  x = step(x, dpp(x, std::integral_constant<int, kDppXor15>{}));
  auto rl = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
  auto rh = __builtin_amdgcn_permlane16_swap((uint32_t)(x >> 32), (uint32_t)(x >> 32), false, false);
  x = step(((uint64_t)(uint32_t)rh[0] << 32) | (uint32_t)rl[0],
           ((uint64_t)(uint32_t)rh[1] << 32) | (uint32_t)rl[1]);
  rl = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
  rh = __builtin_amdgcn_permlane32_swap((uint32_t)(x >> 32), (uint32_t)(x >> 32), false, false);
  return step(((uint64_t)(uint32_t)rh[0] << 32) | (uint32_t)rl[0],
              ((uint64_t)(uint32_t)rh[1] << 32) | (uint32_t)rl[1]);
}
// Minimum over the wave, in every lane.
__device__ __forceinline__ int wave_min(int x) {
  x = min(x, __builtin_amdgcn_mov_dpp(x, kDppXor1, 0xf, 0xf, false));
  x = min(x, __builtin_amdgcn_mov_dpp(x, kDppXor2, 0xf, 0xf, false));
  x = min(x, __builtin_amdgcn_mov_dpp(x, kDppXor7, 0xf, 0xf, false));
  x = min(x, __builtin_amdgcn_mov_dpp(x, kDppXor15, 0xf, 0xf, false));
  auto r = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
  x = min((int)r[0], (int)r[1]);
  r = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
  return min((int)r[0], (int)r[1]);
}
// Inclusive prefix sum over the wave in lane order: shifts by 1, 2, 4 and 8
// inside each row, then row 0's total into row 1 and row 2's into row 3, then
// the total of lanes 0..31 into rows 2 and 3.
__device__ __forceinline__ double wave_scan(double x) {
  x += dpp_d0<kDppShr1>(x);
  x += dpp_d0<kDppShr2>(x);
  x += dpp_d0<kDppShr4>(x);
  x += dpp_d0<kDppShr8>(x);
  x += dpp_d0<kDppBcast15, 0xa>(x);
  x += dpp_d0<kDppBcast31, 0xc>(x);
  return x;
}
__device__ __forceinline__ float wave_scan(float x) {
  x += dpp_f0<kDppShr1>(x);
  x += dpp_f0<kDppShr2>(x);
  x += dpp_f0<kDppShr4>(x);
  x += dpp_f0<kDppShr8>(x);
  x += dpp_f0<kDppBcast15, 0xa>(x);
  x += dpp_f0<kDppBcast31, 0xc>(x);
  return x;
}
// The previous lane's value, 0 in lane 0.
__device__ __forceinline__ double wave_prev(double x) { return dpp_d0<kDppWaveShr1>(x); }
__device__ __forceinline__ float wave_prev(float x) { return dpp_f0<kDppWaveShr1>(x); }

// 2^x on the hardware transcendental unit.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- launch plans -------------------------------------------------------------
struct AttnPlan {
  int mfma;        // 1: bf16 MFMA kernel, 0: VALU kernel
  int rows;        // R = G * T grouped rows per KV head
  int rmax;        // VALU: rows handled per block (1, 2, 4 or 8)
  int rt;          // MFMA: 16-row tiles per wave (1..4)
  int waves;       // waves per block (MFMA: compute waves, plus one loader wave)
  int row_chunks;  // blocks along the row axis
  int splits;      // S: key-range splits per (sequence, KV head)
  int chunk;       // keys per split (multiple of the kernel's key tile)
  size_t part_o_bytes, part_ml_bytes, total_bytes;
};

struct ChainPlan {
  int rows_per_seq;  // 2N + 1
  int chunk;         // logits per stats block
  int nchunks;       // stats chunks per row
  int dchunks;       // draw chunks per row
  int cpb;           // draw chunks per chain_chunks block: 1, or more on large batches
  size_t stats_bytes, csum_bytes, decision_bytes, total_bytes;
};

struct TreePlan {
  int chunk;
  int nchunks;
  size_t part_bytes, total_bytes;
};

struct STreePlan {
  int nchunks;     // 8192-logit statistics chunks per row
  size_t s_bytes, m_bytes, g_bytes, total_bytes;
};

struct NgramPlan {
  int tiles;       // 4096-position tiles per sequence
  size_t total_bytes;
};

// A paged KV cache (see AttnArgs): position i of sequence b is row
// i % page_size of page block_table[b][i / page_size].
struct PagedKV {
  const int32_t* block_table;  // [B, max_blocks]
  const int32_t* ctx_lens;     // [B] or nullptr
  int page_size;               // a power of two
  int max_blocks, num_pages;
  int position_major;          // 0: [pages, Hkv, page_size, D]; 1: [pages, page_size, Hkv, D]
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Size of the static scratch array of the allocation-free chain acceptance
// (one per GPU; it holds the workspace spec_accept_chain would take).
constexpr size_t kChainScratchBytes = size_t(4) << 20;
constexpr int kMaxScratchDevices = 64;

}  // namespace sv
