// Device helpers and launch-plan structures shared by the verify-step kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

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

// ---- wave-level reductions (64 lanes) ---------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

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
  size_t s_bytes, m_bytes, total_bytes;
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
