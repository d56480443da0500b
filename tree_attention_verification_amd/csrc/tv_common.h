// Internal helpers shared by the HIP translation units of libtreeverify.so.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/treeverify.h"

#define TV_CHECK_LAUNCH()                                   \
  do {                                                      \
    if (hipGetLastError() != hipSuccess) return TV_ELAUNCH; \
  } while (0)

namespace tv {

// Paged K/V cache (the TensorRT-LLM EAGLE-3 dissection, "after acceptance: KV
// from tree layout back to linear": a token's physical slot is its request's
// block-table entry plus the offset inside the block).  Pools are
// [n_blocks][Hkv][1 << lbs][d]; logical row s of request b is row
// s & ((1 << lbs) - 1) of block table[b * max_blocks + (s >> lbs)] (kv head g's
// rows of a block are contiguous).  A null table means the linear cache
// [B][Hkv][S_cap][d].
struct Paging {
  const int* table;
  int max_blocks;      // table row stride (blocks per request)
  int lbs;             // log2 of tokens per block
  long long n_blocks;  // blocks in each pool
};

// log2 of a power of two in [1, 1024], else -1 (host)
inline int log2_block(int tokens_per_block) {
  for (int l = 0; l <= 10; ++l)
    if (tokens_per_block == (1 << l)) return l;
  return -1;
}

// Largest supported padded node count: one wavefront lane per node up to 64,
// one workgroup thread per node up to 256.
constexpr int kTMaxLimit = 256;
// Largest supported top_k (per-thread register lists).
constexpr int kKMax = 16;

// Order-preserving map of a float to uint32 (larger float -> larger key);
// -0.0 is first canonicalised to +0.0 so both rank equal.
__device__ __forceinline__ uint32_t order_key(float v) {
  if (v == 0.0f) v = 0.0f;
  uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// 64-bit rank key: value descending, then index ascending (max key = best).
__device__ __forceinline__ unsigned long long rank_key(float v, uint32_t idx) {
  return ((unsigned long long)order_key(v) << 32) | (unsigned long long)(0xFFFFFFFFu - idx);
}

__device__ __forceinline__ uint32_t key_index(unsigned long long k) {
  return 0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull);
}

__device__ __forceinline__ float key_value(unsigned long long k) {
  uint32_t o = (uint32_t)(k >> 32);
  uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int m) {
  int lo = __shfl_xor((int)(uint32_t)v, m, 64);
  int hi = __shfl_xor((int)(uint32_t)(v >> 32), m, 64);
  return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}

// DPP lane moves (VALU-rate, no LDS round trip).  Control codes: quad_perm
// [1,0,3,2] = 0xB1 (lane ^ 1), quad_perm [2,3,0,1] = 0x4E (lane ^ 2),
// row_half_mirror = 0x141 (lane i <-> 7 - i within 8), row_mirror = 0x140
// (lane i <-> 15 - i within 16).
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long v) {
  const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ unsigned long long umax64(unsigned long long a, unsigned long long b) { return a > b ? a : b; }

// max over aligned groups of G lanes (G = 1, 2, 4, 8, 16); every lane gets its group's max
template <int G>
__device__ __forceinline__ unsigned long long group_max_u64(unsigned long long v) {
  if (G >= 2) v = umax64(v, dpp_u64<0xB1>(v));
  if (G >= 4) v = umax64(v, dpp_u64<0x4E>(v));
  if (G >= 8) v = umax64(v, dpp_u64<0x141>(v));
  if (G >= 16) v = umax64(v, dpp_u64<0x140>(v));
  return v;
}

__device__ __forceinline__ unsigned long long readlane_u64(unsigned long long v, int lane) {
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, lane);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
  return ((unsigned long long)hi << 32) | lo;
}

// max over the whole wavefront: 16-lane groups by DPP, then the four group maxima
// combined through scalar registers
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
  v = group_max_u64<16>(v);
  return umax64(umax64(readlane_u64(v, 0), readlane_u64(v, 16)), umax64(readlane_u64(v, 32), readlane_u64(v, 48)));
}

}  // namespace tv
