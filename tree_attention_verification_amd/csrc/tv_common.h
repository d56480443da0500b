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

// Largest supported padded node count (one wavefront lane per node).
constexpr int kTMaxLimit = 64;
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

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    unsigned long long o = shfl_xor_u64(v, m);
    v = o > v ? o : v;
  }
  return v;
}

}  // namespace tv
