// The per-request part of tree_mask_positions, shared by its own kernel and by
// the tree-build kernel that also produces the metadata (one wavefront, lane i =
// node i, T_max <= 64).  See tree_meta.hip for what is computed and why.
#pragma once
#include "tv_common.h"

namespace tv {
namespace {

// LDS written by any lane of this wavefront is visible to every lane after this
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ unsigned long long shfl_u64(unsigned long long v, int src) {
  int lo = __shfl((int)(uint32_t)v, src, 64);
  int hi = __shfl((int)(uint32_t)(v >> 32), src, 64);
  return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}

struct Anc {
  unsigned long long mask;
  int depth;
};

// Ancestor mask of lane i in a tree of T nodes with parent p (lanes >= T: 0).
__device__ __forceinline__ Anc ancestors(int i, int T, int p) {
  unsigned long long m = i < T ? (1ull << i) : 0ull;
  int a = (i < T && i > 0) ? p : -1;
  for (int r = 0; r < 6; ++r) {
    if (!__ballot(a >= 0)) break;  // every lane reached the root (depth < 2^r)
    const unsigned long long ma = shfl_u64(m, a < 0 ? i : a);
    const int aa = __shfl(a, a < 0 ? i : a, 64);
    if (a >= 0) {
      m |= ma;
      a = aa;
    }
  }
  return {m, (int)__popcll(m) - 1};
}

// The checks of tree_mask_positions on a tree of (claimed) size T with status
// st, lane i's parent entry p_l: T out of range -> size status; a parent that is
// not an earlier node (or a root with a parent) -> parents status.  Any bad
// status leaves the root alone (T = 1).  Returns this lane's parent (-1 for the
// root and lanes past the tree).
__device__ __forceinline__ int check_tree(int i, int T_max, int& st, int& T, int p_l) {
  if (st == TV_ST_OK && (T < 1 || T > T_max)) st = TV_ST_SIZE;
  int p = -1;
  if (st == TV_ST_OK) {
    p = i < T ? p_l : -1;
    const bool bad = (i == 0) ? (p != -1) : (i < T && !(p >= 0 && p < i));
    if (__ballot(bad)) st = TV_ST_PARENTS;
  }
  if (st != TV_ST_OK) {
    T = 1;
    p = -1;
  }
  return p;
}

// Where the metadata goes (the output arguments of tree_mask_positions).
struct MetaOut {
  int dcap, W;
  const int* prefix_len;
  uint32_t* tree_mask;
  int* tree_position_ids;
  int* positions;
  int* retrieve_indices;
  int* leaf_count;
  int* first_child;   // nullable
  int* next_sibling;  // nullable
};

// Request b's metadata from its tree size T, status st and this lane's parent
// p (already checked: p < i for 0 < i < T, p = -1 otherwise, and T = 1, p = -1
// when st is not ok).  Writes every output row of the request.
__device__ __forceinline__ void meta_body(int b, int i, int T_max, int dcap, int W, int T, int st, int p, int P,
                                          uint32_t* __restrict__ tree_mask, int* __restrict__ tree_position_ids,
                                          int* __restrict__ positions, int* __restrict__ retrieve_indices,
                                          int* __restrict__ leaf_count, int* __restrict__ first_child,
                                          int* __restrict__ next_sibling, int* __restrict__ status_out) {
  const long long ob = (long long)b * T_max;
  Anc an = ancestors(i, T, p);
  if (st == TV_ST_OK && __ballot(i < T && an.depth > dcap)) {
    st = TV_ST_DEPTH;
    T = 1;
    p = -1;
    an = ancestors(i, T, p);
  }
  const bool in = i < T;

  // packed mask row i: bit j&31 of word j>>5
  if (i < T_max) {
    for (int w = 0; w < W; ++w) tree_mask[(ob + i) * W + w] = in ? (uint32_t)(an.mask >> (32 * w)) : 0u;
    tree_position_ids[ob + i] = in ? an.depth : 0;
    positions[ob + i] = in ? P + an.depth : 0;
  }

  // children in ascending id: every node sets its bit in its parent's child mask
  // (one LDS atomic per node); the first child of i is the lowest bit of i's mask,
  // the next sibling of i the lowest bit of its parent's mask above i
  __shared__ unsigned long long s_cm[64];
  s_cm[i] = 0ull;
  wave_sync();
  if (in && i > 0) atomicOr(&s_cm[p], 1ull << i);
  wave_sync();
  const unsigned long long cm = in ? s_cm[i] : 0ull;
  const int fc = cm ? __ffsll((long long)cm) - 1 : -1;
  int ns = -1;
  if (in && i > 0) {
    const unsigned long long later = s_cm[p] & ~((2ull << i) - 1ull);  // i = 63: 2 << 63 wraps to 0, no bits
    ns = later ? __ffsll((long long)later) - 1 : -1;
  }
  if (i < T_max) {
    if (first_child) first_child[ob + i] = fc;
    if (next_sibling) next_sibling[ob + i] = ns;
  }

  // leaves (no child), ranked by id; retrieve row r = path of the r-th leaf
  const bool leaf = in && fc == -1;
  const unsigned long long lb = __ballot(leaf);
  const int nleaf = __popcll(lb);
  __shared__ int s_leaf[64];
  if (leaf) s_leaf[__popcll(lb & ((1ull << i) - 1ull))] = i;
  wave_sync();
  // every lane needs the mask of leaf s_leaf[i]: fetch with a shuffle from that lane
  const int src = i < nleaf ? s_leaf[i] : i;
  const unsigned long long lm = shfl_u64(an.mask, src);
  if (i < T_max) {
    int* row = retrieve_indices + (ob + i) * (dcap + 1);
    unsigned long long m = i < nleaf ? lm : 0ull;
    for (int k = 0; k <= dcap; ++k) {
      int v = -1;
      if (m) {
        v = __ffsll((long long)m) - 1;  // ancestors in ascending id = ascending depth
        m &= m - 1ull;
      }
      row[k] = v;
    }
  }
  if (i == 0) {
    leaf_count[b] = nleaf;
    status_out[b] = st;
  }
}

}  // namespace
}  // namespace tv

// ---------------------------------------------------------------------------
// Trees of up to 256 nodes (T_max in (64, 256]): the same metadata computed by a
// 256-thread workgroup, thread i = node i, each ancestor set a 256-bit mask of
// four 64-bit words.  Pointer jumping runs through LDS (a round reads the jump
// target's mask and pointer, then all threads write theirs), eight rounds at most.
// ---------------------------------------------------------------------------
namespace tv {
namespace {

constexpr int kWideNodes = 256;
constexpr int kWideWords = kWideNodes / 64;

struct WideShared {
  unsigned long long m[kWideNodes][kWideWords];   // ancestor masks (final)
  unsigned long long cm[kWideNodes][kWideWords];  // child masks
  int a[kWideNodes];                              // jump pointers
  int leaf[kWideNodes];
  int cnt[kWideNodes / 64];
  int flag;
};

// block-wide OR of a predicate (every thread of the 256 gets it)
__device__ __forceinline__ bool block_any_wide(bool v, int* s_flag) {
  __syncthreads();
  if (threadIdx.x == 0) *s_flag = 0;
  __syncthreads();
  if (v) *s_flag = 1;
  __syncthreads();
  return *s_flag != 0;
}

// The checks of check_tree for a 256-thread workgroup (thread i = node i).
__device__ __forceinline__ int check_tree_wide(int i, int T_max, int& st, int& T, int p_l, WideShared& sh) {
  if (st == TV_ST_OK && (T < 1 || T > T_max)) st = TV_ST_SIZE;
  int p = -1;
  bool bad = false;
  if (st == TV_ST_OK) {
    p = i < T ? p_l : -1;
    bad = (i == 0) ? (p != -1) : (i < T && !(p >= 0 && p < i));
  }
  if (block_any_wide(bad, &sh.flag)) st = TV_ST_PARENTS;
  if (st != TV_ST_OK) {
    T = 1;
    p = -1;
  }
  return p;
}

// Ancestor masks of every node (thread i = node i, parent p) into sh.m; returns depth.
__device__ __forceinline__ int ancestors_wide(int i, int T, int p, WideShared& sh, unsigned long long (&m)[kWideWords]) {
#pragma unroll
  for (int w = 0; w < kWideWords; ++w) m[w] = (i < T && (i >> 6) == w) ? (1ull << (i & 63)) : 0ull;
  int a = (i < T && i > 0) ? p : -1;
  for (int r = 0; r < 8; ++r) {
#pragma unroll
    for (int w = 0; w < kWideWords; ++w) sh.m[i][w] = m[w];
    sh.a[i] = a;
    if (!block_any_wide(a >= 0, &sh.flag)) break;  // block_any_wide starts with a barrier: the writes are visible
    unsigned long long ma[kWideWords];
    int aa = -1;
    if (a >= 0) {
      aa = sh.a[a];
#pragma unroll
      for (int w = 0; w < kWideWords; ++w) ma[w] = sh.m[a][w];
    }
    __syncthreads();  // every read of this round before the next round's writes
    if (a >= 0) {
#pragma unroll
      for (int w = 0; w < kWideWords; ++w) m[w] |= ma[w];
      a = aa;
    }
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kWideWords; ++w) sh.m[i][w] = m[w];
  __syncthreads();
  int pc = 0;
#pragma unroll
  for (int w = 0; w < kWideWords; ++w) pc += __popcll(m[w]);
  return pc - 1;
}

// meta_body for trees of up to 256 nodes: every thread of the 256-thread
// workgroup calls it with its node i.
__device__ __forceinline__ void meta_body_wide(int b, int i, int T_max, int dcap, int W, int T, int st, int p, int P,
                                               uint32_t* __restrict__ tree_mask,
                                               int* __restrict__ tree_position_ids, int* __restrict__ positions,
                                               int* __restrict__ retrieve_indices, int* __restrict__ leaf_count,
                                               int* __restrict__ first_child, int* __restrict__ next_sibling,
                                               int* __restrict__ status_out, WideShared& sh) {
  const long long ob = (long long)b * T_max;
  unsigned long long m[kWideWords];
  int depth = ancestors_wide(i, T, p, sh, m);
  if (st == TV_ST_OK && block_any_wide(i < T && depth > dcap, &sh.flag)) {
    st = TV_ST_DEPTH;
    T = 1;
    p = -1;
    depth = ancestors_wide(i, T, p, sh, m);
  }
  const bool in = i < T;
  if (i < T_max) {
    for (int w = 0; w < W; ++w) tree_mask[(ob + i) * W + w] = in ? (uint32_t)(m[w >> 1] >> (32 * (w & 1))) : 0u;
    tree_position_ids[ob + i] = in ? depth : 0;
    positions[ob + i] = in ? P + depth : 0;
  }
  // child masks: one LDS atomic per node into its parent's mask
#pragma unroll
  for (int w = 0; w < kWideWords; ++w) sh.cm[i][w] = 0ull;
  __syncthreads();
  if (in && i > 0) atomicOr(&sh.cm[p][i >> 6], 1ull << (i & 63));
  __syncthreads();
  int fc = -1, ns = -1;
  if (in) {
#pragma unroll
    for (int w = kWideWords - 1; w >= 0; --w)
      if (sh.cm[i][w]) fc = 64 * w + __ffsll((long long)sh.cm[i][w]) - 1;
    if (i > 0) {
      for (int w = kWideWords - 1; w >= (i >> 6); --w) {
        unsigned long long later = sh.cm[p][w];
        if (w == (i >> 6)) later &= (i & 63) == 63 ? 0ull : ~((2ull << (i & 63)) - 1ull);
        if (later) ns = 64 * w + __ffsll((long long)later) - 1;
      }
    }
  }
  if (i < T_max) {
    if (first_child) first_child[ob + i] = fc;
    if (next_sibling) next_sibling[ob + i] = ns;
  }
  // leaves ranked by id: per-wavefront ballots, then the wavefronts' counts
  const bool leaf = in && fc == -1;
  const unsigned long long lb = __ballot(leaf);
  const int lane = i & 63, wv = i >> 6;
  if (lane == 0) sh.cnt[wv] = __popcll(lb);
  __syncthreads();
  int before = 0, nleaf = 0;
  for (int w = 0; w < kWideNodes / 64; ++w) {
    if (w < wv) before += sh.cnt[w];
    nleaf += sh.cnt[w];
  }
  if (leaf) sh.leaf[before + __popcll(lb & ((1ull << lane) - 1ull))] = i;
  __syncthreads();
  if (i < T_max) {
    int* row = retrieve_indices + (ob + i) * (dcap + 1);
    unsigned long long lm[kWideWords];
    const int lf = i < nleaf ? sh.leaf[i] : -1;
#pragma unroll
    for (int w = 0; w < kWideWords; ++w) lm[w] = lf >= 0 ? sh.m[lf][w] : 0ull;
    int w = 0;
    for (int k = 0; k <= dcap; ++k) {
      while (w < kWideWords && lm[w] == 0ull) ++w;
      int v = -1;
      if (w < kWideWords) {
        v = 64 * w + __ffsll((long long)lm[w]) - 1;  // ancestors in ascending id = ascending depth
        lm[w] &= lm[w] - 1ull;
      }
      row[k] = v;
    }
  }
  if (i == 0) {
    leaf_count[b] = nleaf;
    status_out[b] = st;
  }
}

}  // namespace
}  // namespace tv
