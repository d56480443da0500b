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
