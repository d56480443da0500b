// tree_mask_positions: parent pointers -> packed ancestor mask, depths and
// positions, retrieve paths, child/sibling lists, per-request status.
//
// What is computed: the tree-build kernel of the TensorRT-LLM EAGLE-3 dissection
// (section "dynamic draft tree": parents in, packed mask [N][ceil(N/32)] and
// position offsets out, child/sibling lists for the verifier, outputs fully
// rewritten every step so no stale bits survive), the handbook's tree_mask /
// depths (tree_spec.py), and the EAGLE v2 walkthrough's retrieve_indices /
// tree_position_ids (section 3, third step).
//
// One wavefront per request, lane i = node i (T_max <= 64).  The ancestor set of
// every node is built at once by pointer jumping in registers: after round r a
// lane's mask holds its ancestors up to distance 2^r - 1 and its jump pointer
// points 2^r levels up, so six rounds cover any tree of <= 64 nodes.  The mask
// lives in a 64-bit register per lane; no T x T boolean matrix is formed.
#include "tv_common.h"

namespace tv {
namespace {

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
#pragma unroll
  for (int r = 0; r < 6; ++r) {
    const unsigned long long ma = shfl_u64(m, a < 0 ? i : a);
    const int aa = __shfl(a, a < 0 ? i : a, 64);
    if (a >= 0) {
      m |= ma;
      a = aa;
    }
  }
  return {m, (int)__popcll(m) - 1};
}

__global__ __launch_bounds__(64) void k_tree_mask_positions(int T_max, int dcap, int W,
                                                            const int* __restrict__ parents,
                                                            const int* __restrict__ tree_size,
                                                            const int* __restrict__ prefix_len,
                                                            uint32_t* __restrict__ tree_mask,
                                                            int* __restrict__ tree_position_ids,
                                                            int* __restrict__ positions,
                                                            int* __restrict__ retrieve_indices,
                                                            int* __restrict__ leaf_count,
                                                            int* __restrict__ first_child,
                                                            int* __restrict__ next_sibling,
                                                            const int* status_in, int* status_out) {
  const int b = blockIdx.x, i = threadIdx.x;
  const long long ob = (long long)b * T_max;
  // all loads issued together (one memory round trip)
  int st = status_in ? status_in[b] : TV_ST_OK;
  int T = tree_size[b];
  const int P = prefix_len[b];
  const int p_l = i < T_max ? parents[ob + i] : -1;
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
  __syncthreads();
  if (in && i > 0) atomicOr(&s_cm[p], 1ull << i);
  __syncthreads();
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
  __syncthreads();
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

extern "C" int tree_mask_positions(int B, int T_max, int dcap, const int* parents, const int* tree_size,
                                   const int* prefix_len, uint32_t* tree_mask, int* tree_position_ids,
                                   int* positions, int* retrieve_indices, int* leaf_count, int* first_child,
                                   int* next_sibling, const int* status_in, int* status_out, void* stream) {
  if (B <= 0 || T_max <= 0 || dcap < 0 || dcap >= T_max) return TV_EINVAL;
  if (T_max > tv::kTMaxLimit) return TV_EUNSUPPORTED;
  if (!parents || !tree_size || !prefix_len || !tree_mask || !tree_position_ids || !positions ||
      !retrieve_indices || !leaf_count || !status_out)
    return TV_EINVAL;
  if (B > 2147483647 / 64) return TV_EINVAL;
  const int W = (T_max + 31) / 32;
  hipLaunchKernelGGL(tv::k_tree_mask_positions, dim3(B), dim3(64), 0, reinterpret_cast<hipStream_t>(stream), T_max,
                     dcap, W, parents, tree_size, prefix_len, tree_mask, tree_position_ids, positions,
                     retrieve_indices, leaf_count, first_child, next_sibling, status_in, status_out);
  TV_CHECK_LAUNCH();
  return TV_OK;
}
