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
// One wavefront per request, lane i = node i (T_max <= 64; larger trees, up to
// 256 nodes, take the 256-thread workgroup version in tree_meta_body.h).  The ancestor set of
// every node is built at once by pointer jumping in registers: after round r a
// lane's mask holds its ancestors up to distance 2^r - 1 and its jump pointer
// points 2^r levels up, so six rounds cover any tree of <= 64 nodes.  The mask
// lives in a 64-bit register per lane; no T x T boolean matrix is formed.
#include "tree_meta_body.h"

namespace tv {
namespace {

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
  const int p = check_tree(i, T_max, st, T, p_l);
  meta_body(b, i, T_max, dcap, W, T, st, p, P, tree_mask, tree_position_ids, positions, retrieve_indices,
            leaf_count, first_child, next_sibling, status_out);
}

// Trees of more than 64 nodes: one 256-thread workgroup per request.
__global__ __launch_bounds__(kWideNodes) void k_tree_mask_positions_wide(
    int T_max, int dcap, int W, const int* __restrict__ parents, const int* __restrict__ tree_size,
    const int* __restrict__ prefix_len, uint32_t* __restrict__ tree_mask, int* __restrict__ tree_position_ids,
    int* __restrict__ positions, int* __restrict__ retrieve_indices, int* __restrict__ leaf_count,
    int* __restrict__ first_child, int* __restrict__ next_sibling, const int* status_in, int* status_out) {
  __shared__ WideShared sh;
  const int b = blockIdx.x, i = threadIdx.x;
  const long long ob = (long long)b * T_max;
  int st = status_in ? status_in[b] : TV_ST_OK;
  int T = tree_size[b];
  const int P = prefix_len[b];
  const int p_l = i < T_max ? parents[ob + i] : -1;
  const int p = check_tree_wide(i, T_max, st, T, p_l, sh);
  meta_body_wide(b, i, T_max, dcap, W, T, st, p, P, tree_mask, tree_position_ids, positions, retrieve_indices,
                 leaf_count, first_child, next_sibling, status_out, sh);
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
  if (T_max <= 64)
    hipLaunchKernelGGL(tv::k_tree_mask_positions, dim3(B), dim3(64), 0, reinterpret_cast<hipStream_t>(stream),
                       T_max, dcap, W, parents, tree_size, prefix_len, tree_mask, tree_position_ids, positions,
                       retrieve_indices, leaf_count, first_child, next_sibling, status_in, status_out);
  else
    hipLaunchKernelGGL(tv::k_tree_mask_positions_wide, dim3(B), dim3(tv::kWideNodes), 0,
                       reinterpret_cast<hipStream_t>(stream), T_max, dcap, W, parents, tree_size, prefix_len,
                       tree_mask, tree_position_ids, positions, retrieve_indices, leaf_count, first_child,
                       next_sibling, status_in, status_out);
  TV_CHECK_LAUNCH();
  return TV_OK;
}
