// tree_accept: greedy acceptance walk; kv_compact: accepted K/V rows to
// contiguous slots.
//
// tree_accept follows the greedy verification of the TensorRT-LLM EAGLE-3
// dissection (walk from the root; at each node accept the child whose draft
// token equals the target's argmax there, else stop; the path is at most
// depth + 1 long) and the handbook's tree_speculative_generate (the matching
// child is the first by index; the next root is the target's argmax at the end
// of the path).  One wavefront per request, lane c = node c: each step is one
// ballot over "parent == current node and token == prediction" and the lowest
// set lane is the child, so a step costs O(1) instead of a scan of the tree.
//
// kv_compact follows the KV note after the handbook's tree_spec.py and the
// dissection's "after acceptance: KV from tree layout back to linear": the
// accepted nodes' K/V are moved (not recomputed) to rows P+1..P+L.  One
// workgroup per (request, kv head, layer) stages every source row of K and V in
// LDS, synchronises, then writes, so a source that is also an earlier
// destination is read before it is overwritten.
#include "tv_common.h"

namespace tv {
namespace {

struct Walk {
  int len;    // accepted draft nodes past the root
  int mine;   // path entry c for lane c <= len (entry 0 is the root), else -1
  int bonus;  // the target's prediction at the last accepted node
};

// The walk of request b on one wavefront (lane c = node c, T_max <= 64).
__device__ __forceinline__ Walk accept_walk(int b, int c, int T_max, int dcap, const int* __restrict__ draft_tokens,
                                            const int* __restrict__ parents, const int* __restrict__ tree_size,
                                            const int* __restrict__ target_predict, const int* __restrict__ status) {
  const long long ob = (long long)b * T_max;
  // every per-node value is fetched at once (lane c holds node c); the walk itself
  // then only moves data between lanes
  int T = tree_size[b];
  const int st = status[b];
  const int tok_l = c < T_max ? draft_tokens[ob + c] : -1;
  const int par_l = c < T_max ? parents[ob + c] : -2;
  const int pred_l = c < T_max ? target_predict[ob + c] : -1;
  if (st != TV_ST_OK || T < 1 || T > T_max) T = 1;
  const int tok = c < T ? tok_l : -1;
  const int par = (c > 0 && c < T) ? par_l : -2;
  int node = 0, len = 0, mine = c == 0 ? 0 : -1;
  // node is wave-uniform, so the prediction at it is read with readlane
  for (int step = 0; step < dcap; ++step) {
    const int pred = __builtin_amdgcn_readlane(pred_l, node);
    const unsigned long long hit = __ballot(par == node && tok == pred);
    if (!hit) break;
    node = __ffsll((long long)hit) - 1;  // lowest-index matching child
    ++len;
    if (c == len) mine = node;
  }
  return {len, mine, __builtin_amdgcn_readlane(pred_l, node)};
}

// The same walk for trees of up to 256 nodes, by a 256-thread workgroup (thread
// c = node c; every thread must call it).  Each step broadcasts the prediction
// at the current node through LDS and takes the lowest matching child with an
// LDS atomic minimum.  Path entries 0..len go to s_path (at least dcap + 1).
struct WalkWide {
  int len, bonus;
};

__device__ __forceinline__ WalkWide accept_walk_wide(int b, int c, int T_max, int dcap,
                                                     const int* __restrict__ draft_tokens,
                                                     const int* __restrict__ parents,
                                                     const int* __restrict__ tree_size,
                                                     const int* __restrict__ target_predict,
                                                     const int* __restrict__ status, int* s_path) {
  __shared__ int s_bc, s_next;
  const long long ob = (long long)b * T_max;
  int T = tree_size[b];
  const int st = status[b];
  const int tok_l = c < T_max ? draft_tokens[ob + c] : -1;
  const int par_l = c < T_max ? parents[ob + c] : -2;
  const int pred_l = c < T_max ? target_predict[ob + c] : -1;
  if (st != TV_ST_OK || T < 1 || T > T_max) T = 1;
  const int tok = c < T ? tok_l : -1;
  const int par = (c > 0 && c < T) ? par_l : -2;
  if (c == 0) s_path[0] = 0;
  int node = 0, len = 0;
  for (int step = 0; step < dcap; ++step) {
    if (c == node) s_bc = pred_l;
    if (c == 0) s_next = 0x7FFFFFFF;
    __syncthreads();
    const int pred = s_bc;
    if (par == node && tok == pred) atomicMin(&s_next, c);
    __syncthreads();
    const int nx = s_next;
    __syncthreads();  // every read before the next step's writes
    if (nx == 0x7FFFFFFF) break;
    node = nx;
    ++len;
    if (c == 0) s_path[len] = node;
  }
  if (c == node) s_bc = pred_l;
  __syncthreads();
  const int bonus = s_bc;
  __syncthreads();
  return {len, bonus};
}

__global__ __launch_bounds__(256) void k_tree_accept_wide(int T_max, int dcap, const int* __restrict__ draft_tokens,
                                                          const int* __restrict__ parents,
                                                          const int* __restrict__ tree_size,
                                                          const int* __restrict__ target_predict,
                                                          const int* __restrict__ status,
                                                          int* __restrict__ accept_len, int* __restrict__ accept_path,
                                                          int* __restrict__ bonus_token) {
  __shared__ int s_path[256];
  const int b = blockIdx.x, c = threadIdx.x;
  const WalkWide w = accept_walk_wide(b, c, T_max, dcap, draft_tokens, parents, tree_size, target_predict, status,
                                      s_path);
  if (c <= dcap) accept_path[(long long)b * (dcap + 1) + c] = c <= w.len ? s_path[c] : -1;
  if (c == 0) {
    accept_len[b] = w.len;
    bonus_token[b] = w.bonus;
  }
}

__global__ __launch_bounds__(64) void k_tree_accept(int T_max, int dcap, const int* __restrict__ draft_tokens,
                                                    const int* __restrict__ parents,
                                                    const int* __restrict__ tree_size,
                                                    const int* __restrict__ target_predict,
                                                    const int* __restrict__ status, int* __restrict__ accept_len,
                                                    int* __restrict__ accept_path, int* __restrict__ bonus_token) {
  const int b = blockIdx.x, c = threadIdx.x;
  const Walk w = accept_walk(b, c, T_max, dcap, draft_tokens, parents, tree_size, target_predict, status);
  if (c <= dcap) accept_path[(long long)b * (dcap + 1) + c] = w.mine;
  if (c == 0) {
    accept_len[b] = w.len;
    bonus_token[b] = w.bonus;
  }
}

// --------------------------------------------------------------------------
// Tree rejection sampling with the target distribution only (the TensorRT-LLM
// dissection's target-only rejection sampling; the handbook's exercise on trees
// when sampling).  The tree's candidates are the drafter's deterministic top-K
// picks, so a candidate's draft distribution is the point mass on its token: at
// node n with target row p (mass Z), children are tried in ascending id and
// child c with token x is accepted iff u_c (Z - R) < p(x), R the mass of the
// tokens already rejected at n; if none is accepted (or the depth cap is
// reached) the correction token is drawn from p with the rejected tokens'
// mass removed: the smallest v whose cumulative residual mass exceeds u_0 times
// the residual total.  Sums are float64.
//
// One 1024-thread workgroup per request (a row is 128 KB at V = 32000: eight
// 16-byte loads in flight per thread cover it in one round trip).  Per visited
// node one coalesced pass over the row gives Z while the
// first wavefront fetches p(x) of every child at once (lane c = node c), so the
// sequential decisions only move data between lanes.  With Z of every row
// already known (k_row_mass, one workgroup per row, for calls whose rows are few
// enough that reading them all costs less than the walk's chain of passes), the
// first wavefront fetches every child's p(x) from its parent's row up front and
// the walk reads no row at all.  The correction cuts the
// row into 1024 contiguous chunks: each wavefront sums its chunks with coalesced
// loads, a block scan of the chunk sums finds the chunk holding the target, and
// the first wavefront scans that chunk.
// --------------------------------------------------------------------------
constexpr int kSampleThreads = 1024;
constexpr int kPiece = 8 * kSampleThreads;  // row entries read per pass step (8 per thread)
constexpr int kMaxPieces = 32;              // V <= 262144

// A float64 moved between lanes by one DPP control (both halves alike); lanes
// with no source (bound_ctrl) or outside row_mask read 0.
template <int CTRL, int ROWS, bool BOUND>
__device__ __forceinline__ double dpp_f64(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(b & 0xFFFFFFFF), CTRL, ROWS, 0xF, BOUND);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, ROWS, 0xF, BOUND);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// inclusive prefix sum over the 16 lanes of each row (row_shr 1, 2, 4, 8)
__device__ __forceinline__ double row_incl_f64(double v) {
  v += dpp_f64<0x111, 0xF, true>(v);
  v += dpp_f64<0x112, 0xF, true>(v);
  v += dpp_f64<0x114, 0xF, true>(v);
  v += dpp_f64<0x118, 0xF, true>(v);
  return v;
}

// inclusive prefix sum over the wavefront: within the rows, then row 0's total
// into row 1 and row 2's into row 3 (row_bcast:15), rows 0-1's into rows 2-3
// (row_bcast:31); no LDS round trip
__device__ __forceinline__ double wave_incl_f64(double v) {
  v = row_incl_f64(v);
  v += dpp_f64<0x142, 0xA, false>(v);
  v += dpp_f64<0x143, 0xC, false>(v);
  return v;
}

// the wavefront's sum (every lane gets it)
__device__ __forceinline__ double wave_sum_f64(double v) {
  const long long b = __double_as_longlong(wave_incl_f64(v));
  const int lo = __builtin_amdgcn_readlane((int)(b & 0xFFFFFFFF), 63);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), 63);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

__device__ __forceinline__ double readlane_f64(double v, int l) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)(b & 0xFFFFFFFF), l);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), l);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

constexpr int kSampleWaves = kSampleThreads / 64;

// A row is read in pieces of kPiece entries; in piece k thread t owns the 8
// contiguous entries [k kPiece + 8 t, + 8) (a wavefront reads 2 KB contiguous).
__device__ __forceinline__ void load8(const float* __restrict__ row, int V, int vec4, int k, float (&x)[8]) {
  const int v0 = k * kPiece + 8 * (int)threadIdx.x;
  if (vec4 && v0 + 8 <= V) {
    typedef float f4 __attribute__((ext_vector_type(4)));
    const f4 a = *reinterpret_cast<const f4*>(row + v0), c = *reinterpret_cast<const f4*>(row + v0 + 4);
    x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
    x[4] = c[0]; x[5] = c[1]; x[6] = c[2]; x[7] = c[3];
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = v0 + e < V ? row[v0 + e] : 0.0f;
  }
}

// the workgroup's float64 sum of one value per thread: wavefront butterflies,
// then the wavefronts in order (every thread gets it)
__device__ __forceinline__ double sample_block_sum(double v, double* s_red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum_f64(v);
  if (lane == 0) s_red[wave] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int w = 0; w < kSampleWaves; ++w) t += s_red[w];
  __syncthreads();
  return t;
}

// float64 sum of a whole row (four pieces' loads in flight at a time), in the
// one order both kernels use: each thread adds its entries piece by piece, then
// the workgroup sum above
__device__ __forceinline__ double row_sum_f64(const float* __restrict__ row, int V, int vec4, double* s_red) {
  const int n_pieces = (V + kPiece - 1) / kPiece;
  double acc = 0.0;
  for (int k0 = 0; k0 < n_pieces; k0 += 4) {
    float x[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (k0 + u < n_pieces) load8(row, V, vec4, k0 + u, x[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (k0 + u < n_pieces)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += (double)x[u][e];
  }
  return sample_block_sum(acc, s_red);
}

// Z of row (b, i) for every node i < T_b: one workgroup per row, grid (T_max, B)
__global__ __launch_bounds__(kSampleThreads) void k_row_mass(int T_max, int V, int vec4,
                                                             const int* __restrict__ tree_size,
                                                             const int* __restrict__ status,
                                                             const float* __restrict__ target_probs,
                                                             double* __restrict__ Z) {
  const int i = blockIdx.x, b = blockIdx.y;
  int T = tree_size[b];
  if (!(status[b] == TV_ST_OK && T >= 1 && T <= T_max)) T = 1;
  if (i >= T) return;
  __shared__ double s_red[kSampleWaves];
  const long long r = (long long)b * T_max + i;
  const double z = row_sum_f64(target_probs + r * V, V, vec4, s_red);
  if (threadIdx.x == 0) Z[r] = z;
}

__global__ __launch_bounds__(kSampleThreads) void k_tree_accept_sample(
    int T_max, int dcap, int V, int vec4, const int* __restrict__ draft_tokens, const int* __restrict__ parents,
    const int* __restrict__ tree_size, const float* __restrict__ target_probs, const float* __restrict__ uniforms,
    const int* __restrict__ status, const double* __restrict__ Zpre, int* __restrict__ accept_len,
    int* __restrict__ accept_path, int* __restrict__ bonus_token) {
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int NWV = kSampleWaves;
  __shared__ double s_red[NWV];
  __shared__ int s_rem[kTMaxLimit];  // tokens rejected at the current node
  __shared__ int s_cx[64], s_cid[64];  // up to 64 children of the current node: token, node id
  __shared__ float s_cp[64], s_cu[64];  // and p(x), draw
  __shared__ int s_path[kTMaxLimit];
  __shared__ int s_next, s_nrem, s_pick;
  const long long ob = (long long)b * T_max;
  int T = tree_size[b];
  const bool ok = status[b] == TV_ST_OK && T >= 1 && T <= T_max;
  if (!ok) T = 1;
  // per-node data in the first wavefront's lanes: node c = lane + 64 q, q < 4
  constexpr int NQ = kTMaxLimit / 64;
  int tok_q[NQ], par_q[NQ];
  float u_q[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int c = lane + 64 * q;
    tok_q[q] = c < T ? draft_tokens[ob + c] : -1;
    par_q[q] = (c > 0 && c < T) ? parents[ob + c] : -2;
    u_q[q] = c < T_max ? uniforms[ob + c] : 0.0f;
  }
  auto block_sum = [&](double v) -> double { return sample_block_sum(v, s_red); };
  const int n_pieces = (V + kPiece - 1) / kPiece;
  auto load8 = [&](const float* row, int k, float (&x)[8]) __attribute__((always_inline)) {
    tv::load8(row, V, vec4, k, x);
  };
  // With every row's Z given: p(x) of every node, from its parent's row, fetched
  // once (first wavefront; a token outside the vocabulary has no mass)
  // and Z of every node (lane c = node c)
  float pall_q[NQ];
  double z_q[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    pall_q[q] = 0.0f;
    z_q[q] = 0.0;
    if (Zpre && wave == 0 && par_q[q] >= 0 && par_q[q] < T && tok_q[q] >= 0 && tok_q[q] < V)
      pall_q[q] = target_probs[(ob + par_q[q]) * (long long)V + tok_q[q]];
    if (Zpre && wave == 0 && lane + 64 * q < T) z_q[q] = Zpre[ob + lane + 64 * q];
  }
  // Z of node n (wave-uniform n) from the lane that holds it
  auto z_of = [&](int n) -> double {
    double z = z_q[0];
#pragma unroll
    for (int q = 1; q < NQ; ++q) z = (n >> 6) == q ? z_q[q] : z;
    const long long bits = __double_as_longlong(z);
    const int lo = __builtin_amdgcn_readlane((int)(bits & 0xFFFFFFFF), n & 63);
    const int hi = __builtin_amdgcn_readlane((int)(bits >> 32), n & 63);
    return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
  };

  int node = 0, len = 0, nrem = 0;
  if (tid == 0) s_path[0] = 0;
  while (ok && len < dcap) {
    const float* row = target_probs + (ob + node) * (long long)V;
    // p(x) of every child of this node, fetched together (first wavefront)
    float pc_q[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      pc_q[q] = 0.0f;
      if (wave == 0 && par_q[q] == node) {
        if (Zpre) pc_q[q] = pall_q[q];
        else if (tok_q[q] >= 0 && tok_q[q] < V) pc_q[q] = row[tok_q[q]];
      }
    }
    const double Z = Zpre ? z_of(node) : row_sum_f64(row, V, vec4, s_red);
    if (wave == 0) {
      // the node's children (ascending id) and their number
      unsigned long long km[NQ];
      int m = 0;
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        km[q] = __ballot(par_q[q] == node);
        m += __popcll(km[q]);
      }
      if (m <= 64) {
        // Up to 64 children, child j (in ascending id) in lane j: whether an
        // earlier child has its token (then it brings no mass), R_j = the mass of
        // the earlier rejected tokens added in child order, and every child's
        // test at once; the first child that passes is taken.  The same additions
        // and comparisons as one child at a time.
        int before = 0;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          if ((km[q] >> lane) & 1ull) {
            const int j = before + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(km[q] >> 32),
                                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)km[q], 0u));
            s_cx[j] = tok_q[q];
            s_cp[j] = pc_q[q];
            s_cu[j] = u_q[q];
            s_cid[j] = 64 * q + lane;
          }
          before += __popcll(km[q]);
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        const bool live = lane < m;
        const int xj = live ? s_cx[lane] : 0;
        const float pj = live ? s_cp[lane] : 0.0f, uj = live ? s_cu[lane] : 0.0f;
        const int idj = live ? s_cid[lane] : -1;
        bool dup = false;
        for (int i = 0; i < m; ++i) dup |= i < lane && __builtin_amdgcn_readlane(xj, i) == xj;
        const double pe = (live && !dup) ? (double)pj : 0.0;
        double R = 0.0, Rj = 0.0;
        for (int i = 0; i < m; ++i) {
          Rj = lane == i ? R : Rj;
          const long long pb = __double_as_longlong(pe);
          const int lo = __builtin_amdgcn_readlane((int)(pb & 0xFFFFFFFF), i);
          const int hi = __builtin_amdgcn_readlane((int)(pb >> 32), i);
          R += __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
        }
        const unsigned long long am = __ballot(live && (double)uj * (Z - Rj) < pe);
        int next = -1, nr = 0;
        if (am) {
          next = __builtin_amdgcn_readlane(idj, __ffsll((long long)am) - 1);
        } else {  // every child rejected: their distinct tokens
          const unsigned long long kk = __ballot(live && !dup);
          if (live && !dup)
            s_rem[(int)__builtin_amdgcn_mbcnt_hi((uint32_t)(kk >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)kk, 0u))] = xj;
          nr = __popcll(kk);
        }
        if (lane == 0) {
          s_next = next;
          s_nrem = nr;
        }
      } else {
        // children in ascending id (the current node and every decision are
        // wave-uniform); rejected token r sits in lane r % 64, slot r / 64
        double R = 0.0;
        int next = -1, nr = 0, rem_q[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) rem_q[q] = -1;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          unsigned long long kids = next < 0 ? __ballot(par_q[q] == node) : 0ull;
          while (kids) {
            const int c = __ffsll((long long)kids) - 1;
            kids &= kids - 1;
            const int x = __builtin_amdgcn_readlane(tok_q[q], c);
            bool any = false;
#pragma unroll
            for (int r = 0; r < NQ; ++r) any |= rem_q[r] == x;
            const bool seen = __ballot(any) != 0ull;
            const double px =
                seen ? 0.0 : (double)__int_as_float(__builtin_amdgcn_readlane(__float_as_int(pc_q[q]), c));
            const double uc = (double)__int_as_float(__builtin_amdgcn_readlane(__float_as_int(u_q[q]), c));
            if (uc * (Z - R) < px) {
              next = 64 * q + c;
              break;
            }
            if (!seen) {
              R += px;
#pragma unroll
              for (int r = 0; r < NQ; ++r)
                if (lane == (nr & 63) && (nr >> 6) == r) rem_q[r] = x;
              ++nr;
            }
          }
        }
#pragma unroll
        for (int r = 0; r < NQ; ++r)
          if (lane + 64 * r < nr) s_rem[lane + 64 * r] = rem_q[r];
        if (lane == 0) {
          s_next = next;
          s_nrem = nr;
        }
      }
    }
    __syncthreads();
    const int next = s_next;
    nrem = s_nrem;
    if (next < 0) break;
    ++len;
    node = next;
    nrem = 0;
    if (tid == 0) s_path[len] = node;
  }
  __syncthreads();

  // ---- the correction token at `node`, from the row with the nrem rejected tokens removed
  const float* row = target_probs + (ob + node) * (long long)V;
  auto removed = [&](int v) {
    bool r = false;
    for (int q = 0; q < nrem; ++q) r |= s_rem[q] == v;
    return r;
  };
  // which of this thread's entries are removed: bit e of byte k stands for entry
  // k kPiece + 8 tid + e (each thread writes and reads only its own bytes)
  __shared__ uint8_t s_rbits[kMaxPieces * kSampleThreads];
  for (int k = 0; k < n_pieces; ++k) s_rbits[k * kSampleThreads + tid] = 0;
  for (int q = 0; q < nrem; ++q) {
    const int v = s_rem[q];
    if (v >= 0 && v < V && ((v % kPiece) >> 3) == tid) s_rbits[(v / kPiece) * kSampleThreads + tid] |= 1u << (v & 7);
  }
  // residual mass of this thread's run of a piece
  auto run_mass = [&](int k, float (&x)[8]) -> double {
    const int v0 = k * kPiece + 8 * tid;
    const uint32_t rb = s_rbits[k * kSampleThreads + tid];
    double run = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (v0 + e < V && !((rb >> e) & 1u)) run += (double)x[e];
    return run;
  };
  // pass 1: the residual total, hence the target (pieces 0..3 stay in registers
  // for pass 2)
  float xa[4][8];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (u < n_pieces) load8(row, u, xa[u]);
  double acc = 0.0;
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (u < n_pieces) acc += run_mass(u, xa[u]);
  for (int k0 = 4; k0 < n_pieces; k0 += 4) {
    float x[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (k0 + u < n_pieces) load8(row, k0 + u, x[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (k0 + u < n_pieces) acc += run_mass(k0 + u, x[u]);
  }
  const double total = block_sum(acc);
  if (tid == 0) s_pick = -1;
  __syncthreads();
  const double target = (double)__int_as_float(__builtin_amdgcn_readlane(__float_as_int(u_q[0]), 0)) * total;
  __shared__ double s_last[4][NWV];
  if (total > 0.0) {
    // pass 2, four pieces at a time: a block inclusive scan of the runs' masses
    // (within a wavefront by DPP); run (k, t) spans [lo, hi) of the cumulative
    // mass, each boundary one computed number that both neighbours take, so the
    // runs tile the total.  Wavefront w starts at carry + t_0 + ... + t_(w-1)
    // added in this order (t: the wavefronts' totals), which every wavefront
    // forms alike, and its last lane ends where wavefront w + 1 starts.  A run of
    // no width takes no target; should rounding still leave two runs holding it,
    // the larger token is taken.
    double carry = 0.0;
    auto scan_group = [&](int k0, float (&x)[4][8]) __attribute__((always_inline)) {
      double incl[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) incl[u] = k0 + u < n_pieces ? wave_incl_f64(run_mass(k0 + u, x[u])) : 0.0;
      if (lane == 63) {
#pragma unroll
        for (int u = 0; u < 4; ++u) s_last[u][wave] = incl[u];
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (k0 + u >= n_pieces) break;
        const double tv = lane < NWV ? s_last[u][lane] : 0.0;
        double o = carry, off = carry, nxt = carry;
        for (int w = 0; w < NWV; ++w) {
          const double tw = readlane_f64(tv, w);
          if (w == wave) {
            off = o;
            nxt = o + tw;
          }
          o = o + tw;
        }
        const double hi = lane == 63 ? nxt : off + incl[u];
        const double up = __shfl_up(hi, 1, 64);
        const double lo = lane > 0 ? up : off;
        if (lo < hi && lo <= target && target < hi) {
          // this run holds the target: walk it; if rounding keeps the sum below
          // the target, its last entry with mass
          const int v0 = (k0 + u) * kPiece + 8 * tid;
          const uint32_t rb = s_rbits[(k0 + u) * kSampleThreads + tid];
          double cum = lo;
          int pick = -1, last = -1;
          for (int e = 0; e < 8 && v0 + e < V; ++e) {
            if ((rb >> e) & 1u) continue;
            if (x[u][e] > 0.0f) last = v0 + e;
            cum += (double)x[u][e];
            if (cum > target) {
              pick = v0 + e;
              break;
            }
          }
          atomicMax(&s_pick, pick >= 0 ? pick : last);
        }
        carry = o;
      }
      __syncthreads();  // (s_last is rewritten by the next group)
    };
    scan_group(0, xa);
    for (int k0 = 4; k0 < n_pieces; k0 += 4) {
      float x[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (k0 + u < n_pieces) load8(row, k0 + u, x[u]);
      scan_group(k0, x);
    }
    __syncthreads();
    if (s_pick < 0) {  // rounding left the target past the total: the last token with residual mass
      int last = -1;
      for (int v = tid; v < V; v += kSampleThreads)
        if (row[v] > 0.0f && !removed(v)) last = v;
      if (last >= 0) atomicMax(&s_pick, last);
      __syncthreads();
    }
  } else {
    // no residual mass: the row's best token (probability desc, token asc)
    unsigned long long best = 0ull;
    for (int v = tid; v < V; v += kSampleThreads) best = umax64(best, rank_key(row[v], (uint32_t)v));
    best = wave_max_u64(best);
    __shared__ unsigned long long s_best[NWV];
    if (lane == 0) s_best[wave] = best;
    __syncthreads();
    if (tid == 0) {
      unsigned long long m = 0ull;
      for (int w = 0; w < NWV; ++w) m = umax64(m, s_best[w]);
      s_pick = (int)key_index(m);
    }
    __syncthreads();
  }
  if (tid <= dcap) accept_path[(long long)b * (dcap + 1) + tid] = tid <= len ? s_path[tid] : -1;
  if (tid == 0) {
    accept_len[b] = len;
    bonus_token[b] = s_pick;
  }
}

constexpr int kCompactThreads = 256;

// Moves request b's accepted rows of one (kv head, layer).  The caller has
// written s_path[0..dcap] (the first barrier here publishes it) and passes the
// length L.  S_cap is the rows a request can hold (the linear slab, or the
// block-table capacity); with a paged cache every source and destination row is
// looked up in the request's block table once, and an entry outside the pool
// leaves the request untouched like a path that does not fit.
__device__ __forceinline__ void compact_rows(int b, int g, int layer, int Hkv, int chunks16, uint4* __restrict__ Kc,
                                             uint4* __restrict__ Vc, long long S_cap, long long layer_stride16,
                                             int P, int L, const int* s_path, int dcap,
                                             int* __restrict__ new_prefix_len, const Paging& pg) {
  const int tid = threadIdx.x;
  __shared__ int s_bad;
  __shared__ long long s_src[64], s_dst[64];  // 16-byte chunk offsets of rows P + path[k] and P + k
  if (tid == 0) s_bad = 0;
  __syncthreads();
  // offset of logical row s (0 <= s < S_cap) of (b, g) in this layer; false for a
  // block-table entry outside the pool
  auto row16 = [&](long long s, long long& off) -> bool {
    long long r;
    if (pg.table) {
      const long long blk = pg.table[(long long)b * pg.max_blocks + (s >> pg.lbs)];
      if (blk < 0 || blk >= pg.n_blocks) return false;
      r = ((blk * Hkv + g) << pg.lbs) + (s & ((1 << pg.lbs) - 1));
    } else {
      r = ((long long)b * Hkv + g) * S_cap + s;
    }
    off = layer * layer_stride16 + r * chunks16;
    return true;
  };
  // every source and destination row must lie inside the cache
  if (tid >= 1 && tid <= L && tid <= dcap) {
    const int n = s_path[tid];
    long long so = 0, dof = 0;
    const bool bad = P < 0 || n < tid || (long long)P + n >= S_cap || !row16((long long)P + n, so) ||
                     !row16((long long)P + tid, dof);
    if (bad) s_bad = 1;
    s_src[tid] = so;
    s_dst[tid] = dof;
  }
  __syncthreads();
  const bool ok = L >= 1 && L <= dcap && P >= 0 && s_bad == 0;
  // a request whose path does not fit is left untouched (its prefix grows by the root only)
  if (g == 0 && layer == 0 && tid == 0 && new_prefix_len) new_prefix_len[b] = P + (ok ? L : 0) + 1;
  if (!ok) return;
  // every K and V source row is read into LDS before any destination is written
  // (a source may be an earlier destination); stage = [K rows | V rows]
  extern __shared__ uint4 s_stage[];
  const int items = L * chunks16;
#pragma unroll 4
  for (int q = tid; q < 2 * items; q += kCompactThreads) {
    const int t = q >= items, r = q - t * items;
    const int k = 1 + r / chunks16, c = r % chunks16;
    s_stage[q] = (t ? Vc : Kc)[s_src[k] + c];
  }
  __syncthreads();
#pragma unroll 4
  for (int q = tid; q < 2 * items; q += kCompactThreads) {
    const int t = q >= items, r = q - t * items;
    const int k = 1 + r / chunks16, c = r % chunks16;
    (t ? Vc : Kc)[s_dst[k] + c] = s_stage[q];
  }
}

__global__ __launch_bounds__(kCompactThreads) void k_kv_compact(int Hkv, int chunks16, uint4* __restrict__ Kc,
                                                                uint4* __restrict__ Vc, long long S_cap,
                                                                long long layer_stride16,
                                                                const int* __restrict__ prefix_len,
                                                                const int* __restrict__ accept_path,
                                                                const int* __restrict__ accept_len, int dcap,
                                                                int* __restrict__ new_prefix_len, Paging pg) {
  const int g = blockIdx.x % Hkv;
  const int b = blockIdx.x / Hkv;
  const int tid = threadIdx.x;
  // the request's prefix, length and path, read once (path entries by the first
  // dcap + 1 threads, into LDS)
  __shared__ int s_path[64];
  const int P = prefix_len[b];
  const int L = accept_len[b];
  if (tid <= dcap) s_path[tid] = accept_path[(long long)b * (dcap + 1) + tid];
  compact_rows(b, g, blockIdx.y, Hkv, chunks16, Kc, Vc, S_cap, layer_stride16, P, L, s_path, dcap, new_prefix_len,
               pg);
}

// tree_accept and kv_compact in one launch: every (request, kv head, layer)
// workgroup runs the request's walk on its first wavefront (the walk reads a few
// hundred bytes and is the same in every workgroup), the (request, 0, 0)
// workgroup also writes the acceptance outputs, then the rows are moved.
__global__ __launch_bounds__(kCompactThreads) void k_accept_compact(
    int T_max, int dcap, const int* __restrict__ draft_tokens, const int* __restrict__ parents,
    const int* __restrict__ tree_size, const int* __restrict__ target_predict, const int* __restrict__ status,
    int* __restrict__ accept_len, int* __restrict__ accept_path, int* __restrict__ bonus_token, int Hkv,
    int chunks16, uint4* __restrict__ Kc, uint4* __restrict__ Vc, long long S_cap, long long layer_stride16,
    const int* __restrict__ prefix_len, int* __restrict__ new_prefix_len, Paging pg) {
  const int g = blockIdx.x % Hkv;
  const int b = blockIdx.x / Hkv;
  const int tid = threadIdx.x;
  __shared__ int s_path[64];
  __shared__ int s_len;
  const int P = prefix_len[b];
  if (T_max <= 64) {
    if (tid < 64) {
      const Walk w = accept_walk(b, tid, T_max, dcap, draft_tokens, parents, tree_size, target_predict, status);
      if (tid <= dcap) s_path[tid] = w.mine;
      if (tid == 0) s_len = w.len;
      if (g == 0 && blockIdx.y == 0) {
        if (tid <= dcap) accept_path[(long long)b * (dcap + 1) + tid] = w.mine;
        if (tid == 0) {
          accept_len[b] = w.len;
          bonus_token[b] = w.bonus;
        }
      }
    }
  } else {  // up to 256 nodes (dcap < 64 here: the compaction stages at most 63 rows)
    const WalkWide w = accept_walk_wide(b, tid, T_max, dcap, draft_tokens, parents, tree_size, target_predict,
                                        status, s_path);
    if (tid == 0) s_len = w.len;
    if (g == 0 && blockIdx.y == 0) {
      if (tid <= dcap) accept_path[(long long)b * (dcap + 1) + tid] = tid <= w.len ? s_path[tid] : -1;
      if (tid == 0) {
        accept_len[b] = w.len;
        bonus_token[b] = w.bonus;
      }
    }
  }
  __syncthreads();
  compact_rows(b, g, blockIdx.y, Hkv, chunks16, Kc, Vc, S_cap, layer_stride16, P, s_len, s_path, dcap,
               new_prefix_len, pg);
}

}  // namespace
}  // namespace tv

extern "C" int tree_accept(int B, int T_max, int dcap, const int* draft_tokens, const int* parents,
                           const int* tree_size, const int* target_predict, const int* status, int* accept_len,
                           int* accept_path, int* bonus_token, void* stream) {
  if (B <= 0 || T_max <= 0 || dcap < 0 || dcap >= T_max) return TV_EINVAL;
  if (T_max > tv::kTMaxLimit) return TV_EUNSUPPORTED;
  if (!draft_tokens || !parents || !tree_size || !target_predict || !status || !accept_len || !accept_path ||
      !bonus_token)
    return TV_EINVAL;
  if (T_max <= 64)
    hipLaunchKernelGGL(tv::k_tree_accept, dim3(B), dim3(64), 0, reinterpret_cast<hipStream_t>(stream), T_max, dcap,
                       draft_tokens, parents, tree_size, target_predict, status, accept_len, accept_path,
                       bonus_token);
  else
    hipLaunchKernelGGL(tv::k_tree_accept_wide, dim3(B), dim3(256), 0, reinterpret_cast<hipStream_t>(stream), T_max,
                       dcap, draft_tokens, parents, tree_size, target_predict, status, accept_len, accept_path,
                       bonus_token);
  TV_CHECK_LAUNCH();
  return TV_OK;
}

namespace tv {
namespace {

// checks shared by the compaction entry points; returns TV_OK and the 16-byte
// chunks per row, or an error code.  S_cap: rows a request can hold; per_layer:
// elements of one layer's cache (pool) per tensor.
int compact_checks(int B, int n_layers, int Hkv, int d, int elem_bytes, const void* Kc, const void* Vc,
                   long long S_cap, long long per_layer, long long layer_stride_elems, int dcap, int* chunks16,
                   size_t* stage) {
  if (B <= 0 || n_layers <= 0 || Hkv <= 0 || d <= 0 || S_cap <= 0 || dcap < 0 || dcap >= 64) return TV_EINVAL;
  if (elem_bytes != 2 && elem_bytes != 4) return TV_EINVAL;
  if (!Kc || !Vc) return TV_EINVAL;
  const long long row_bytes = (long long)d * elem_bytes;
  if (row_bytes % 16 != 0 || row_bytes > 1024) return TV_EUNSUPPORTED;
  if (n_layers > 1 && layer_stride_elems < per_layer) return TV_EINVAL;
  if ((layer_stride_elems * elem_bytes) % 16 != 0) return TV_EINVAL;
  if ((reinterpret_cast<uintptr_t>(Kc) & 15) || (reinterpret_cast<uintptr_t>(Vc) & 15)) return TV_EINVAL;
  if ((long long)B * Hkv > 2147483647LL || n_layers > 65535) return TV_EINVAL;
  *chunks16 = (int)(row_bytes / 16);
  *stage = 2 * (size_t)dcap * (size_t)(row_bytes / 16) * 16;  // K and V rows of one path
  if (*stage > 65536) return TV_EUNSUPPORTED;
  return TV_OK;
}

// the paged-cache arguments: Paging and the capacity per request, or an error
int paged_args(int B, int Hkv, int d, long long num_blocks, int tokens_per_block, const int* block_table,
               int max_blocks_per_seq, Paging* pg, long long* cap, long long* per_layer) {
  const int lbs = log2_block(tokens_per_block);
  if (lbs < 0 || !block_table || max_blocks_per_seq <= 0 || num_blocks <= 0 || Hkv <= 0 || d <= 0) return TV_EINVAL;
  if ((long long)B * max_blocks_per_seq > (1LL << 31)) return TV_EINVAL;
  if (num_blocks > (1LL << 40) / ((long long)Hkv * tokens_per_block)) return TV_EINVAL;
  *pg = Paging{block_table, max_blocks_per_seq, lbs, num_blocks};
  *cap = (long long)max_blocks_per_seq << lbs;
  *per_layer = num_blocks * Hkv * tokens_per_block * d;
  return TV_OK;
}

// [a, a + na) and [b, b + nb) share a byte (host: pointers are only compared)
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return a && b && x < y + nb && y < x + na;
}

int kv_compact_impl(int B, int n_layers, int Hkv, int d, int elem_bytes, void* Kc, void* Vc, long long S_cap,
                    long long per_layer, long long layer_stride_elems, const int* prefix_len, const int* accept_path,
                    const int* accept_len, int dcap, int* new_prefix_len, void* stream, const Paging& pg) {
  int chunks16 = 0;
  size_t stage = 0;
  const int rc = compact_checks(B, n_layers, Hkv, d, elem_bytes, Kc, Vc, S_cap, per_layer, layer_stride_elems, dcap,
                                &chunks16, &stage);
  if (rc != TV_OK) return rc;
  if (!prefix_len || !accept_path || !accept_len) return TV_EINVAL;
  // every workgroup of a request reads these while one of them writes new_prefix_len
  const size_t nb = (size_t)B * sizeof(int);
  if (overlaps(new_prefix_len, nb, prefix_len, nb) || overlaps(new_prefix_len, nb, accept_len, nb) ||
      overlaps(new_prefix_len, nb, accept_path, nb * (dcap + 1)))
    return TV_EINVAL;
  hipLaunchKernelGGL(k_kv_compact, dim3(B * Hkv, n_layers), dim3(kCompactThreads), stage,
                     reinterpret_cast<hipStream_t>(stream), Hkv, chunks16, reinterpret_cast<uint4*>(Kc),
                     reinterpret_cast<uint4*>(Vc), S_cap, layer_stride_elems * elem_bytes / 16, prefix_len,
                     accept_path, accept_len, dcap, new_prefix_len, pg);
  TV_CHECK_LAUNCH();
  return TV_OK;
}

int accept_compact_impl(int B, int T_max, int dcap, const int* draft_tokens, const int* parents,
                        const int* tree_size, const int* target_predict, const int* status, int* accept_len,
                        int* accept_path, int* bonus_token, int n_layers, int Hkv, int d, int elem_bytes, void* Kc,
                        void* Vc, long long S_cap, long long per_layer, long long layer_stride_elems,
                        const int* prefix_len, int* new_prefix_len, void* stream, const Paging& pg) {
  // the checks of tree_accept, then those of kv_compact
  if (B <= 0 || T_max <= 0 || dcap < 0 || dcap >= T_max) return TV_EINVAL;
  if (T_max > kTMaxLimit) return TV_EUNSUPPORTED;
  if (!draft_tokens || !parents || !tree_size || !target_predict || !status || !accept_len || !accept_path ||
      !bonus_token)
    return TV_EINVAL;
  int chunks16 = 0;
  size_t stage = 0;
  const int rc = compact_checks(B, n_layers, Hkv, d, elem_bytes, Kc, Vc, S_cap, per_layer, layer_stride_elems, dcap,
                                &chunks16, &stage);
  if (rc != TV_OK) return rc;
  if (!prefix_len) return TV_EINVAL;
  // every workgroup of a request reads prefix_len while one of them writes new_prefix_len
  const size_t nb = (size_t)B * sizeof(int);
  if (overlaps(new_prefix_len, nb, prefix_len, nb)) return TV_EINVAL;
  hipLaunchKernelGGL(k_accept_compact, dim3(B * Hkv, n_layers), dim3(kCompactThreads), stage,
                     reinterpret_cast<hipStream_t>(stream), T_max, dcap, draft_tokens, parents, tree_size,
                     target_predict, status, accept_len, accept_path, bonus_token, Hkv, chunks16,
                     reinterpret_cast<uint4*>(Kc), reinterpret_cast<uint4*>(Vc), S_cap,
                     layer_stride_elems * elem_bytes / 16, prefix_len, new_prefix_len, pg);
  TV_CHECK_LAUNCH();
  return TV_OK;
}

}  // namespace
}  // namespace tv

extern "C" size_t tree_accept_sample_workspace_bytes(int B, int T_max) {
  if (B <= 0 || T_max <= 0) return 0;
  return (size_t)B * T_max * sizeof(double);
}

extern "C" int tree_accept_sample(int B, int T_max, int dcap, int V, const int* draft_tokens, const int* parents,
                                  const int* tree_size, const float* target_probs, const float* uniforms,
                                  const int* status, int* accept_len, int* accept_path, int* bonus_token,
                                  void* workspace, size_t ws_bytes, void* stream) {
  if (B <= 0 || T_max <= 0 || dcap < 0 || dcap >= T_max || V <= 0) return TV_EINVAL;
  if (T_max > tv::kTMaxLimit || V > tv::kMaxPieces * tv::kPiece || B > 65535) return TV_EUNSUPPORTED;
  if (!draft_tokens || !parents || !tree_size || !target_probs || !uniforms || !status || !accept_len ||
      !accept_path || !bonus_token)
    return TV_EINVAL;
  const size_t zbytes = (size_t)B * T_max * sizeof(double);
  if (workspace && (ws_bytes < zbytes || (reinterpret_cast<uintptr_t>(workspace) & 7))) return TV_EWORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int vec4 = (V % 4 == 0) && ((reinterpret_cast<uintptr_t>(target_probs) & 15) == 0);
  // Every row's Z first, on as many CUs as there are rows, when reading all the
  // rows costs less than the walk's passes over the visited ones (up to 32 MB of
  // rows: a few microseconds; the walk spends a few per visited node).
  double* Z = nullptr;
  if (workspace && (double)B * T_max * V * sizeof(float) <= 32.0 * (1 << 20)) {
    Z = reinterpret_cast<double*>(workspace);
    hipLaunchKernelGGL(tv::k_row_mass, dim3(T_max, B), dim3(tv::kSampleThreads), 0, st, T_max, V, vec4, tree_size,
                       status, target_probs, Z);
    TV_CHECK_LAUNCH();
  }
  hipLaunchKernelGGL(tv::k_tree_accept_sample, dim3(B), dim3(tv::kSampleThreads), 0, st, T_max, dcap, V, vec4,
                     draft_tokens, parents, tree_size, target_probs, uniforms, status, Z, accept_len, accept_path,
                     bonus_token);
  TV_CHECK_LAUNCH();
  return TV_OK;
}

extern "C" int kv_compact(int B, int n_layers, int Hkv, int d, int elem_bytes, void* Kc, void* Vc, long long S_cap,
                          long long layer_stride_elems, const int* prefix_len, const int* accept_path,
                          const int* accept_len, int dcap, int* new_prefix_len, void* stream) {
  return tv::kv_compact_impl(B, n_layers, Hkv, d, elem_bytes, Kc, Vc, S_cap, (long long)B * Hkv * S_cap * d,
                             layer_stride_elems, prefix_len, accept_path, accept_len, dcap, new_prefix_len, stream,
                             tv::Paging{});
}

extern "C" int kv_compact_paged(int B, int n_layers, int Hkv, int d, int elem_bytes, void* K_pool, void* V_pool,
                                long long num_blocks, int tokens_per_block, const int* block_table,
                                int max_blocks_per_seq, long long layer_stride_elems, const int* prefix_len,
                                const int* accept_path, const int* accept_len, int dcap, int* new_prefix_len,
                                void* stream) {
  tv::Paging pg{};
  long long cap = 0, per_layer = 0;
  const int rc = tv::paged_args(B, Hkv, d, num_blocks, tokens_per_block, block_table, max_blocks_per_seq, &pg, &cap,
                                &per_layer);
  if (rc != TV_OK) return rc;
  return tv::kv_compact_impl(B, n_layers, Hkv, d, elem_bytes, K_pool, V_pool, cap, per_layer, layer_stride_elems,
                             prefix_len, accept_path, accept_len, dcap, new_prefix_len, stream, pg);
}

extern "C" int tree_accept_compact(int B, int T_max, int dcap, const int* draft_tokens, const int* parents,
                                   const int* tree_size, const int* target_predict, const int* status,
                                   int* accept_len, int* accept_path, int* bonus_token, int n_layers, int Hkv, int d,
                                   int elem_bytes, void* Kc, void* Vc, long long S_cap, long long layer_stride_elems,
                                   const int* prefix_len, int* new_prefix_len, void* stream) {
  return tv::accept_compact_impl(B, T_max, dcap, draft_tokens, parents, tree_size, target_predict, status, accept_len,
                                 accept_path, bonus_token, n_layers, Hkv, d, elem_bytes, Kc, Vc, S_cap,
                                 (long long)B * Hkv * S_cap * d, layer_stride_elems, prefix_len, new_prefix_len,
                                 stream, tv::Paging{});
}

extern "C" int tree_accept_compact_paged(int B, int T_max, int dcap, const int* draft_tokens, const int* parents,
                                         const int* tree_size, const int* target_predict, const int* status,
                                         int* accept_len, int* accept_path, int* bonus_token, int n_layers, int Hkv,
                                         int d, int elem_bytes, void* K_pool, void* V_pool, long long num_blocks,
                                         int tokens_per_block, const int* block_table, int max_blocks_per_seq,
                                         long long layer_stride_elems, const int* prefix_len, int* new_prefix_len,
                                         void* stream) {
  tv::Paging pg{};
  long long cap = 0, per_layer = 0;
  const int rc = tv::paged_args(B, Hkv, d, num_blocks, tokens_per_block, block_table, max_blocks_per_seq, &pg, &cap,
                                &per_layer);
  if (rc != TV_OK) return rc;
  return tv::accept_compact_impl(B, T_max, dcap, draft_tokens, parents, tree_size, target_predict, status, accept_len,
                                 accept_path, bonus_token, n_layers, Hkv, d, elem_bytes, K_pool, V_pool, cap,
                                 per_layer, layer_stride_elems, prefix_len, new_prefix_len, stream, pg);
}

extern "C" const char* tv_error_string(int code) {
  switch (code) {
    case TV_OK: return "ok";
    case TV_EINVAL: return "invalid argument";
    case TV_EUNSUPPORTED: return "unsupported size or type";
    case TV_EWORKSPACE: return "workspace missing or too small";
    case TV_ELAUNCH: return "kernel launch failed";
    default: return "unknown error";
  }
}

extern "C" const char* tv_status_string(int st) {
  switch (st) {
    case TV_ST_OK: return "ok";
    case TV_ST_PARENTS: return "malformed parents";
    case TV_ST_DEPTH: return "tree deeper than dcap";
    case TV_ST_SIZE: return "tree size out of range";
    case TV_ST_LOGPROB: return "invalid log-prob or unclosed tree";
    default: return "unknown status";
  }
}
