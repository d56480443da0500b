// tree_build: EAGLE-2 dynamic draft tree (global top-k over cumulative draft
// log-probs) and static branching trees, for gfx950.
//
// What is computed follows the EAGLE v2 walkthrough, section 3 (topK_generate:
// base layer top_k, `depth` rounds of cu_scores = topk_p + parent score with a
// global top_k over top_k*top_k, then the total_tokens best of all candidates),
// and the handbook's build_draft_tree for static branching.  Ties rank by
// (value descending, index ascending) everywhere.
//
// Kernels
//   k_row_topk    one workgroup per (draft row, vocabulary chunk): streams its
//                 chunk once with 16-byte loads (HBM-bound scan), bounds the
//                 chunk's K-th best entry by the K-th largest sixteen-lane group
//                 maximum, ranks the few entries that reach the bound and writes
//                 the chunk's sorted top-K keys (the select kernel merges chunks).
//   k_tree_select one workgroup per request: runs the D dependent K*K rounds and
//                 the final top-total_tokens selection (one bucket histogram of
//                 the score range, then an exact rank inside the boundary
//                 bucket) entirely in LDS, and writes the numbered tree.  Static
//                 mode builds level by level instead.
#include "tree_meta_body.h"

namespace tv {
namespace {

constexpr int kTopkThreads = 256;                       // one workgroup per (draft row, vocabulary chunk)
constexpr int kTopkVec = 8;                              // 16-byte loads per thread per tile
constexpr int kTopkTile = kTopkThreads * kTopkVec * 4;   // 8192 vocabulary entries
constexpr int kTopkGroups = kTopkThreads / 16;           // sixteen-lane groups per workgroup (>= K)
// A grid of row chunks that fits the chip in one pass (a single request) takes
// 512-thread workgroups over the same 8192-entry tiles (16 entries per thread):
// measured on MI355X for 61 rows x 32000, the step 48.4 -> 47.1 us; larger
// grids keep 256 threads (784 rows: 1% faster than 512, 20% faster than 1024).
constexpr int kTopkWideThreads = 512;
constexpr int kMaxSplit = 8;                             // vocabulary chunks per row
constexpr int kStageKeys = 6144;                         // chunk lists staged in the select kernel (48 KB)
static_assert(kTopkGroups >= kKMax, "the group-maximum bound needs at least K groups");
constexpr int kCandCap = 2048;                           // LDS candidate buffer (8 B each)
constexpr int kSelectThreads = 256;
// row keys staged per thread by the select kernels' single load batch
constexpr int kLoadBatch = 24;
static_assert(kLoadBatch * kSelectThreads >= kStageKeys, "one batch stages every chunk list");
constexpr int kMaxCand = 3072;   // LDS: 16 B per candidate
constexpr int kMaxLevels = 64;

struct Branching {
  int n;
  int w[kMaxLevels];
};

// A draft row is split into S vocabulary chunks, each ranked by its own
// workgroup, so that a small batch still spreads its rows over the CUs: one
// chunk per 8192 entries, at most kMaxSplit, and no more than the select
// kernel can stage next to its 16 B per candidate within 48 KB of dynamic LDS
// (R*K*16 + R*S*K*8 <= 8 * kStageKeys).
inline int pick_split(int V, int K, int R) {
  int S = (V + kTopkTile - 1) / kTopkTile;
  if (S > kMaxSplit) S = kMaxSplit;
  const long long rk = (long long)R * K;
  const long long cap = (kStageKeys - 2 * rk) / rk;
  if (S > cap) S = (int)cap;
  return S < 1 ? 1 : S;
}

// Workspace layout (rows = B * rows_per_req): K1 writes the sorted top-K rank
// keys and a bad-value flag of every (row, chunk); K2 merges a row's chunks.
struct BuildWs {
  unsigned long long* row_keys;  // [rows][S][K]
  int* row_bad;                  // [rows][S]
  int S;
  // raw-logit rows only: every (row, chunk)'s maximum and sum of exp(x - max)
  float* row_max;                // [rows][S]
  double* row_sum;               // [rows][S]
};

inline size_t build_ws_bytes(long long rows, int K, int S) {
  return (size_t)rows * S * ((size_t)K * 8 + 4) + 256;
}

inline BuildWs build_ws(void* base, long long rows, int K, int S) {
  BuildWs w;
  unsigned char* p = reinterpret_cast<unsigned char*>(base);
  w.row_keys = reinterpret_cast<unsigned long long*>(p);
  w.row_bad = reinterpret_cast<int*>(p + (size_t)rows * S * K * 8);
  w.S = S;
  w.row_max = nullptr;
  w.row_sum = nullptr;
  return w;
}

// The sorted top-K rank keys of every row of one request into LDS (s_key[row*K
// + r], r = rank in the row), and the OR of the rows' bad-value flags.  With S
// chunks per row, the chunk lists are staged in s_stage and merged by groups of
// G lanes (G = S rounded up to a power of two, one lane per chunk list): K
// rounds of a DPP group maximum over the list heads; the winning lane moves to
// its next key (already in a register) and prefetches two ahead.
template <int G>
__device__ void merge_chunk_lists(const unsigned long long* s_stage, int R, int K, int S,
                                  unsigned long long* s_key) {
  const int tid = threadIdx.x, c = tid % G;
  for (int row0 = 0; row0 < R; row0 += kSelectThreads / G) {
    const int row = row0 + tid / G;
    const bool live = row < R && c < S;
    const unsigned long long* lst = s_stage + ((long long)row * S + c) * K;
    // the head and the next two keys of this lane's list are in registers, so
    // the LDS read a win triggers is not needed before the round after next
    unsigned long long head = live ? lst[0] : 0ull;
    unsigned long long n1 = live && K > 1 ? lst[1] : 0ull;
    unsigned long long n2 = live && K > 2 ? lst[2] : 0ull;
    int ptr = 2;  // index of n2
    for (int k = 0; k < K; ++k) {
      const unsigned long long best = group_max_u64<G>(head);
      if (row < R && c == 0) s_key[row * K + k] = best;
      if (head == best && head != 0ull) {  // keys are unique: exactly one lane wins
        head = n1;
        n1 = n2;
        ++ptr;
        n2 = live && ptr < K ? lst[ptr] : 0ull;
      }
    }
  }
}

__device__ void load_row_keys(const BuildWs& ws, long long row_base, int R, int K, unsigned long long* s_key,
                              unsigned long long* s_stage, int* s_bad) {
  const int S = ws.S;
  const long long base = row_base * S * K;
  // global -> LDS, every load of the block in flight together (n <= 24 per thread)
  unsigned long long* dst = S == 1 ? s_key : s_stage;
  const int n = R * S * K;
  for (int i0 = 0; i0 < n; i0 += kLoadBatch * kSelectThreads) {
    unsigned long long v[kLoadBatch];
#pragma unroll
    for (int u = 0; u < kLoadBatch; ++u) {
      const int i = i0 + u * kSelectThreads + threadIdx.x;
      v[u] = i < n ? ws.row_keys[base + i] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < kLoadBatch; ++u) {
      const int i = i0 + u * kSelectThreads + threadIdx.x;
      if (i < n) dst[i] = v[u];
    }
  }
  for (int i = threadIdx.x; i < R * S; i += blockDim.x)
    if (ws.row_bad[row_base * S + i]) *s_bad = 1;
  if (S == 1) return;
  __syncthreads();
  if (S <= 2) merge_chunk_lists<2>(s_stage, R, K, S, s_key);
  else if (S <= 4) merge_chunk_lists<4>(s_stage, R, K, S, s_key);
  else if (S <= 8) merge_chunk_lists<8>(s_stage, R, K, S, s_key);
  else merge_chunk_lists<16>(s_stage, R, K, S, s_key);
}

typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}

// max over aligned groups of 16 lanes (every lane gets the result)
__device__ __forceinline__ uint32_t group16_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));
  v = max(v, dpp_u32<0x4E>(v));
  v = max(v, dpp_u32<0x141>(v));
  return max(v, dpp_u32<0x140>(v));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = group16_max_u32(v);
  return max(max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
             max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}

// Unique 64-bit rank key of vocabulary entry idx whose order key is k32.
__device__ __forceinline__ unsigned long long make_key64(uint32_t k32, uint32_t idx) {
  return ((unsigned long long)k32 << 32) | (unsigned long long)(0xFFFFFFFFu - idx);
}

// --------------------------------------------------------------------------
// K1: the K best entries of one draft row, by (log-prob desc, token asc).
//
// The row is read in tiles of 32768 entries held in registers (eight 16-byte
// loads per thread, all in flight together).  Per tile:
//   1. every sixteen-lane group takes the maximum of its 16 x 32 entries;
//   2. tau = the largest group maximum that at least K group maxima reach:
//      K distinct entries are >= tau, so no entry below tau is in the top-K;
//   3. entries >= tau that beat the K-th best of the earlier tiles are
//      appended to an LDS buffer next to those K (typically a dozen);
//   4. an exact rank count among the buffer gives the new sorted top-K.
// A buffer overflow (heavy ties, e.g. a constant row) switches that tile to a
// bisection on the unique 64-bit keys, which is exact for any input.
// LOGITS: the row holds raw logits (any finite value; NaN and +-inf are bad
// values), ranked by logit, and the pass also leaves the chunk's maximum m and
// sum of exp(x - m) in float64 (each thread keeps its own running pair, rescaled
// when its maximum rises; the workgroup merges them), from which the layer
// kernel forms the row's log-sum-exp.
// --------------------------------------------------------------------------
template <bool LOGITS, int NT = kTopkThreads>
__global__ __launch_bounds__(NT) void k_row_topk(const float* __restrict__ lp, int V, int K, int vec4, BuildWs ws) {
  constexpr int kTopkThreads = NT;                        // (this instance's workgroup size)
  constexpr int kTopkVec = kTopkTile / (4 * NT);          // 16-byte loads per thread per tile
  constexpr int kTopkGroups = NT / 16;
  static_assert(kTopkVec * 4 * NT == kTopkTile && kTopkGroups >= kKMax, "one tile of 8192 entries, >= K groups");
  const int S = ws.S;
  const long long row = blockIdx.x / S;
  const int chunk = blockIdx.x % S;
  const float* r = lp + row * (long long)V;
  // this workgroup's vocabulary range (a multiple of 4 long, so 16-byte loads stay aligned)
  const int span = ((V + S - 1) / S + 3) & ~3;
  const int begin = chunk * span, end = min(V, begin + span);
  const int tid = threadIdx.x, lane = tid & 63;
  __shared__ __attribute__((aligned(16))) unsigned long long s_cand[kCandCap + 16];  // + one batch of slack
  __shared__ unsigned long long s_best[kKMax];
  __shared__ __attribute__((aligned(16))) uint32_t s_gmax[kTopkGroups];
  __shared__ int s_n, s_bad, s_cnt[3];

  if (tid == 0) s_bad = 0;
  bool bad = false;
  int have = 0;                       // entries in s_best: 0 before the first tile, then K
  unsigned long long tau_run = 0ull;  // K-th best key of the earlier tiles (0: none)
  float lse_m = -INFINITY;            // LOGITS: this thread's running maximum and sum of exp(x - max)
  double lse_s = 0.0;
  // LOGITS: fold this thread's finite entries of a tile into (lse_m, lse_s)
  auto lse_add = [&](const float* xs, auto in_of) __attribute__((always_inline)) {
    float tm = -INFINITY;
#pragma unroll
    for (int j = 0; j < kTopkVec * 4; ++j)
      if (in_of(j) && isfinite(xs[j])) tm = fmaxf(tm, xs[j]);
    if (tm > lse_m) {
      lse_s = lse_m == -INFINITY ? 0.0 : lse_s * exp((double)lse_m - (double)tm);
      lse_m = tm;
    }
#pragma unroll
    for (int j = 0; j < kTopkVec * 4; ++j)
      if (in_of(j) && isfinite(xs[j])) lse_s += exp((double)xs[j] - (double)lse_m);
  };

  for (int t0 = begin; t0 < end; t0 += kTopkTile) {
    // entry j (0..31) of this thread: vocabulary index idx_of(j)
    auto idx_of = [&](int j) -> int {
      return vec4 ? t0 + 4 * ((j >> 2) * kTopkThreads + tid) + (j & 3) : t0 + j * kTopkThreads + tid;
    };
    uint32_t k[kTopkVec * 4];
    if (vec4) {
      typedef float f4 __attribute__((ext_vector_type(4)));
      const f4* r4 = reinterpret_cast<const f4*>(r);
      const int last4 = end / 4 - 1;
      f4 x[kTopkVec];
#pragma unroll
      for (int i = 0; i < kTopkVec; ++i)  // clamped addresses: every load is in bounds and issued at once
        x[i] = __builtin_nontemporal_load(r4 + min(t0 / 4 + i * kTopkThreads + tid, last4));
      // (end is a multiple of 4 here, so a vector is inside the range or past it as a whole)
#pragma unroll
      for (int i = 0; i < kTopkVec; ++i) {
        const bool in = t0 / 4 + i * kTopkThreads + tid <= last4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = x[i][e];
          bad |= in && (LOGITS ? !isfinite(v) : !(v <= 0.0f));  // log-probs: NaN or positive
          // order_key(v): -0.0 + 0.0 = +0.0, then the sign-dependent flip
          const uint32_t u = __float_as_uint(v + 0.0f);
          k[4 * i + e] = in ? u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u) : 0u;
        }
      }
      if constexpr (LOGITS) {
        float xs[kTopkVec * 4];
#pragma unroll
        for (int j = 0; j < kTopkVec * 4; ++j) xs[j] = x[j >> 2][j & 3];
        lse_add(xs, [&](int j) { return idx_of(j) < end; });
      }
    } else {
      float x[kTopkVec * 4];
#pragma unroll
      for (int j = 0; j < kTopkVec * 4; ++j) x[j] = r[min(idx_of(j), end - 1)];
#pragma unroll
      for (int j = 0; j < kTopkVec * 4; ++j) {
        const bool in = idx_of(j) < end;
        bad |= in && (LOGITS ? !isfinite(x[j]) : !(x[j] <= 0.0f));
        k[j] = in ? order_key(x[j]) : 0u;
      }
      if constexpr (LOGITS) lse_add(x, [&](int j) { return idx_of(j) < end; });
    }
    uint32_t tmax = 0u;
#pragma unroll
    for (int j = 0; j < kTopkVec * 4; ++j) tmax = max(tmax, k[j]);
    tmax = group16_max_u32(tmax);
    if ((lane & 15) == 0) s_gmax[tid >> 4] = tmax;
    if (tid < have) s_cand[tid] = s_best[tid];
    if (tid == 0) s_n = have;
    __syncthreads();

    // tau (every wave computes it): lane l holds group maximum g_l and counts
    // the group maxima >= g_l; tau = max { g_l : count >= K }
    uint32_t tau;
    {
      const uint32_t g = lane < kTopkGroups ? s_gmax[lane] : 0u;  // lanes past the groups hold nothing
      int c = 0;
      const uint4* g4 = reinterpret_cast<const uint4*>(s_gmax);
#pragma unroll
      for (int i = 0; i < kTopkGroups / 4; ++i) {
        const uint4 q = g4[i];
        c += (q.x >= g) + (q.y >= g) + (q.z >= g) + (q.w >= g);
      }
      const uint32_t t = group16_max_u32(c >= K ? g : 0u);
      tau = max(max((uint32_t)__builtin_amdgcn_readlane((int)t, 0), (uint32_t)__builtin_amdgcn_readlane((int)t, 16)),
                max((uint32_t)__builtin_amdgcn_readlane((int)t, 32), (uint32_t)__builtin_amdgcn_readlane((int)t, 48)));
    }
#pragma unroll
    for (int j = 0; j < kTopkVec * 4; ++j) {
      if (k[j] != 0u && k[j] >= tau) {
        const unsigned long long kk = make_key64(k[j], (uint32_t)idx_of(j));
        if (kk > tau_run) {
          const int slot = atomicAdd(&s_n, 1);
          if (slot < kCandCap) s_cand[slot] = kk;
        }
      }
    }
    __syncthreads();
    int n = s_n;

    if (n > kCandCap) {
      // exact fallback: the K-th largest unique key x of (earlier best, this
      // tile) by bisection on count(key >= x) >= K, then exactly K candidates
      if (tid < 3) s_cnt[tid] = 0;
      __syncthreads();
      unsigned long long lo = 1ull, hi = ~0ull;  // count(lo) >= K always holds
      for (int it = 0; lo < hi; ++it) {
        const unsigned long long mid = lo + (hi - lo) / 2 + 1;
        int c = (tid < have && s_best[tid] >= mid) ? 1 : 0;
#pragma unroll
        for (int j = 0; j < kTopkVec * 4; ++j) c += k[j] != 0u && make_key64(k[j], (uint32_t)idx_of(j)) >= mid;
        if (c) atomicAdd(&s_cnt[it % 3], c);
        __syncthreads();
        const int tot = s_cnt[it % 3];
        if (tid == 0) s_cnt[(it + 2) % 3] = 0;
        if (tot >= K) lo = mid;
        else hi = mid - 1;
      }
      __syncthreads();
      if (tid == 0) s_n = 0;
      __syncthreads();
      if (tid < have && s_best[tid] >= lo) s_cand[atomicAdd(&s_n, 1)] = s_best[tid];
#pragma unroll
      for (int j = 0; j < kTopkVec * 4; ++j) {
        const unsigned long long kk = make_key64(k[j], (uint32_t)idx_of(j));
        if (k[j] != 0u && kk >= lo) s_cand[atomicAdd(&s_n, 1)] = kk;
      }
      __syncthreads();
      n = s_n;  // == K
    }

    // exact rank among the n unique candidates; the K best, in order, to s_best
    // (16 keys per batch, all reads in flight; entries past n are not counted)
    for (int t = tid; t < n; t += kTopkThreads) {
      const unsigned long long my = s_cand[t];
      int rk = 0;
      for (int o0 = 0; o0 < n; o0 += 16) {
        u64x2 x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = reinterpret_cast<const u64x2*>(s_cand + o0)[u];
#pragma unroll
        for (int u = 0; u < 8; ++u) rk += (o0 + 2 * u < n && x[u][0] > my) + (o0 + 2 * u + 1 < n && x[u][1] > my);
      }
      if (rk < K) s_best[rk] = my;
    }
    __syncthreads();
    have = K;
    tau_run = s_best[K - 1];
  }
  if (bad) s_bad = 1;
  if constexpr (LOGITS) {
    // merge the threads' (max, sum) pairs: the chunk's maximum first (shuffles,
    // then the wavefronts' maxima through LDS), then each thread rescales its own
    // sum to it (one exponential each, all in parallel) and the sums are added
    __shared__ float s_lm[kTopkThreads / 64];
    __shared__ double s_ls[kTopkThreads / 64];
    float M = lse_m;
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    if (lane == 0) s_lm[tid >> 6] = M;
    __syncthreads();
    M = s_lm[0];
#pragma unroll
    for (int w = 1; w < kTopkThreads / 64; ++w) M = fmaxf(M, s_lm[w]);
    double part = lse_m == -INFINITY ? 0.0 : lse_s * exp((double)lse_m - (double)M);
    for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
    if (lane == 0) s_ls[tid >> 6] = part;
    __syncthreads();
    if (tid == 0) {
      double sum = 0.0;
      for (int w = 0; w < kTopkThreads / 64; ++w) sum += s_ls[w];
      ws.row_max[row * S + chunk] = M;
      ws.row_sum[row * S + chunk] = sum;
    }
  }
  __syncthreads();
  if (tid < K) ws.row_keys[(row * S + chunk) * K + tid] = s_best[tid];
  if (tid == 0) ws.row_bad[row * S + chunk] = s_bad;
}

// --------------------------------------------------------------------------
// K2 helpers
// --------------------------------------------------------------------------
// Inclusive prefix sum over the 64 lanes of a wavefront with DPP (no LDS round
// trip): shifts by 1, 2, 4, 8 inside each 16-lane row (lanes shifted in from
// outside the row read 0), then row 0's total is broadcast into row 1 and row
// 2's into row 3 (row_bcast:15), and rows 0-1's total into rows 2 and 3
// (row_bcast:31).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);
  return v;
}

// Block-wide exclusive scan of one int per thread; returns the exclusive prefix
// and writes the total to *total.
__device__ int block_excl_scan(int v, int* s_tmp, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int x = wave_incl_scan(v);
  if (lane == 63) s_tmp[wave] = x;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < kSelectThreads / 64; ++w) {
    if (w < wave) base += s_tmp[w];
    tot += s_tmp[w];
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

__device__ unsigned long long block_reduce_u64(unsigned long long v, bool take_max, unsigned long long* s_tmp) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const unsigned long long o = shfl_xor_u64(v, m);
    v = take_max ? (o > v ? o : v) : (o < v ? o : v);
  }
  if (lane == 0) s_tmp[wave] = v;
  __syncthreads();
  v = s_tmp[0];
  for (int w = 1; w < kSelectThreads / 64; ++w) v = take_max ? (s_tmp[w] > v ? s_tmp[w] : v) : (s_tmp[w] < v ? s_tmp[w] : v);
  __syncthreads();
  return v;
}

// Radix select: threshold tau such that exactly n of the C unique keys
// rank_key(s_sc[id], id) are >= tau.  Digits of 8 bits, starting at the first
// byte where the largest and smallest key differ.
__device__ unsigned long long radix_select_threshold(const int C, const int n, const float* s_sc, int* s_hist,
                                                     unsigned long long* s_bcast, unsigned long long* s_tmp) {
  const int tid = threadIdx.x;
  if (n <= 0) return ~0ull;  // nothing: no key reaches all-ones
  if (n >= C) return 0ull;
  unsigned long long kmax = 0ull, kmin = ~0ull;
  for (int id = tid; id < C; id += kSelectThreads) {
    const unsigned long long k = rank_key(s_sc[id], (uint32_t)id);
    kmax = k > kmax ? k : kmax;
    kmin = k < kmin ? k : kmin;
  }
  kmax = block_reduce_u64(kmax, true, s_tmp);
  kmin = block_reduce_u64(kmin, false, s_tmp);
  int shift = 56;
  while (shift > 0 && ((kmax ^ kmin) >> shift) == 0ull) shift -= 8;
  // bytes above `shift` are common to every key: they form the starting prefix
  unsigned long long mask = shift == 56 ? 0ull : ~((1ull << (shift + 8)) - 1ull);
  unsigned long long prefix = kmax & mask;
  int need = n;
  for (; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += kSelectThreads) s_hist[i] = 0;
    __syncthreads();
    for (int id = tid; id < C; id += kSelectThreads) {
      const unsigned long long k = rank_key(s_sc[id], (uint32_t)id);
      if ((k & mask) == prefix) atomicAdd(&s_hist[(k >> shift) & 255], 1);
    }
    __syncthreads();
    if (tid < 64) {
      // lane owns bins 4*(63-lane) .. +3 (lane 0 owns the top bins)
      const int b0 = 4 * (63 - tid);
      const int h3 = s_hist[b0 + 3], h2 = s_hist[b0 + 2], h1 = s_hist[b0 + 1], h0 = s_hist[b0];
      const int mine = h0 + h1 + h2 + h3;
      const int incl = wave_incl_scan(mine);
      const int above = incl - mine;  // keys in strictly higher bins
      if (above < need && need <= incl) {
        int a = above, digit, cnt;
        if (need <= a + h3) { digit = b0 + 3; cnt = h3; }
        else if (need <= a + h3 + h2) { a += h3; digit = b0 + 2; cnt = h2; }
        else if (need <= a + h3 + h2 + h1) { a += h3 + h2; digit = b0 + 1; cnt = h1; }
        else { a += h3 + h2 + h1; digit = b0; cnt = h0; }
        s_bcast[0] = (unsigned long long)digit;
        s_bcast[1] = (unsigned long long)(need - a);   // still needed inside the bin
        s_bcast[2] = (unsigned long long)cnt;
      }
    }
    __syncthreads();
    const int digit = (int)s_bcast[0];
    const int rem = (int)s_bcast[1];
    const int cnt = (int)s_bcast[2];
    __syncthreads();
    prefix |= (unsigned long long)digit << shift;
    mask |= 255ull << shift;
    need = rem;
    if (need == cnt) break;  // the whole bin is kept
  }
  return prefix;
}

// Threshold of the n best of the C candidates under (score desc, id asc):
// returns tau such that exactly n of the unique keys rank_key(s_sc[id], id) are
// >= tau.  One histogram of the 32-bit score keys over at most kBuckets
// equal-width buckets of their range [kmin, kmax] finds the bucket that holds
// the boundary;
// its members are ranked exactly by their 64-bit keys.  A boundary bucket with
// more than kBucketRankMax members (heavy ties) falls back to the radix select.
constexpr int kBucketBits = 10;
constexpr int kBuckets = 1 << kBucketBits;
static_assert(kBuckets == 4 * kSelectThreads, "four buckets per thread in the boundary scan");
constexpr int kBucketRankMax = 256;

__device__ unsigned long long bucket_select_threshold(const int C, const int n, const float* s_sc, uint32_t kmin,
                                                      uint32_t kmax, int* s_hist, short* s_mem, int* s_misc,
                                                      int* s_tmp, unsigned long long* s_bcast,
                                                      unsigned long long* s_tmp64) {
  const int tid = threadIdx.x;
  if (n <= 0) return ~0ull;  // nothing: no key reaches all-ones
  if (n >= C) return 0ull;
  for (int i = tid; i < kBuckets; i += kSelectThreads) s_hist[i] = 0;
  if (tid == 0) s_misc[1] = 0;
  __syncthreads();
  const uint32_t range = kmax - kmin;
  // buckets used: (range >> shift) + 1 <= kBuckets
  const int shift = range < (uint32_t)kBuckets ? 0 : 32 - __clz(range) - kBucketBits;
  for (int id = tid; id < C; id += kSelectThreads) atomicAdd(&s_hist[(order_key(s_sc[id]) - kmin) >> shift], 1);
  __syncthreads();
  // thread t owns buckets b0..b0+3, thread 0 the top four; count from the top
  const int b0 = kBuckets - 4 - 4 * tid;
  const int h3 = s_hist[b0 + 3], h2 = s_hist[b0 + 2], h1 = s_hist[b0 + 1], h0 = s_hist[b0];
  const int mine = h0 + h1 + h2 + h3;
  int total = 0;
  const int above = block_excl_scan(mine, s_tmp, &total);
  if (above < n && n <= above + mine) {
    int a = above, bk;
    if (n <= a + h3) bk = b0 + 3;
    else if (n <= a + h3 + h2) { a += h3; bk = b0 + 2; }
    else if (n <= a + h3 + h2 + h1) { a += h3 + h2; bk = b0 + 1; }
    else { a += h3 + h2 + h1; bk = b0; }
    s_misc[0] = bk;
    s_misc[2] = n - a;  // still needed inside the bucket
  }
  __syncthreads();
  const uint32_t bstar = (uint32_t)s_misc[0];
  const int need = s_misc[2];
  for (int id = tid; id < C; id += kSelectThreads)
    if (((order_key(s_sc[id]) - kmin) >> shift) == bstar) {
      const int slot = atomicAdd(&s_misc[1], 1);
      if (slot < kBucketRankMax) s_mem[slot] = (short)id;
    }
  __syncthreads();
  const int m = s_misc[1];
  if (m > kBucketRankMax) return radix_select_threshold(C, n, s_sc, s_hist, s_bcast, s_tmp64);
  for (int t = tid; t < m; t += kSelectThreads) {
    const int id = s_mem[t];
    const unsigned long long my = rank_key(s_sc[id], (uint32_t)id);
    int rk = 0;
    for (int o = 0; o < m; ++o) {
      const int io = s_mem[o];
      rk += rank_key(s_sc[io], (uint32_t)io) > my;
    }
    if (rk == need - 1) s_bcast[3] = my;
  }
  __syncthreads();
  return s_bcast[3];
}

// With META, the first wavefront then also runs tree_mask_positions on the tree
// just built (its parents taken from LDS), so the step saves a launch.
template <int K, bool META>
__global__ __launch_bounds__(kSelectThreads) void k_tree_select_dynamic(
    BuildWs ws, int R, int D, int total_tokens, const int* __restrict__ root_token, int T_max,
    int* __restrict__ draft_tokens, int* __restrict__ parents, int* __restrict__ tree_size,
    float* __restrict__ node_score, int* __restrict__ status, MetaOut mo) {
  extern __shared__ unsigned char smem[];
  const int C = R * K;  // = K + D*K*K: candidate id == row*K + rank
  unsigned long long* s_key = reinterpret_cast<unsigned long long*>(smem);
  float* s_sc = reinterpret_cast<float*>(s_key + C);
  short* s_par = reinterpret_cast<short*>(s_sc + C);
  short* s_node = s_par + C;
  __shared__ int s_hist[kBuckets];
  __shared__ short s_mem[kBucketRankMax];
  __shared__ int s_misc[4];
  __shared__ unsigned long long s_bcast[4], s_tmp64[kSelectThreads / 64];
  __shared__ int s_front[2][kKMax];
  __shared__ float s_fsc[2][kKMax];
  __shared__ __attribute__((aligned(16))) unsigned long long s_cand[kKMax * kKMax + 32];
  __shared__ float s_cand_sc[kKMax * kKMax];
  __shared__ uint32_t s_krange[2];
  __shared__ int s_tmp[kSelectThreads / 64];
  __shared__ int s_bad;
  __shared__ int s_pn[META ? kTMaxLimit : 1];  // parent of each node (META)

  const int b = blockIdx.x, tid = threadIdx.x;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  load_row_keys(ws, (long long)b * R, R, K, s_key, reinterpret_cast<unsigned long long*>(s_node + C), &s_bad);
  __syncthreads();
  for (int id = tid; id < C; id += kSelectThreads) {
    s_sc[id] = key_value(s_key[id]);
    s_par[id] = -1;
  }
  if (tid < K) {
    s_front[0][tid] = tid;
    s_fsc[0][tid] = key_value(s_key[tid]);
  }
  __syncthreads();

  // D dependent rounds: the K*K cumulative scores of a layer, then its K best
  // (score desc, index asc) become the next frontier.  Wavefront 0 runs them
  // alone, so no workgroup barrier is needed inside a round:
  //   1. each lane forms the scores of candidates lane + 64 i in registers
  //      (and records score and parent slot in LDS for the final selection);
  //   2. tau = the worst of the K list heads (candidate j*K is the best child of
  //      frontier slot j): K distinct candidates reach tau, so nothing below it
  //      can be in the frontier;
  //   3. the candidates >= tau are compacted into LDS (ballot + mbcnt);
  //   4. an exact rank count among them places the K best.
  constexpr int KK = K * K;
  constexpr int kPerLane = (KK + 63) / 64;
  // order-key range of every candidate score (wavefront 0), for the final selection
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  if (tid < 64) {
    if (tid < K) kmin = kmax = order_key(key_value(s_key[tid]));
    for (int l = 1; l <= D; ++l) {
      const int cur = (l - 1) & 1, nxt = l & 1;
      const int base = K + (l - 1) * KK;
      unsigned long long key[kPerLane];
      float sc[kPerLane];
#pragma unroll
      for (int i = 0; i < kPerLane; ++i) {
        const int o = tid + 64 * i;
        key[i] = 0ull;
        sc[i] = 0.0f;
        if (o < KK) {
          const int j = o / K;
          sc[i] = __fadd_rn(key_value(s_key[base + o]), s_fsc[cur][j]);
          s_sc[base + o] = sc[i];
          s_par[base + o] = (short)s_front[cur][j];
          key[i] = rank_key(sc[i], (uint32_t)o);
          const uint32_t k32 = (uint32_t)(key[i] >> 32);
          kmin = min(kmin, k32);
          kmax = max(kmax, k32);
        }
      }
      // the list heads (candidate j*K, the best child of slot j) in lanes 0..K-1
      unsigned long long head = ~0ull;
      if (tid < K) head = rank_key(__fadd_rn(key_value(s_key[base + tid * K]), s_fsc[cur][tid]), (uint32_t)(tid * K));
      const unsigned long long tau = readlane_u64(~group_max_u64<16>(~head), 0);
      int n = 0;
#pragma unroll
      for (int i = 0; i < kPerLane; ++i) {
        const bool keep = key[i] != 0ull && key[i] >= tau;
        const unsigned long long m = __ballot(keep);
        const int pos = n + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (keep) {
          s_cand[pos] = key[i];
          s_cand_sc[pos] = sc[i];
        }
        n += __popcll(m);
      }
      if (tid < 32) s_cand[n + tid] = 0ull;  // zero keys pad the last batch
      wave_sync();
      for (int t = tid; t < n; t += 64) {
        const unsigned long long my = s_cand[t];
        const float my_sc = s_cand_sc[t];
        int rk = 0;
        for (int o0 = 0; o0 < n; o0 += 32) {  // 32 keys per batch, all reads in flight
          u64x2 x[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) x[u] = reinterpret_cast<const u64x2*>(s_cand + o0)[u];
#pragma unroll
          for (int u = 0; u < 16; ++u) rk += (x[u][0] > my) + (x[u][1] > my);
        }
        if (rk < K) {
          s_front[nxt][rk] = base + (int)key_index(my);
          s_fsc[nxt][rk] = my_sc;
        }
      }
      wave_sync();
    }
    kmin = ~wave_max_u32(~kmin);
    kmax = wave_max_u32(kmax);
    if (tid == 0) {
      s_krange[0] = kmin;
      s_krange[1] = kmax;
    }
  }
  __syncthreads();

  // final: keep the total_tokens best candidates, number them by ascending id
  const unsigned long long tau = bucket_select_threshold(C, total_tokens, s_sc, s_krange[0], s_krange[1], s_hist,
                                                        s_mem, s_misc, s_tmp, s_bcast, s_tmp64);
  const int per = (C + kSelectThreads - 1) / kSelectThreads;
  const int lo = min(C, tid * per), hi = min(C, lo + per);
  int cnt = 0;
  for (int id = lo; id < hi; ++id) cnt += rank_key(s_sc[id], (uint32_t)id) >= tau;
  int total = 0;
  int node = 1 + block_excl_scan(cnt, s_tmp, &total);
  for (int id = lo; id < hi; ++id) {
    const bool keep = rank_key(s_sc[id], (uint32_t)id) >= tau;
    s_node[id] = keep ? (short)node++ : (short)-1;
  }
  __syncthreads();
  // closure check: a kept node's parent must be kept
  for (int id = tid; id < C; id += kSelectThreads)
    if (s_node[id] > 0 && s_par[id] >= 0 && s_node[s_par[id]] < 0) s_bad = 1;
  __syncthreads();

  const long long ob = (long long)b * T_max;
  const bool ok = s_bad == 0;
  const int T = ok ? total + 1 : 1;
  // the root and the padding; kept nodes 1..T-1 are written from their candidates
  for (int i = tid; i < T_max; i += kSelectThreads)
    if (i == 0 || i >= T) {
      draft_tokens[ob + i] = i == 0 ? root_token[b] : -1;
      parents[ob + i] = -1;
      if (node_score) node_score[ob + i] = i == 0 ? 0.0f : -INFINITY;
    }
  if (ok) {
    for (int id = tid; id < C; id += kSelectThreads) {
      const int n = s_node[id];
      if (n > 0) {
        const int pn = s_par[id] < 0 ? 0 : s_node[s_par[id]];
        draft_tokens[ob + n] = (int)key_index(s_key[id]);
        parents[ob + n] = pn;
        if (node_score) node_score[ob + n] = s_sc[id];
        if constexpr (META) s_pn[n] = pn;
      }
    }
  }
  if (tid == 0) tree_size[b] = T;
  if constexpr (!META) {
    if (tid == 0) status[b] = ok ? TV_ST_OK : TV_ST_LOGPROB;
  } else {
    __syncthreads();
    if (T_max <= 64) {
      if (tid < 64) {
        int st = ok ? TV_ST_OK : TV_ST_LOGPROB, Tm = T;
        const int P = mo.prefix_len[b];
        const int p = check_tree(tid, T_max, st, Tm, (tid > 0 && tid < T) ? s_pn[tid] : -1);
        meta_body(b, tid, T_max, mo.dcap, mo.W, Tm, st, p, P, mo.tree_mask, mo.tree_position_ids, mo.positions,
                  mo.retrieve_indices, mo.leaf_count, mo.first_child, mo.next_sibling, status);
      }
    } else {  // up to 256 nodes: every thread of the workgroup is one node
      __shared__ WideShared sh_wide;
      int st = ok ? TV_ST_OK : TV_ST_LOGPROB, Tm = T;
      const int P = mo.prefix_len[b];
      const int p = check_tree_wide(tid, T_max, st, Tm, (tid > 0 && tid < T) ? s_pn[tid] : -1, sh_wide);
      meta_body_wide(b, tid, T_max, mo.dcap, mo.W, Tm, st, p, P, mo.tree_mask, mo.tree_position_ids, mo.positions,
                     mo.retrieve_indices, mo.leaf_count, mo.first_child, mo.next_sibling, status, sh_wide);
    }
  }
}

template <bool META>
__global__ __launch_bounds__(kSelectThreads) void k_tree_select_static(
    BuildWs ws, int R, int K, Branching br, const int* __restrict__ root_token, int T_max,
    int* __restrict__ draft_tokens, int* __restrict__ parents, int* __restrict__ tree_size,
    float* __restrict__ node_score, int* __restrict__ status, MetaOut mo) {
  extern __shared__ unsigned char smem[];
  unsigned long long* rk = reinterpret_cast<unsigned long long*>(smem);
  __shared__ int t_tok[kTMaxLimit], t_par[kTMaxLimit];
  __shared__ float t_sc[kTMaxLimit];
  __shared__ int s_T, s_bad;
  const int b = blockIdx.x, tid = threadIdx.x;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  load_row_keys(ws, (long long)b * R, R, K, rk, rk + R * K, &s_bad);
  __syncthreads();
  if (tid == 0) {
    // level by level: every frontier node, in order, appends its row's top-w
    int T = 1;
    t_tok[0] = root_token[b];
    t_par[0] = -1;
    t_sc[0] = 0.0f;
    int fs = 0, fe = 1;
    for (int l = 0; l < br.n; ++l) {
      const int w = br.w[l];
      for (int nd = fs; nd < fe; ++nd)
        for (int r = 0; r < w; ++r) {
          const unsigned long long k = rk[nd * K + r];
          t_tok[T] = (int)key_index(k);
          t_par[T] = nd;
          t_sc[T] = __fadd_rn(key_value(k), t_sc[nd]);
          ++T;
        }
      fs = fe;
      fe = T;
    }
    s_T = T;
  }
  __syncthreads();
  const bool ok = s_bad == 0;
  const int T = ok ? s_T : 1;
  const long long ob = (long long)b * T_max;
  for (int i = tid; i < T_max; i += kSelectThreads) {
    const bool in = i < T;
    draft_tokens[ob + i] = i == 0 ? root_token[b] : (in ? t_tok[i] : -1);
    parents[ob + i] = in ? t_par[i] : -1;
    if (node_score) node_score[ob + i] = i == 0 ? 0.0f : (in ? t_sc[i] : -INFINITY);
  }
  if (tid == 0) tree_size[b] = T;
  if constexpr (!META) {
    if (tid == 0) status[b] = ok ? TV_ST_OK : TV_ST_LOGPROB;
  } else {
    if (T_max <= 64) {
      if (tid < 64) {  // t_par was published by the barrier after the levels
        int st = ok ? TV_ST_OK : TV_ST_LOGPROB, Tm = T;
        const int P = mo.prefix_len[b];
        const int p = check_tree(tid, T_max, st, Tm, (tid > 0 && tid < T) ? t_par[tid] : -1);
        meta_body(b, tid, T_max, mo.dcap, mo.W, Tm, st, p, P, mo.tree_mask, mo.tree_position_ids, mo.positions,
                  mo.retrieve_indices, mo.leaf_count, mo.first_child, mo.next_sibling, status);
      }
    } else {  // up to 256 nodes: every thread of the workgroup is one node
      __shared__ WideShared sh_wide;
      int st = ok ? TV_ST_OK : TV_ST_LOGPROB, Tm = T;
      const int P = mo.prefix_len[b];
      const int p = check_tree_wide(tid, T_max, st, Tm, (tid > 0 && tid < T) ? t_par[tid] : -1, sh_wide);
      meta_body_wide(b, tid, T_max, mo.dcap, mo.W, Tm, st, p, P, mo.tree_mask, mo.tree_position_ids, mo.positions,
                     mo.retrieve_indices, mo.leaf_count, mo.first_child, mo.next_sibling, status, sh_wide);
    }
  }
}

// --------------------------------------------------------------------------
// Layer-by-layer build ([E2] section 3: the draft model runs on each round's
// frontier, so a round's rows exist only after the round before it).  The state
// keeps every layer's merged row lists in the layout the select kernel reads
// (one chunk per row), so tree_build_finish is k_tree_select_dynamic on it: it
// replays the rounds (the same float32 adds and ranking, hence the same
// frontiers) and makes the final selection.
// --------------------------------------------------------------------------
struct LayerState {
  unsigned long long* keys;  // [B][R][K] sorted rank keys of every row (R = 1 + D K)
  int* bad;                  // [B][R]
  float* fsc;                // [B][K] scores of the current frontier
};

// Merge one layer's rows (1 at layer 0, else K: row j = frontier slot j) into
// the state, and choose the next frontier: at layer 0 the root row's K best, at
// layer l the K best of the K*K cumulative scores fl32(log-prob + score of slot
// j), ranked (score desc, jK + r asc) -- the rounds of k_tree_select_dynamic.
template <int K, bool LOGITS>
__global__ __launch_bounds__(kSelectThreads) void k_build_layer(BuildWs rws, int layer, int R, LayerState st,
                                                                int* __restrict__ frontier_tokens,
                                                                int* __restrict__ frontier_parents) {
  extern __shared__ unsigned char smem[];  // chunk lists of this layer's rows (when a row has several)
  constexpr int KK = K * K;
  __shared__ unsigned long long s_key[KK];
  __shared__ __attribute__((aligned(16))) unsigned long long s_ck[KK + 2];
  __shared__ float s_fsc[K];
  __shared__ double s_lse[K];
  __shared__ int s_bad;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int Rl = layer == 0 ? 1 : K;
  if (tid == 0) s_bad = 0;
  if (layer > 0 && tid < K) s_fsc[tid] = st.fsc[(long long)b * K + tid];
  __syncthreads();
  load_row_keys(rws, (long long)b * Rl, Rl, K, s_key, reinterpret_cast<unsigned long long*>(smem), &s_bad);
  __syncthreads();
  if constexpr (LOGITS) {
    // log-sum-exp of each row from its chunks' (max, sum), then every kept logit
    // becomes its log-prob fl32(x - lse); the order inside a row is the logits'
    // one thread per (row, chunk): the row's maximum from all its chunks, this
    // chunk's sum rescaled to it (the exponentials in parallel), then per row the
    // sum of its chunks' terms and the logarithm
    __shared__ double s_part[kKMax * 16];
    const int S = rws.S;
    if (tid < Rl * S) {
      const int rw = tid / S, c = tid % S;
      const long long rb = ((long long)b * Rl + rw) * S;
      float M = -INFINITY;
      for (int q = 0; q < S; ++q) M = fmaxf(M, rws.row_max[rb + q]);
      const float m = rws.row_max[rb + c];
      s_part[tid] = m == -INFINITY ? 0.0 : rws.row_sum[rb + c] * exp((double)m - (double)M);
      if (c == 0) s_lse[rw] = (double)M;
    }
    __syncthreads();
    if (tid < Rl) {
      double sum = 0.0;
      for (int q = 0; q < S; ++q) sum += s_part[tid * S + q];
      s_lse[tid] += log(sum);
    }
    __syncthreads();
    for (int i = tid; i < Rl * K; i += kSelectThreads) {
      const unsigned long long k0 = s_key[i];
      const float lpv = (float)((double)key_value(k0) - s_lse[i / K]);
      s_key[i] = rank_key(lpv, key_index(k0));
    }
    __syncthreads();
  }
  // the rows into the state (row 0 at layer 0, rows 1 + (layer-1) K + j after)
  const long long rrow = (long long)b * R + (layer == 0 ? 0 : 1 + (long long)(layer - 1) * K);
  for (int i = tid; i < Rl * K; i += kSelectThreads) st.keys[rrow * K + i] = s_key[i];
  if (tid < Rl) st.bad[rrow + tid] = s_bad;
  if (tid >= 64) return;
  // the next frontier, on the first wavefront
  const long long fo = (long long)b * K;
  if (layer == 0) {
    if (tid < K) {
      st.fsc[fo + tid] = key_value(s_key[tid]);
      frontier_tokens[fo + tid] = (int)key_index(s_key[tid]);
      if (frontier_parents) frontier_parents[fo + tid] = -1;
    }
    return;
  }
  constexpr int kPerLane = (KK + 63) / 64;
  unsigned long long key[kPerLane];
  float sc[kPerLane];
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const int o = tid + 64 * i;
    key[i] = 0ull;
    sc[i] = 0.0f;
    if (o < KK) {
      sc[i] = __fadd_rn(key_value(s_key[o]), s_fsc[o / K]);
      key[i] = rank_key(sc[i], (uint32_t)o);
      s_ck[o] = key[i];
    }
  }
  if (tid < 2) s_ck[KK + tid] = 0ull;  // pads the last pair read
  wave_sync();
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const int o = tid + 64 * i;
    if (o < KK) {
      int rk = 0;
      for (int q = 0; q < KK; q += 2) {
        const u64x2 x = *reinterpret_cast<const u64x2*>(s_ck + q);
        rk += (x[0] > key[i]) + (x[1] > key[i]);
      }
      if (rk < K) {
        st.fsc[fo + rk] = sc[i];
        frontier_tokens[fo + rk] = (int)key_index(s_key[o]);
        if (frontier_parents) frontier_parents[fo + rk] = o / K;
      }
    }
  }
}

// Vocabulary chunks per row in a layer call: one layer has at most K rows per
// request, so rows are cut finer than in the batch build (chunks of ~4096
// entries, up to 16) to put more workgroups on the chip; with raw logits each
// chunk also evaluates its float64 exponentials, ~16 per thread at 4096.
inline int pick_split_layer(int V, int K) {
  int S = (V + 4095) / 4096;
  if (S > 16) S = 16;
  const long long rk = (long long)K * K;
  const long long cap = (kStageKeys - 2 * rk) / rk;
  if (S > cap) S = (int)cap;
  return S < 1 ? 1 : S;
}

size_t layer_state_bytes(int B, int V, int K, int D, int* S_out) {
  const long long R = 1 + (long long)D * K;
  const int S = pick_split_layer(V, K);
  if (S_out) *S_out = S;
  const long long rows = (long long)B * K;  // row-top-K scratch: one layer's rows
  size_t n = (size_t)B * R * K * 8 + (size_t)B * R * 4 + (size_t)B * K * 4;
  n = (n + 255) & ~(size_t)255;
  n += build_ws_bytes(rows, K, S);
  n = (n + 255) & ~(size_t)255;
  n += (size_t)rows * S * (4 + 8) + 256;
  return n;
}

// carve the state: [keys | bad | fsc] then the row-top-K scratch and its log-sum-exp parts
void layer_state(void* base, int B, int V, int K, int D, LayerState* st, BuildWs* rws) {
  const long long R = 1 + (long long)D * K;
  int S = 1;
  layer_state_bytes(B, V, K, D, &S);
  unsigned char* p = reinterpret_cast<unsigned char*>(base);
  st->keys = reinterpret_cast<unsigned long long*>(p);
  st->bad = reinterpret_cast<int*>(p + (size_t)B * R * K * 8);
  st->fsc = reinterpret_cast<float*>(p + (size_t)B * R * K * 8 + (size_t)B * R * 4);
  size_t off = (size_t)B * R * K * 8 + (size_t)B * R * 4 + (size_t)B * K * 4;
  off = (off + 255) & ~(size_t)255;
  const long long rows = (long long)B * K;
  *rws = build_ws(p + off, rows, K, S);
  off += build_ws_bytes(rows, K, S);
  off = (off + 255) & ~(size_t)255;
  rws->row_sum = reinterpret_cast<double*>(p + off);
  rws->row_max = reinterpret_cast<float*>(p + off + (size_t)rows * S * 8);
}

}  // namespace
}  // namespace tv

extern "C" size_t tree_build_workspace_bytes(int mode, int B, int V, int K, int rows_per_req) {
  (void)mode;
  (void)V;
  if (B <= 0 || K <= 0 || rows_per_req <= 0) return 0;
  return tv::build_ws_bytes((long long)B * rows_per_req, K, tv::pick_split(V, K, rows_per_req));
}

namespace {
int build_impl(int mode, int B, int V, int K, int D, int total_tokens, const int* branching, int n_levels,
               const float* logprobs, int rows_per_req, const int* root_token, int T_max, int* draft_tokens,
               int* parents, int* tree_size, float* node_score, int* status, void* workspace, size_t ws_bytes,
               const tv::MetaOut* meta, void* stream) {
  using namespace tv;
  if (B <= 0 || V <= 0 || T_max <= 0 || rows_per_req <= 0) return TV_EINVAL;
  if (!logprobs || !root_token || !draft_tokens || !parents || !tree_size || !status) return TV_EINVAL;
  if (T_max > kTMaxLimit) return TV_EUNSUPPORTED;
  tv::Branching br{};
  if (mode == TV_MODE_DYNAMIC) {
    if (K < 1 || D < 0 || D > 64 || total_tokens < 0) return TV_EINVAL;
    if (K > kKMax) return TV_EUNSUPPORTED;
    if (K > V) return TV_EINVAL;
    const long long C = (long long)K + (long long)D * K * K;
    if (C > kMaxCand) return TV_EUNSUPPORTED;
    if (total_tokens > C || total_tokens + 1 > T_max) return TV_EINVAL;
    if (rows_per_req != 1 + D * K) return TV_EINVAL;
  } else if (mode == TV_MODE_STATIC) {
    if (!branching || n_levels < 1 || n_levels > kMaxLevels - 1) return TV_EINVAL;
    long long width = 1, T = 1, expanded = 0;
    int wmax = 0;
    for (int l = 0; l < n_levels; ++l) {
      if (branching[l] < 1) return TV_EINVAL;
      if (branching[l] > kKMax) return TV_EUNSUPPORTED;
      expanded += width;
      width *= branching[l];
      T += width;
      if (T > T_max) return TV_EINVAL;
      wmax = branching[l] > wmax ? branching[l] : wmax;
      br.w[l] = branching[l];
    }
    br.n = n_levels;
    if (rows_per_req != expanded) return TV_EINVAL;
    if (wmax > V) return TV_EINVAL;
    K = wmax;
  } else {
    return TV_EINVAL;
  }
  const size_t need = tree_build_workspace_bytes(mode, B, V, K, rows_per_req);
  if (!workspace || ws_bytes < need) return TV_EWORKSPACE;

  const long long rows_total = (long long)B * rows_per_req;
  if (rows_total > 0x7FFFFFFFll) return TV_EUNSUPPORTED;
  const int S = pick_split(V, K, rows_per_req);
  if (rows_total * S > 0x7FFFFFFFll) return TV_EUNSUPPORTED;
  const BuildWs ws = build_ws(workspace, rows_total, K, S);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t stage = S > 1 ? (size_t)rows_per_req * S * K * 8 : 0;  // chunk lists merged in the select kernel

  const int vec4 = (V % 4 == 0) && ((reinterpret_cast<uintptr_t>(logprobs) & 15) == 0);
  if (rows_total * S <= 256) {
    hipLaunchKernelGGL((k_row_topk<false, kTopkWideThreads>), dim3((unsigned)(rows_total * S)), dim3(kTopkWideThreads),
                       0, s, logprobs, V, K, vec4, ws);
  } else {
    hipLaunchKernelGGL(k_row_topk<false>, dim3((unsigned)(rows_total * S)), dim3(kTopkThreads), 0, s, logprobs, V, K,
                       vec4, ws);
  }
  TV_CHECK_LAUNCH();

  if (mode == TV_MODE_DYNAMIC) {
    const int C = rows_per_req * K;
    const size_t smem = (size_t)C * 16 + stage;
    switch (K) {
#define TV_SELECT_CASE(k)                                                                                          \
  case k:                                                                                                          \
    if (meta)                                                                                                      \
      hipLaunchKernelGGL((k_tree_select_dynamic<k, true>), dim3(B), dim3(kSelectThreads), smem, s, ws,           \
                         rows_per_req, D, total_tokens, root_token, T_max, draft_tokens, parents, tree_size,      \
                         node_score, status, *meta);                                                               \
    else                                                                                                           \
      hipLaunchKernelGGL((k_tree_select_dynamic<k, false>), dim3(B), dim3(kSelectThreads), smem, s, ws,          \
                         rows_per_req, D, total_tokens, root_token, T_max, draft_tokens, parents, tree_size,      \
                         node_score, status, MetaOut{});                                                           \
    break;
      TV_SELECT_CASE(1) TV_SELECT_CASE(2) TV_SELECT_CASE(3) TV_SELECT_CASE(4) TV_SELECT_CASE(5) TV_SELECT_CASE(6)
      TV_SELECT_CASE(7) TV_SELECT_CASE(8) TV_SELECT_CASE(9) TV_SELECT_CASE(10) TV_SELECT_CASE(11)
      TV_SELECT_CASE(12) TV_SELECT_CASE(13) TV_SELECT_CASE(14) TV_SELECT_CASE(15) TV_SELECT_CASE(16)
#undef TV_SELECT_CASE
      default: return TV_EUNSUPPORTED;
    }
  } else {
    const size_t smem = (size_t)rows_per_req * K * 8 + stage;
    if (meta)
      hipLaunchKernelGGL(k_tree_select_static<true>, dim3(B), dim3(kSelectThreads), smem, s, ws, rows_per_req, K,
                         br, root_token, T_max, draft_tokens, parents, tree_size, node_score, status, *meta);
    else
      hipLaunchKernelGGL(k_tree_select_static<false>, dim3(B), dim3(kSelectThreads), smem, s, ws, rows_per_req, K,
                         br, root_token, T_max, draft_tokens, parents, tree_size, node_score, status, MetaOut{});
  }
  TV_CHECK_LAUNCH();
  return TV_OK;
}
}  // namespace

extern "C" int tree_build(int mode, int B, int V, int K, int D, int total_tokens, const int* branching,
                          int n_levels, const float* logprobs, int rows_per_req, const int* root_token, int T_max,
                          int* draft_tokens, int* parents, int* tree_size, float* node_score, int* status,
                          void* workspace, size_t ws_bytes, void* stream) {
  return build_impl(mode, B, V, K, D, total_tokens, branching, n_levels, logprobs, rows_per_req, root_token, T_max,
                    draft_tokens, parents, tree_size, node_score, status, workspace, ws_bytes, nullptr, stream);
}

extern "C" int tree_build_meta(int mode, int B, int V, int K, int D, int total_tokens, const int* branching,
                               int n_levels, const float* logprobs, int rows_per_req, const int* root_token,
                               int T_max, int* draft_tokens, int* parents, int* tree_size, float* node_score,
                               int* status, void* workspace, size_t ws_bytes, int dcap, const int* prefix_len,
                               uint32_t* tree_mask, int* tree_position_ids, int* positions, int* retrieve_indices,
                               int* leaf_count, int* first_child, int* next_sibling, void* stream) {
  // the checks of tree_mask_positions (those of tree_build follow)
  if (B <= 0 || T_max <= 0 || dcap < 0 || dcap >= T_max) return TV_EINVAL;
  if (T_max > tv::kTMaxLimit) return TV_EUNSUPPORTED;
  if (!prefix_len || !tree_mask || !tree_position_ids || !positions || !retrieve_indices || !leaf_count)
    return TV_EINVAL;
  if (B > 2147483647 / 64) return TV_EINVAL;
  const tv::MetaOut mo{dcap, (T_max + 31) / 32, prefix_len, tree_mask, tree_position_ids, positions,
                       retrieve_indices, leaf_count, first_child, next_sibling};
  return build_impl(mode, B, V, K, D, total_tokens, branching, n_levels, logprobs, rows_per_req, root_token, T_max,
                    draft_tokens, parents, tree_size, node_score, status, workspace, ws_bytes, &mo, stream);
}

extern "C" size_t tree_build_layer_workspace_bytes(int B, int V, int K, int D) {
  if (B <= 0 || V <= 0 || K <= 0 || K > tv::kKMax || D < 0 || D > 64) return 0;
  return tv::layer_state_bytes(B, V, K, D, nullptr);
}

namespace {
// the dynamic-mode checks shared by the layer calls
int layer_checks(int B, int V, int K, int D) {
  using namespace tv;
  if (B <= 0 || V <= 0 || K < 1 || D < 0 || D > 64) return TV_EINVAL;
  if (K > kKMax) return TV_EUNSUPPORTED;
  if (K > V) return TV_EINVAL;
  const long long C = (long long)K + (long long)D * K * K;
  if (C > kMaxCand) return TV_EUNSUPPORTED;
  if ((long long)B * K * tv::pick_split_layer(V, K) > 0x7FFFFFFFll) return TV_EUNSUPPORTED;
  return TV_OK;
}
}  // namespace

extern "C" int tree_build_layer(int layer, int B, int V, int K, int D, const float* rows, int rows_are_logits,
                                void* state, size_t state_bytes, int* frontier_tokens, int* frontier_parents,
                                void* stream) {
  using namespace tv;
  const int rc = layer_checks(B, V, K, D);
  if (rc != TV_OK) return rc;
  if (layer < 0 || layer > D) return TV_EINVAL;
  if (!rows || !state || !frontier_tokens) return TV_EINVAL;
  if (state_bytes < layer_state_bytes(B, V, K, D, nullptr)) return TV_EWORKSPACE;
  LayerState st{};
  BuildWs rws{};
  layer_state(state, B, V, K, D, &st, &rws);
  const int Rl = layer == 0 ? 1 : K;
  const long long rows_total = (long long)B * Rl;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int vec4 = (V % 4 == 0) && ((reinterpret_cast<uintptr_t>(rows) & 15) == 0);
  if (rows_are_logits)
    hipLaunchKernelGGL(k_row_topk<true>, dim3((unsigned)(rows_total * rws.S)), dim3(kTopkThreads), 0, s, rows, V, K,
                       vec4, rws);
  else
    hipLaunchKernelGGL(k_row_topk<false>, dim3((unsigned)(rows_total * rws.S)), dim3(kTopkThreads), 0, s, rows, V,
                       K, vec4, rws);
  TV_CHECK_LAUNCH();
  const size_t stage = rws.S > 1 ? (size_t)Rl * rws.S * K * 8 : 0;
  const int R = 1 + D * K;
  switch (K) {
#define TV_LAYER_CASE(k)                                                                                         \
  case k:                                                                                                        \
    if (rows_are_logits)                                                                                         \
      hipLaunchKernelGGL((k_build_layer<k, true>), dim3(B), dim3(kSelectThreads), stage, s, rws, layer, R, st,   \
                         frontier_tokens, frontier_parents);                                                     \
    else                                                                                                         \
      hipLaunchKernelGGL((k_build_layer<k, false>), dim3(B), dim3(kSelectThreads), stage, s, rws, layer, R, st,  \
                         frontier_tokens, frontier_parents);                                                     \
    break;
    TV_LAYER_CASE(1) TV_LAYER_CASE(2) TV_LAYER_CASE(3) TV_LAYER_CASE(4) TV_LAYER_CASE(5) TV_LAYER_CASE(6)
    TV_LAYER_CASE(7) TV_LAYER_CASE(8) TV_LAYER_CASE(9) TV_LAYER_CASE(10) TV_LAYER_CASE(11) TV_LAYER_CASE(12)
    TV_LAYER_CASE(13) TV_LAYER_CASE(14) TV_LAYER_CASE(15) TV_LAYER_CASE(16)
#undef TV_LAYER_CASE
    default: return TV_EUNSUPPORTED;
  }
  TV_CHECK_LAUNCH();
  return TV_OK;
}

extern "C" int tree_build_finish(int B, int V, int K, int D, int total_tokens, const int* root_token, int T_max,
                                 const void* state, size_t state_bytes, int* draft_tokens, int* parents,
                                 int* tree_size, float* node_score, int* status, int dcap, const int* prefix_len,
                                 uint32_t* tree_mask, int* tree_position_ids, int* positions, int* retrieve_indices,
                                 int* leaf_count, int* first_child, int* next_sibling, void* stream) {
  using namespace tv;
  const int rc = layer_checks(B, V, K, D);
  if (rc != TV_OK) return rc;
  if (T_max <= 0) return TV_EINVAL;
  if (T_max > kTMaxLimit) return TV_EUNSUPPORTED;
  const long long C = (long long)K + (long long)D * K * K;
  if (total_tokens < 0 || total_tokens > C || total_tokens + 1 > T_max) return TV_EINVAL;
  if (!root_token || !state || !draft_tokens || !parents || !tree_size || !status) return TV_EINVAL;
  if (state_bytes < layer_state_bytes(B, V, K, D, nullptr)) return TV_EWORKSPACE;
  MetaOut mo{};
  const bool meta = prefix_len != nullptr;
  if (meta) {  // the checks of tree_mask_positions
    if (dcap < 0 || dcap >= T_max) return TV_EINVAL;
    if (!tree_mask || !tree_position_ids || !positions || !retrieve_indices || !leaf_count) return TV_EINVAL;
    if (B > 2147483647 / 64) return TV_EINVAL;
    mo = MetaOut{dcap, (T_max + 31) / 32, prefix_len, tree_mask, tree_position_ids, positions, retrieve_indices,
                 leaf_count, first_child, next_sibling};
  }
  LayerState st{};
  BuildWs rws{};
  layer_state(const_cast<void*>(state), B, V, K, D, &st, &rws);
  BuildWs ws{};
  ws.row_keys = st.keys;
  ws.row_bad = st.bad;
  ws.S = 1;
  const int R = 1 + D * K;
  const size_t smem = (size_t)R * K * 16;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  switch (K) {
#define TV_FINISH_CASE(k)                                                                                         \
  case k:                                                                                                         \
    if (meta)                                                                                                     \
      hipLaunchKernelGGL((k_tree_select_dynamic<k, true>), dim3(B), dim3(kSelectThreads), smem, s, ws, R, D,      \
                         total_tokens, root_token, T_max, draft_tokens, parents, tree_size, node_score, status, mo); \
    else                                                                                                          \
      hipLaunchKernelGGL((k_tree_select_dynamic<k, false>), dim3(B), dim3(kSelectThreads), smem, s, ws, R, D,     \
                         total_tokens, root_token, T_max, draft_tokens, parents, tree_size, node_score, status, mo); \
    break;
    TV_FINISH_CASE(1) TV_FINISH_CASE(2) TV_FINISH_CASE(3) TV_FINISH_CASE(4) TV_FINISH_CASE(5) TV_FINISH_CASE(6)
    TV_FINISH_CASE(7) TV_FINISH_CASE(8) TV_FINISH_CASE(9) TV_FINISH_CASE(10) TV_FINISH_CASE(11) TV_FINISH_CASE(12)
    TV_FINISH_CASE(13) TV_FINISH_CASE(14) TV_FINISH_CASE(15) TV_FINISH_CASE(16)
#undef TV_FINISH_CASE
    default: return TV_EUNSUPPORTED;
  }
  TV_CHECK_LAUNCH();
  return TV_OK;
}
