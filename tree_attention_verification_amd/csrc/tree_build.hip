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
//   k_row_topk    one workgroup per (draft row, vocabulary chunk): streams the
//                 row once with 16-byte loads (HBM-bound scan), keeps a per-thread
//                 sorted top-K in registers, merges the 256 lists with K rounds
//                 of a workgroup argmax, writes the chunk's sorted top-K keys.
//   k_tree_select one workgroup per request: merges the chunk lists of every row
//                 (lane groups, one lane per chunk), then runs the D dependent
//                 K*K rounds and the final top-total_tokens selection (radix
//                 select on unique 64-bit rank keys) entirely in LDS, and writes
//                 the numbered tree.  Static mode builds level by level instead.
#include "tv_common.h"

namespace tv {
namespace {

constexpr int kTopkThreads = 256;
constexpr int kSelectThreads = 256;
constexpr int kMaxChunks = 8;
constexpr int kMaxCand = 3072;   // LDS: 16 B per candidate
constexpr int kMaxLevels = 64;

struct Branching {
  int n;
  int w[kMaxLevels];
};

// Workspace layout (rows = B * rows_per_req): each (row, chunk) workgroup of K1
// writes its sorted top-K rank keys and a bad-value flag; K2 merges the chunks.
struct BuildWs {
  unsigned long long* chunk_keys;  // [rows][n_chunks][K]
  int* chunk_bad;                  // [rows][n_chunks]
  int n_chunks;
};

__host__ __device__ inline size_t build_ws_bytes(long long rows, int K) {
  return (size_t)rows * ((size_t)kMaxChunks * K * 8 + kMaxChunks * 4) + 256;
}

__host__ __device__ inline BuildWs build_ws(void* base, long long rows, int K, int n_chunks) {
  BuildWs w;
  unsigned char* p = reinterpret_cast<unsigned char*>(base);
  w.chunk_keys = reinterpret_cast<unsigned long long*>(p);
  p += (size_t)rows * n_chunks * K * 8;
  w.chunk_bad = reinterpret_cast<int*>(p);
  w.n_chunks = n_chunks;
  return w;
}

// Merge the n_chunks sorted chunk lists of every row of request b into the row's
// top-K rank keys, written to s_key[row*K + r] (r = rank in the row).  A group of
// n_chunks lanes (power of two <= 8) handles a row: each lane holds one chunk's
// list in registers and K rounds of a group argmax pop the winners.
__device__ void merge_rows(const BuildWs& ws, long long row_base, int R, int K, unsigned long long* s_key,
                           int* s_bad) {
  const int tid = threadIdx.x;
  const int G = ws.n_chunks;
  const int rows_per_pass = kSelectThreads / G;
  for (int row0 = 0; row0 < R; row0 += rows_per_pass) {
    const int row = row0 + tid / G;
    const int c = tid % G;
    unsigned long long l[kKMax];
#pragma unroll
    for (int i = 0; i < kKMax; ++i) l[i] = 0ull;
    if (row < R) {
      const unsigned long long* src = ws.chunk_keys + ((row_base + row) * G + c) * K;
#pragma unroll
      for (int i = 0; i < kKMax; ++i)
        if (i < K) l[i] = src[i];
      if (ws.chunk_bad[(row_base + row) * G + c]) *s_bad = 1;
    }
    for (int k = 0; k < K; ++k) {
      const unsigned long long best = G == 8 ? group_max_u64<8>(l[0])
                                      : G == 4 ? group_max_u64<4>(l[0])
                                      : G == 2 ? group_max_u64<2>(l[0]) : l[0];
      if (row < R && c == 0) s_key[row * K + k] = best;
      if (l[0] == best) {
#pragma unroll
        for (int i = 0; i < kKMax - 1; ++i) l[i] = l[i + 1];
        l[kKMax - 1] = 0ull;
      }
    }
  }
}

// --------------------------------------------------------------------------
// K1: per-(row, chunk) top-K, then the row's top-K by the last chunk to finish.
// --------------------------------------------------------------------------
template <int K>
__device__ __forceinline__ void list_insert(uint32_t (&lv)[K], uint32_t (&li)[K], uint32_t key, uint32_t idx) {
  // lv is sorted descending; the caller guarantees key > lv[K-1].  An equal key
  // never displaces an earlier (lower-index) entry because indices increase.
#pragma unroll
  for (int i = K - 1; i >= 1; --i) {
    const bool shift = key > lv[i - 1];
    const bool here = !shift && key > lv[i];
    lv[i] = shift ? lv[i - 1] : (here ? key : lv[i]);
    li[i] = shift ? li[i - 1] : (here ? idx : li[i]);
  }
  if (key > lv[0]) {
    lv[0] = key;
    li[0] = idx;
  }
}

// Rank-count selection inside one wavefront: n (<= 64) unique non-zero keys in
// LDS (zeros pad), the K largest are written in order to out[0..K).  Each lane
// holds one key; the others are broadcast through scalar registers.
__device__ __forceinline__ void wave_select_sorted(const unsigned long long* keys, int n, int K,
                                                   unsigned long long* out, int lane) {
  const unsigned long long my = lane < n ? keys[lane] : 0ull;
  int rank = 0;
  for (int o = 0; o < n; ++o) rank += readlane_u64(my, o) > my;
  if (lane < K) out[lane] = 0ull;
  __builtin_amdgcn_wave_barrier();
  if (lane < n && my != 0ull && rank < K) out[rank] = my;
  __builtin_amdgcn_wave_barrier();
}

template <int K>
__global__ __launch_bounds__(kTopkThreads) void k_row_topk(const float* __restrict__ lp, int V, int chunk_len,
                                                           int vec4, BuildWs ws) {
  const int chunk = blockIdx.x, n_chunks = gridDim.x;
  const long long row = blockIdx.y;
  const float* r = lp + row * (long long)V;
  const int begin = chunk * chunk_len;
  const int end = min(V, begin + chunk_len);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  uint32_t lv[K], li[K];
#pragma unroll
  for (int i = 0; i < K; ++i) {
    lv[i] = 0u;  // below every real key (order_key(-inf) = 0x007FFFFF)
    li[i] = 0xFFFFFFFFu;
  }
  bool bad = false;
  auto consider = [&](float v, int idx) {
    bad |= !(v <= 0.0f);  // NaN or positive
    const uint32_t key = order_key(v);
    if (key > lv[K - 1]) list_insert<K>(lv, li, key, (uint32_t)idx);
  };
  if (vec4) {
    // 16-byte loads (V % 4 == 0 and a 16-byte aligned base; chunk_len is a
    // multiple of 4, so every float4 is aligned).
    typedef float f4 __attribute__((ext_vector_type(4)));
    const f4* r4 = reinterpret_cast<const f4*>(r);
    for (int e = begin + 4 * tid; e < end; e += 4 * kTopkThreads) {
      const f4 x = __builtin_nontemporal_load(r4 + (e >> 2));
      consider(x[0], e);
      consider(x[1], e + 1);
      consider(x[2], e + 2);
      consider(x[3], e + 3);
    }
  } else {
    for (int e = begin + tid; e < end; e += kTopkThreads) consider(r[e], e);
  }

  // wavefront merge without barriers: K rounds of a wave argmax over list heads,
  // the round-k winner is kept by lane k
  unsigned long long mine = 0ull;
  for (int k = 0; k < K; ++k) {
    const unsigned long long head = lv[0] ? (((unsigned long long)lv[0] << 32) | (0xFFFFFFFFu - li[0])) : 0ull;
    const unsigned long long best = wave_max_u64(head);
    if (head == best && head != 0ull) {
#pragma unroll
      for (int i = 0; i < K - 1; ++i) {
        lv[i] = lv[i + 1];
        li[i] = li[i + 1];
      }
      lv[K - 1] = 0u;
      li[K - 1] = 0xFFFFFFFFu;
    }
    if (lane == k) mine = best;
  }
  __shared__ unsigned long long s_w[4 * kKMax];
  __shared__ unsigned long long s_out[kKMax];
  __shared__ int s_bad;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  if (lane < K) s_w[wave * K + lane] = mine;
  if (__ballot(bad) && lane == 0) atomicOr(&s_bad, 1);
  __syncthreads();
  if (wave == 0) wave_select_sorted(s_w, 4 * K, K, s_out, lane);
  __syncthreads();
  if (tid < K) ws.chunk_keys[(row * n_chunks + chunk) * K + tid] = s_out[tid];
  if (tid == 0) ws.chunk_bad[row * n_chunks + chunk] = s_bad;
}

// --------------------------------------------------------------------------
// K2 helpers
// --------------------------------------------------------------------------
// Block-wide exclusive scan of one int per thread; returns the exclusive prefix
// and writes the total to *total.
__device__ int block_excl_scan(int v, int* s_tmp, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
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
      int incl = mine;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        int y = __shfl_up(incl, o, 64);
        if (tid >= o) incl += y;
      }
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

__global__ __launch_bounds__(kSelectThreads) void k_tree_select_dynamic(
    BuildWs ws, int R, int K, int D, int total_tokens, const int* __restrict__ root_token, int T_max,
    int* __restrict__ draft_tokens, int* __restrict__ parents, int* __restrict__ tree_size,
    float* __restrict__ node_score, int* __restrict__ status) {
  extern __shared__ unsigned char smem[];
  const int C = R * K;  // = K + D*K*K: candidate id == row*K + rank
  unsigned long long* s_key = reinterpret_cast<unsigned long long*>(smem);
  float* s_sc = reinterpret_cast<float*>(s_key + C);
  short* s_par = reinterpret_cast<short*>(s_sc + C);
  short* s_node = s_par + C;
  __shared__ int s_hist[256];
  __shared__ unsigned long long s_bcast[4], s_tmp64[kSelectThreads / 64];
  __shared__ int s_front[2][kKMax];
  __shared__ float s_fsc[2][kKMax];
  __shared__ unsigned long long s_lkey[256];
  __shared__ int s_rank[256];
  __shared__ int s_tmp[kSelectThreads / 64];
  __shared__ int s_bad;

  const int b = blockIdx.x, tid = threadIdx.x;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  merge_rows(ws, (long long)b * R, R, K, s_key, &s_bad);
  __syncthreads();
  for (int id = tid; id < C; id += kSelectThreads) {
    s_sc[id] = key_value(s_key[id]);
    s_par[id] = -1;
  }
  __syncthreads();
  if (tid < K) {
    s_front[0][tid] = tid;
    s_fsc[0][tid] = s_sc[tid];
  }
  __syncthreads();

  // D dependent rounds of K*K cumulative scores and a frontier top-K
  const int KK = K * K;
  const int split = KK <= 64 ? 4 : (KK <= 128 ? 2 : 1);
  for (int l = 1; l <= D; ++l) {
    const int cur = (l - 1) & 1, nxt = l & 1;
    const int base = K + (l - 1) * KK;
    for (int q = tid; q < KK; q += kSelectThreads) {
      const int j = q / K;
      const float sc = __fadd_rn(s_sc[base + q], s_fsc[cur][j]);
      s_sc[base + q] = sc;
      s_par[base + q] = (short)s_front[cur][j];
      s_lkey[q] = rank_key(sc, (uint32_t)q);
      s_rank[q] = 0;
    }
    __syncthreads();
    for (int t = tid; t < KK * split; t += kSelectThreads) {
      const int q = t % KK, part = t / KK;
      const unsigned long long mine = s_lkey[q];
      const int o0 = part * (KK / split), o1 = part == split - 1 ? KK : o0 + KK / split;
      int cnt = 0;
      int o = o0;
      for (; o + 16 <= o1; o += 16) {  // sixteen keys per batch of LDS reads
        unsigned long long x[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) x[u] = s_lkey[o + u];
#pragma unroll
        for (int u = 0; u < 16; ++u) cnt += x[u] > mine;
      }
      for (; o < o1; ++o) cnt += s_lkey[o] > mine;
      if (split == 1) s_rank[q] = cnt;
      else atomicAdd(&s_rank[q], cnt);
    }
    __syncthreads();
    for (int q = tid; q < KK; q += kSelectThreads) {
      const int rk2 = s_rank[q];
      if (rk2 < K) {
        s_front[nxt][rk2] = base + q;
        s_fsc[nxt][rk2] = s_sc[base + q];
      }
    }
    __syncthreads();
  }

  // final: keep the total_tokens best candidates, number them by ascending id
  const unsigned long long tau = radix_select_threshold(C, total_tokens, s_sc, s_hist, s_bcast, s_tmp64);
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
        draft_tokens[ob + n] = (int)key_index(s_key[id]);
        parents[ob + n] = s_par[id] < 0 ? 0 : s_node[s_par[id]];
        if (node_score) node_score[ob + n] = s_sc[id];
      }
    }
  }
  if (tid == 0) {
    tree_size[b] = T;
    status[b] = ok ? TV_ST_OK : TV_ST_LOGPROB;
  }
}

__global__ __launch_bounds__(kSelectThreads) void k_tree_select_static(
    BuildWs ws, int R, int K, Branching br, const int* __restrict__ root_token, int T_max,
    int* __restrict__ draft_tokens, int* __restrict__ parents, int* __restrict__ tree_size,
    float* __restrict__ node_score, int* __restrict__ status) {
  extern __shared__ unsigned char smem[];
  unsigned long long* rk = reinterpret_cast<unsigned long long*>(smem);
  __shared__ int t_tok[kTMaxLimit], t_par[kTMaxLimit];
  __shared__ float t_sc[kTMaxLimit];
  __shared__ int s_T, s_bad;
  const int b = blockIdx.x, tid = threadIdx.x;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  merge_rows(ws, (long long)b * R, R, K, rk, &s_bad);
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
  if (tid == 0) {
    tree_size[b] = T;
    status[b] = ok ? TV_ST_OK : TV_ST_LOGPROB;
  }
}

int pick_chunks(long long rows_total, int V, int K) {
  int n = 1;
  while (n < kMaxChunks && rows_total * n < 256 && (V / (n * 2)) >= 4 * kTopkThreads && V / (n * 2) >= K) n *= 2;
  return n;
}

template <int K>
void launch_topk(dim3 grid, const float* lp, int V, int chunk_len, int vec4, BuildWs ws, hipStream_t s) {
  hipLaunchKernelGGL(k_row_topk<K>, grid, dim3(kTopkThreads), 0, s, lp, V, chunk_len, vec4, ws);
}

void launch_topk_any(int K, dim3 grid, const float* lp, int V, int chunk_len, int vec4, BuildWs ws,
                     hipStream_t s) {
  switch (K) {
#define TV_TOPK_CASE(k) \
  case k:               \
    launch_topk<k>(grid, lp, V, chunk_len, vec4, ws, s); break;
    TV_TOPK_CASE(1) TV_TOPK_CASE(2) TV_TOPK_CASE(3) TV_TOPK_CASE(4) TV_TOPK_CASE(5) TV_TOPK_CASE(6)
    TV_TOPK_CASE(7) TV_TOPK_CASE(8) TV_TOPK_CASE(9) TV_TOPK_CASE(10) TV_TOPK_CASE(11) TV_TOPK_CASE(12)
    TV_TOPK_CASE(13) TV_TOPK_CASE(14) TV_TOPK_CASE(15) TV_TOPK_CASE(16)
#undef TV_TOPK_CASE
    default: break;
  }
}

}  // namespace
}  // namespace tv

extern "C" size_t tree_build_workspace_bytes(int mode, int B, int V, int K, int rows_per_req) {
  (void)mode;
  (void)V;
  if (B <= 0 || K <= 0 || rows_per_req <= 0) return 0;
  return tv::build_ws_bytes((long long)B * rows_per_req, K);
}

extern "C" int tree_build(int mode, int B, int V, int K, int D, int total_tokens, const int* branching,
                          int n_levels, const float* logprobs, int rows_per_req, const int* root_token, int T_max,
                          int* draft_tokens, int* parents, int* tree_size, float* node_score, int* status,
                          void* workspace, size_t ws_bytes, void* stream) {
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
  if (rows_total > 65535) return TV_EUNSUPPORTED;
  const int n_chunks = pick_chunks(rows_total, V, K);
  int chunk_len = (V + n_chunks - 1) / n_chunks;
  chunk_len = (chunk_len + 3) & ~3;
  const BuildWs ws = build_ws(workspace, rows_total, K, n_chunks);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);

  dim3 grid(n_chunks, (unsigned)rows_total);
  const int vec4 = (V % 4 == 0) && ((reinterpret_cast<uintptr_t>(logprobs) & 15) == 0);
  launch_topk_any(K, grid, logprobs, V, chunk_len, vec4, ws, s);
  TV_CHECK_LAUNCH();

  if (mode == TV_MODE_DYNAMIC) {
    const int C = rows_per_req * K;
    const size_t smem = (size_t)C * 16;
    hipLaunchKernelGGL(k_tree_select_dynamic, dim3(B), dim3(kSelectThreads), smem, s, ws, rows_per_req, K, D,
                       total_tokens, root_token, T_max, draft_tokens, parents, tree_size, node_score, status);
  } else {
    const size_t smem = (size_t)rows_per_req * K * 8;
    hipLaunchKernelGGL(k_tree_select_static, dim3(B), dim3(kSelectThreads), smem, s, ws, rows_per_req, K, br,
                       root_token, T_max, draft_tokens, parents, tree_size, node_score, status);
  }
  TV_CHECK_LAUNCH();
  return TV_OK;
}
