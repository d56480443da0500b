// Sampling-side calls, for gfx950:
//   tree_sampling_probs       target logits -> probabilities under each request's
//                             temperature, top-k, top-p and min-p (the TensorRT-LLM
//                             EAGLE-3 dissection, "non-greedy: rejection from the
//                             target distribution alone": the logits of every tree
//                             node are filtered with the request's parameters
//                             before the rejection step);
//   tree_accept_sample_draft  tree rejection sampling with the drafter's
//                             distribution q (the handbook's exercise "trees when
//                             sampling": children accepted with min(1, p/q), the
//                             target replaced by norm(max(0, p - q)) after a
//                             rejection, q adjusted to how the candidates were
//                             drawn, the correction drawn from the last residual).
//
// Both run one 1024-thread workgroup per row (filter) or per request (walk).
// Every float64 sum is formed in a fixed order (each thread in index order, the
// wavefront by a butterfly, the wavefronts in index order), so results do not
// depend on scheduling.  Products and differences that decide an outcome are
// rounded one at a time (no fused multiply-add), as written.
#include "tv_common.h"

namespace tv {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxV = 262144;  // vocabulary limit (the removed-token bitmap is 32 KB of LDS)

__device__ __forceinline__ double wave_sum_d(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// sum over the workgroup; every thread gets the same value (s: (NT / 64) slots)
template <int NT = kThreads>
__device__ __forceinline__ double block_sum_d(double v, double* s) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum_d(v);
  if (lane == 0) s[wave] = v;
  __syncthreads();
  double t = 0.0;
  for (int w = 0; w < (NT / 64); ++w) t += s[w];
  __syncthreads();
  return t;
}
template <int NT = kThreads>
__device__ __forceinline__ unsigned long long block_sum_u64(unsigned long long v, unsigned long long* s) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if (lane == 0) s[wave] = v;
  __syncthreads();
  unsigned long long t = 0ull;
  for (int w = 0; w < (NT / 64); ++w) t += s[w];
  __syncthreads();
  return t;
}

// Exclusive / inclusive prefix of per-thread values in thread order: lo = sum of
// the earlier threads' values, hi = lo + own.  hi of thread t and lo of thread
// t + 1 are the same stored number.  total = sum of all.
template <typename T, int NT = kThreads>
__device__ __forceinline__ void block_scan(T v, T* s, T& lo, T& hi, T& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  T incl = v;
  for (int o = 1; o < 64; o <<= 1) {
    const T y = __shfl_up(incl, o, 64);
    if (lane >= o) incl = incl + y;
  }
  if (lane == 63) s[wave] = incl;
  __syncthreads();
  T off = T(0), tot = T(0);
  for (int w = 0; w < (NT / 64); ++w) {
    if (w < wave) off = off + s[w];
    tot = tot + s[w];
  }
  __syncthreads();
  const T up = __shfl_up(incl, 1, 64);
  lo = lane > 0 ? off + up : off;
  hi = off + incl;
  total = tot;
}

template <int NT = kThreads>
__device__ __forceinline__ unsigned long long block_max_u64(unsigned long long v, unsigned long long* s) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_max_u64(v);
  if (lane == 0) s[wave] = v;
  __syncthreads();
  unsigned long long t = 0ull;
  for (int w = 0; w < (NT / 64); ++w) t = umax64(t, s[w]);
  __syncthreads();
  return t;
}

// Visits v = threadIdx.x + j NT (j = 0, 1, ...) in increasing v, with the
// loads of NB visits issued together (one memory round trip per NB entries);
// indices past the row are clamped for the load and skipped for the body.
constexpr int kNB = 8;
template <int NT = kThreads, class Load, class Body>
__device__ __forceinline__ void row_pass(int V, Load load, Body body) {
  using T = decltype(load(0));
  for (int base = threadIdx.x; base < V; base += kNB * NT) {
    T x[kNB];
#pragma unroll
    for (int j = 0; j < kNB; ++j) x[j] = load(min(base + j * NT, V - 1));
#pragma unroll
    for (int j = 0; j < kNB; ++j)
      if (base + j * NT < V) body(base + j * NT, x[j]);
  }
}
// The same over a contiguous range [c0, c1), in order; body returns true to stop.
template <class Load, class Body>
__device__ __forceinline__ void range_pass(int c0, int c1, Load load, Body body) {
  using T = decltype(load(0));
  for (int base = c0; base < c1; base += kNB) {
    T x[kNB];
#pragma unroll
    for (int j = 0; j < kNB; ++j) x[j] = load(min(base + j, c1 - 1));
    bool stop = false;
#pragma unroll
    for (int j = 0; j < kNB; ++j)
      if (!stop && base + j < c1) stop = body(base + j, x[j]);
    if (stop) return;
  }
}

// logits: NaN ranks as -inf; order_key canonicalises -0.0
__device__ __forceinline__ float clean_logit(float x) { return x != x ? -INFINITY : x; }
__device__ __forceinline__ uint32_t logit_key(float x) { return order_key(clean_logit(x)); }
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// --------------------------------------------------------------------------
// tree_sampling_probs: one workgroup per (node row, request).
//
// Tokens rank by (logit descending, token ascending).  Weights
// w = fp32(exp((l - l_max) / temperature)) (exactly 1 at the largest logit) are
// written into the output row first and re-read from there.  Each filter keeps
// a prefix of the ranking, described by a cut (key t, token c): token v with key
// k is inside iff k > t or (k == t and v <= c).  The top-k and top-p cuts are
// found by radix selection over the 32-bit order keys, eight bits per pass from
// the top, with exact integer totals (counts for top-k, weights in units of
// 2^-32 for top-p).  Equal keys have equal weights; the cut inside a group of
// equal keys is the n-th of them in token order, found by a scan over contiguous
// token ranges.
// --------------------------------------------------------------------------
// NPT > 0: V <= NPT NT and every thread keeps its NPT (key, weight) pairs in
// registers after the first read; NPT = 0: the row is re-read on every pass.
template <int NT, int NPT>
__global__ __launch_bounds__(NT) void k_sampling_probs(int T_max, int V, const float* __restrict__ logits,
                                                             const int* __restrict__ tree_size,
                                                             const int* __restrict__ status,
                                                             const float* __restrict__ temperature,
                                                             const int* __restrict__ top_k,
                                                             const float* __restrict__ top_p,
                                                             const float* __restrict__ min_p,
                                                             float* __restrict__ probs) {
#pragma clang fp contract(off)
  constexpr int NW = NT / 64;  // wavefronts
  const int i = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  int T = tree_size[b];
  if ((status && status[b] != TV_ST_OK) || T < 1 || T > T_max) T = 1;
  if (i >= T) return;
  const float* lr = logits + ((long long)b * T_max + i) * V;
  float* orow = probs + ((long long)b * T_max + i) * V;
  __shared__ double s_d[NW * 16];
  __shared__ unsigned long long s_u[NW];
  __shared__ unsigned long long s_hist[4096];  // radix bins, ballot entries (V / 64), or the survivor list
  __shared__ unsigned long long s_abv, s_bin;
  __shared__ int s_pick, s_sel, s_cnt;

  // the first-ranked token
  struct KW {
    uint32_t k;
    float w;
  };
  KW reg[NPT > 0 ? NPT : 1];
  auto ld_l = [&](int v) { return lr[v]; };
  unsigned long long best = 0ull;
  if constexpr (NPT > 0) {
    float x[NPT];
#pragma unroll
    for (int j = 0; j < NPT; ++j) x[j] = lr[min(tid + j * NT, V - 1)];
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      reg[j].k = logit_key(x[j]);
      if (tid + j * NT < V) best = umax64(best, rank_key(clean_logit(x[j]), (uint32_t)(tid + j * NT)));
    }
  } else {
    row_pass<NT>(V, ld_l, [&](int v, float x) { best = umax64(best, rank_key(clean_logit(x), (uint32_t)v)); });
  }
  best = block_max_u64<NT>(best, s_u);
  const uint32_t kmax = (uint32_t)(best >> 32);
  const int tok0 = (int)key_index(best);
  const float tau = temperature[b];
  const int kk = top_k[b];
  const float tp = top_p[b], mp = min_p[b];
  // greedy (NaN temperature included); top_k = 1 and top_p <= 0 keep the first token alone
  if (!(tau > 0.0f) || kk == 1 || tp <= 0.0f) {
    for (int v = tid; v < V; v += NT) orow[v] = v == tok0 ? 1.0f : 0.0f;
    return;
  }
  const double dmax = (double)key_float(kmax), dtau = (double)tau;
  auto weight = [&](uint32_t key) -> float {
    return key == kmax ? 1.0f : (float)exp(((double)key_float(key) - dmax) / dtau);
  };
  // (NPT = 0: the weights go to the output row, and each thread re-reads only the
  // weights it wrote: the same v in every row pass)
  auto ld_kw = [&](int v) { return KW{logit_key(lr[v]), orow[v]}; };
  // one pass over the row: body(v, KW) for this thread's tokens in increasing v
  auto pass = [&](auto body) __attribute__((always_inline)) {
    if constexpr (NPT > 0) {
#pragma unroll
      for (int j = 0; j < NPT; ++j)
        if (tid + j * NT < V) body(tid + j * NT, reg[j]);
    } else {
      row_pass<NT>(V, ld_kw, body);
    }
  };
  // weight in units of 2^-32 (w <= 1, so at most 2^32; a row's total stays below 2^51)
  auto fixed = [](float w) { return (unsigned long long)rint((double)w * 4294967296.0); };
  unsigned long long w_all = 0ull;  // this thread's total weight, units of 2^-32
  if constexpr (NPT > 0) {
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      reg[j].w = weight(reg[j].k);
      if (tid + j * NT < V) w_all += fixed(reg[j].w);
    }
  } else {
    row_pass<NT>(V, ld_l, [&](int v, float x) {
      const float w = weight(logit_key(x));
      orow[v] = w;
      w_all += fixed(w);
    });
  }

  const int lane = tid & 63, wave = tid >> 6;
  // The n-th token (token order, n >= 1) with key t inside the top-k cut (tk, ck),
  // in one coalesced pass: for each slice of NT consecutive tokens, every
  // wavefront's ballot of its matching tokens goes to LDS, slice-major, so the
  // entries are in token order; the first wavefront then finds the entry holding
  // the n-th match (64 entries per lane at most, a scan over the lanes) and the
  // bit inside it.  With `mass`, also returns the total weight (units of 2^-32) of
  // the tokens with key > t (all inside the cut, since t >= tk).
  const int nsl = (V + NT - 1) / NT;  // <= 256 slices, <= 4096 entries
  auto nth_with_key = [&](uint32_t t, int n, uint32_t tk, int ck, bool mass, unsigned long long& mass_above) -> int {
    unsigned long long ma = 0ull;
    auto body = [&](int j, uint32_t k, float w) __attribute__((always_inline)) {
      const int v = j * NT + tid;
      const bool f = v < V && k == t && (k > tk || v <= ck);
      const unsigned long long m = __ballot(f);
      if (lane == 0) s_hist[j * NW + wave] = m;
      if (mass && v < V && k > t) ma += fixed(w);
    };
    if (tid == 0) s_pick = V;
    if constexpr (NPT > 0) {
#pragma unroll
      for (int j = 0; j < NPT; ++j)
        if (j < nsl) body(j, reg[j].k, reg[j].w);
    } else {
      for (int j0 = 0; j0 < nsl; j0 += kNB) {
        KW x[kNB];
#pragma unroll
        for (int jj = 0; jj < kNB; ++jj) x[jj] = ld_kw(min((j0 + jj) * NT + tid, V - 1));
#pragma unroll
        for (int jj = 0; jj < kNB; ++jj)
          if (j0 + jj < nsl) body(j0 + jj, x[jj].k, x[jj].w);
      }
    }
    __syncthreads();
    if (wave == 0) {
      const int ne = nsl * NW;
      const int per = (ne + 63) / 64;
      const int e0 = min(ne, lane * per), e1 = min(ne, e0 + per);
      int c = 0;
      for (int e = e0; e < e1; ++e) c += __popcll(s_hist[e]);
      int incl = c;
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      if (incl - c < n && n <= incl) {
        int r = n - (incl - c);
        for (int e = e0; e < e1; ++e) {
          unsigned long long mm = s_hist[e];
          const int pc = __popcll(mm);
          if (r <= pc) {
            for (int q = 1; q < r; ++q) mm &= mm - 1;
            s_pick = (e / NW) * NT + (e % NW) * 64 + (__ffsll((long long)mm) - 1);
            break;
          }
          r -= pc;
        }
      }
    }
    __syncthreads();
    const int res = s_pick;
    __syncthreads();
    mass_above = mass ? block_sum_u64<NT>(ma, s_u) : 0ull;
    return res;
  };

  // ---- radix selection.  Over the tokens with pred, in rank order, each token
  // carrying an integer value (1 to count ranks, its weight in units of 2^-32 for
  // mass), find the key t of the first token at which the running total reaches
  // `target`, and `above` = the total of the tokens with larger keys.  Eight bits
  // of the key per pass from the top: each wavefront adds its tokens' values into
  // its own 256-bin LDS histogram (integer atomics: the totals are exact, so the
  // order of the additions does not matter), then the first wavefront places the
  // target among the bins (four bins per lane, a suffix sum over the lanes).
  // Returns false if the target is never reached.
  auto radix = [&](auto val, auto pred, double target, uint32_t& t_out, unsigned long long& above_out,
                   unsigned long long& bin_out) -> bool {
    unsigned long long bin = 0ull;
    uint32_t prefix = 0u, pmask = 0u;
    unsigned long long above = 0ull;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int e = tid; e < NW * 256; e += NT) s_hist[e] = 0ull;
      __syncthreads();
      pass([&](int v, KW e) {
        if ((e.k & pmask) == prefix && pred(e.k, v)) {
          const unsigned long long x = val(e);
          if (x) atomicAdd(&s_hist[wave * 256 + ((e.k >> shift) & 255u)], x);
        }
      });
      __syncthreads();
      if (wave == 0) {
        unsigned long long m[4], g = 0ull;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          m[j] = 0ull;
          for (int w = 0; w < NW; ++w) m[j] += s_hist[w * 256 + 4 * lane + j];
          g += m[j];
        }
        unsigned long long suf = g;  // total of this lane's bins and every higher lane's
        for (int o = 1; o < 64; o <<= 1) {
          const unsigned long long y = __shfl_down(suf, o, 64);
          if (lane + o < 64) suf += y;
        }
        unsigned long long run = above + (suf - g);
        int cand = -1;
        unsigned long long cabove = 0ull, cbin = 0ull;
        for (int j = 3; j >= 0; --j) {
          if ((double)(run + m[j]) >= target) {
            cand = 4 * lane + j;
            cabove = run;
            cbin = m[j];
            break;
          }
          run += m[j];
        }
        const unsigned long long hit = __ballot(cand >= 0);
        if (lane == 0) s_sel = -1;
        if (hit) {
          const int L = 63 - __builtin_clzll(hit);  // the highest digit that reaches the target
          if (lane == L) {
            s_sel = cand;
            s_abv = cabove;
            s_bin = cbin;
          }
        }
      }
      __syncthreads();
      const int sel = s_sel;
      const unsigned long long nab = s_abv;
      bin = s_bin;
      __syncthreads();
      if (sel < 0) return false;
      prefix |= (uint32_t)sel << shift;
      pmask |= 255u << shift;
      above = nab;
    }
    t_out = prefix;
    above_out = above;
    bin_out = bin;
    return true;
  };
  auto all = [](uint32_t, int) { return true; };
  auto one = [](KW) { return 1ull; };

  // ---- top-k cut (tk, ck); the default keeps everything (every key is > 0)
  uint32_t tk = 0u;
  int ck = V;
  const bool with_p = tp < 1.0f;
  unsigned long long wk = block_sum_u64<NT>(w_all, s_u);  // the survivors' total weight (units of 2^-32)
  if (kk > 1 && kk < V) {
    unsigned long long above = 0ull, bin = 0ull, ma = 0ull;
    radix(one, all, (double)kk, tk, above, bin);  // always reached: kk < V tokens
    const int need = kk - (int)above;
    ck = nth_with_key(tk, need, 0u, V, with_p, ma);
    wk = ma + (unsigned long long)need * fixed(weight(tk));
  }
  auto in_k = [&](uint32_t k, int v) { return k > tk || (k == tk && v <= ck); };

  // ---- top-p cut (tpk, cp) over the top-k survivors
  uint32_t tpk = 0u;
  int cp = V;
  if (with_p && kk > 1 && kk <= NT) {
    // at most NT survivors: gathered into LDS as 64-bit rank keys (key,
    // then token ascending; the order of the appends does not matter), sorted
    // descending by a bitonic network, then one exact prefix sum of their weights
    // in rank order finds the cut
    unsigned long long* s_list = s_hist;  // NT entries
    if (tid == 0) s_cnt = 0;
    __syncthreads();
    pass([&](int v, KW e) {
      if (in_k(e.k, v)) {
        const int pos = atomicAdd(&s_cnt, 1);  // < kk by construction of the cut
        if (pos < NT) s_list[pos] = rank_key(key_float(e.k), (uint32_t)v);
      }
    });
    __syncthreads();
    const int n = min(s_cnt, NT);  // == kk
    if (tid >= n) s_list[tid] = 0ull;
    __syncthreads();
    for (int k2 = 2; k2 <= NT; k2 <<= 1) {
      for (int j = k2 >> 1; j > 0; j >>= 1) {
        const int ixj = tid ^ j;
        if (ixj > tid) {
          const unsigned long long a = s_list[tid], c = s_list[ixj];
          if (((tid & k2) == 0) == (a < c)) {
            s_list[tid] = c;
            s_list[ixj] = a;
          }
        }
        __syncthreads();
      }
    }
    const unsigned long long mine = s_list[tid];
    const unsigned long long x = tid < n ? fixed(weight((uint32_t)(mine >> 32))) : 0ull;
    unsigned long long lo, hi, tot;
    block_scan<unsigned long long, NT>(x, s_u, lo, hi, tot);
    const double target = (double)tp * (double)tot;
    if (tid == 0) s_pick = n;
    __syncthreads();
    if (tid < n && (double)hi >= target) atomicMin(&s_pick, tid);
    __syncthreads();
    const int cut = s_pick;  // the last kept rank
    if (cut < n) {
      const unsigned long long kc = s_list[cut];
      tpk = (uint32_t)(kc >> 32);
      cp = (int)key_index(kc);
    }
    __syncthreads();
  } else if (with_p) {
    const double target = (double)tp * (double)wk;
    unsigned long long above = 0ull, bin = 0ull, unused = 0ull;
    if (radix([&](KW e) { return fixed(e.w); }, in_k, target, tpk, above, bin)) {
      // tokens with key tpk among the survivors, each of the same weight ct (so the
      // last bin holds na ct), join in token order until the running total reaches
      // the target
      const unsigned long long ct = fixed(weight(tpk));
      const int na = (int)(bin / ct);
      int n = 1;
      while ((double)(above + (unsigned long long)n * ct) < target && n < na) ++n;
      cp = nth_with_key(tpk, n, tk, ck, false, unused);
    } else {
      tpk = 0u;  // never reached: every survivor stays
    }
  }

  // ---- min-p, the kept total and the output
  auto keep = [&](uint32_t k, int v, float w) {
    return in_k(k, v) && (k > tpk || (k == tpk && v <= cp)) && (!(mp > 0.0f) || w >= mp || v == tok0);
  };
  double wsum = 0.0;
  pass([&](int v, KW e) {
    if (keep(e.k, v, e.w)) wsum += (double)e.w;
  });
  const double W = block_sum_d<NT>(wsum, s_d);
  pass([&](int v, KW e) { orow[v] = keep(e.k, v, e.w) ? (float)((double)e.w / W) : 0.0f; });
}

// --------------------------------------------------------------------------
// tree_accept_sample_draft: one workgroup per request.  R (the unnormalised
// target residual, float64) lives in the workspace row once a rejection has
// changed it (until then it is the node's target row); Q is the node's draft row
// with the removed tokens (an LDS bitmap) read as 0.  Sums of R and Q are formed
// in fixed order; thread 0 takes each acceptance decision.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_tree_accept_sample_draft(
    int T_max, int dcap, int V, int without_replacement, const int* __restrict__ draft_tokens,
    const int* __restrict__ parents, const int* __restrict__ tree_size, const float* __restrict__ target_probs,
    const float* __restrict__ draft_probs, const float* __restrict__ uniforms, const int* __restrict__ status,
    int* __restrict__ accept_len, int* __restrict__ accept_path, int* __restrict__ bonus_token,
    double* __restrict__ ws) {
#pragma clang fp contract(off)
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ int s_tok[kTMaxLimit], s_par[kTMaxLimit], s_path[kTMaxLimit];
  __shared__ float s_uni[kTMaxLimit];
  __shared__ uint32_t s_rm[kMaxV / 32];
  __shared__ double s_d[kWaves];
  __shared__ unsigned long long s_u[kWaves];
  __shared__ int s_dec, s_pick;
  const long long ob = (long long)b * T_max;
  int T = tree_size[b];
  const bool ok = status[b] == TV_ST_OK && T >= 1 && T <= T_max;
  if (!ok) T = 1;
  for (int c = tid; c < T_max; c += kThreads) {
    s_tok[c] = c < T ? draft_tokens[ob + c] : -1;
    s_par[c] = (c > 0 && c < T) ? parents[ob + c] : -2;
    s_uni[c] = uniforms[ob + c];
  }
  const int nw = (V + 31) / 32;
  for (int w = tid; w < nw; w += kThreads) s_rm[w] = 0u;
  if (tid == 0) s_path[0] = 0;
  __syncthreads();
  double* R = ws + (long long)b * V;
  auto removed = [&](int v) { return (s_rm[v >> 5] >> (v & 31)) & 1u; };

  int node = 0, len = 0;
  bool r_ws = false, dirty = false;
  while (ok && len < dcap) {
    const float* p = target_probs + (ob + node) * (long long)V;
    const float* q = draft_probs + (ob + node) * (long long)V;
    if (dirty) {
      for (int w = tid; w < nw; w += kThreads) s_rm[w] = 0u;
      dirty = false;
      __syncthreads();
    }
    r_ws = false;
    double zp = 0.0, zq = 0.0;
    row_pass(V, [&](int v) { return float2{p[v], q[v]}; }, [&](int, float2 e) {
      zp += (double)e.x;
      zq += (double)e.y;
    });
    double ZR = block_sum_d(zp, s_d);
    double ZQ = block_sum_d(zq, s_d);
    int next = -1;
    for (int c = 1; c < T; ++c) {
      if (s_par[c] != node) continue;
      const int x = s_tok[c];
      const bool inside = x >= 0 && x < V;
      if (tid == 0) {
        const double r = inside ? (r_ws ? R[x] : (double)p[x]) : 0.0;
        const double s = (inside && !removed(x)) ? (double)q[x] : 0.0;
        const double lhs = ((double)s_uni[c] * s) * ZR;
        const double rhs = r * ZQ;
        s_dec = (r > 0.0 && (s == 0.0 || lhs < rhs)) ? 1 : 0;
      }
      __syncthreads();
      const bool acc = s_dec != 0;
      __syncthreads();
      if (acc) {
        next = c;
        break;
      }
      if (ZQ > 0.0) {
        // R <- max(0, R ZQ - Q ZR); without replacement Q loses x's mass
        const bool rm = without_replacement && inside;
        double zr = 0.0, zq2 = 0.0;
        struct RQ {
          double r;
          float q;
        };
        row_pass(V, [&](int v) { return RQ{r_ws ? R[v] : (double)p[v], q[v]}; }, [&](int v, RQ e) {
          const double qv = removed(v) ? 0.0 : (double)e.q;
          const double a = e.r * ZQ;
          const double bq = qv * ZR;
          const double nr = fmax(0.0, a - bq);
          R[v] = nr;
          zr += nr;
          zq2 += (rm && v == x) ? 0.0 : qv;
        });
        ZR = block_sum_d(zr, s_d);
        r_ws = true;
        if (rm) {
          ZQ = block_sum_d(zq2, s_d);
          if (tid == 0) s_rm[x >> 5] |= 1u << (x & 31);
          dirty = true;
          __syncthreads();
        }
      }
    }
    if (next < 0) break;
    ++len;
    node = next;
    r_ws = false;
    if (tid == 0) s_path[len] = node;
  }
  __syncthreads();

  // ---- the correction token at `node`, drawn from X = R (after rejections) or the
  // node's row: each thread sums a contiguous token range, a scan places the target
  const float* prow = target_probs + (ob + node) * (long long)V;
  auto X = [&](int v) -> double { return r_ws ? R[v] : (double)prow[v]; };
  const int L = (V + kThreads - 1) / kThreads;
  const int c0 = min(V, tid * L), c1 = min(V, c0 + L);
  double cs = 0.0;
  range_pass(c0, c1, X, [&](int, double x) {
    cs += x;
    return false;
  });
  double lo, hi, total;
  block_scan<double>(cs, s_d, lo, hi, total);
  if (tid == 0) s_pick = -1;
  __syncthreads();
  if (total > 0.0) {
    const double target = (double)s_uni[0] * total;
    if (lo <= target && target < hi) {
      double cum = lo;
      int pick = -1, last = -1;
      range_pass(c0, c1, X, [&](int v, double x) {
        if (x > 0.0) last = v;
        cum += x;
        if (cum > target) {
          pick = v;
          return true;
        }
        return false;
      });
      s_pick = pick >= 0 ? pick : last;
    }
    __syncthreads();
    if (s_pick < 0) {  // rounding left the target past the total: the last token with mass
      int last = -1;
      range_pass(c0, c1, X, [&](int v, double x) {
        if (x > 0.0) last = v;
        return false;
      });
      if (last >= 0) atomicMax(&s_pick, last);
      __syncthreads();
    }
  } else {
    // no residual mass: the node's best token (probability desc, token asc)
    unsigned long long best = 0ull;
    row_pass(V, [&](int v) { return prow[v]; },
             [&](int v, float x) { best = umax64(best, rank_key(x, (uint32_t)v)); });
    best = block_max_u64(best, s_u);
    if (tid == 0) s_pick = (int)key_index(best);
    __syncthreads();
  }
  (void)lane;
  (void)wave;
  if (tid <= dcap) accept_path[(long long)b * (dcap + 1) + tid] = tid <= len ? s_path[tid] : -1;
  if (tid == 0) {
    accept_len[b] = len;
    bonus_token[b] = s_pick;
  }
}

}  // namespace
}  // namespace tv

extern "C" int tree_sampling_probs(int B, int T_max, int V, const float* logits, const int* tree_size,
                                   const int* status, const float* temperature, const int* top_k,
                                   const float* top_p, const float* min_p, float* probs, void* stream) {
  if (B <= 0 || T_max <= 0 || V <= 0) return TV_EINVAL;
  if (T_max > tv::kTMaxLimit || V > tv::kMaxV || B > 65535) return TV_EUNSUPPORTED;
  if (!logits || !tree_size || !temperature || !top_k || !top_p || !min_p || !probs) return TV_EINVAL;
  const size_t n = (size_t)B * T_max * V * sizeof(float);
  const char* a = reinterpret_cast<const char*>(logits);
  const char* c = reinterpret_cast<const char*>(probs);
  if (a < c + n && c < a + n) return TV_EINVAL;  // the output must not overlap the logits
  // Few rows: 1024 threads per row (each row's chain of passes is latency-bound,
  // so more threads per row finish it sooner).  Many rows: 256 threads per row,
  // several rows per CU hiding each other's latency.  Rows of up to 8 tokens per
  // thread stay in registers (more would spill).
  const bool many = (long long)B * T_max >= 512;
  const int nt = many ? 256 : 1024;
  const bool regs = V <= 8 * nt;
  auto k = many ? (regs ? tv::k_sampling_probs<256, 8> : tv::k_sampling_probs<256, 0>)
                : (regs ? tv::k_sampling_probs<1024, 8> : tv::k_sampling_probs<1024, 0>);
  hipLaunchKernelGGL(k, dim3(T_max, B), dim3(nt), 0, reinterpret_cast<hipStream_t>(stream), T_max, V, logits,
                     tree_size, status, temperature, top_k, top_p, min_p, probs);
  TV_CHECK_LAUNCH();
  return TV_OK;
}

extern "C" size_t tree_accept_sample_draft_workspace_bytes(int B, int V) {
  if (B <= 0 || V <= 0) return 0;
  return (size_t)B * V * sizeof(double);
}

extern "C" int tree_accept_sample_draft(int B, int T_max, int dcap, int V, const int* draft_tokens,
                                        const int* parents, const int* tree_size, const float* target_probs,
                                        const float* draft_probs, const float* uniforms, const int* status,
                                        int without_replacement, int* accept_len, int* accept_path,
                                        int* bonus_token, void* workspace, size_t ws_bytes, void* stream) {
  if (B <= 0 || T_max <= 0 || dcap < 0 || dcap >= T_max || V <= 0) return TV_EINVAL;
  if (T_max > tv::kTMaxLimit || V > tv::kMaxV) return TV_EUNSUPPORTED;
  if (!draft_tokens || !parents || !tree_size || !target_probs || !draft_probs || !uniforms || !status ||
      !accept_len || !accept_path || !bonus_token)
    return TV_EINVAL;
  if (!workspace || ws_bytes < (size_t)B * V * sizeof(double) || (reinterpret_cast<uintptr_t>(workspace) & 7))
    return TV_EWORKSPACE;
  hipLaunchKernelGGL(tv::k_tree_accept_sample_draft, dim3(B), dim3(tv::kThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), T_max, dcap, V, without_replacement ? 1 : 0,
                     draft_tokens, parents, tree_size, target_probs, draft_probs, uniforms, status, accept_len,
                     accept_path, bonus_token, reinterpret_cast<double*>(workspace));
  TV_CHECK_LAUNCH();
  return TV_OK;
}
