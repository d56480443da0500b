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
constexpr int kKlMaxV = 32768;   // largest row whose keys stay in LDS (128 KB)
constexpr int kOnDemandK = 4096; // top-k survivors up to which weights are formed on demand
constexpr int kFastK = 256;      // top-k up to which the candidates of a threshold are ranked directly

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

// ---- exact sums of float32 weights.  Every float32 w in [0, 1] is an integer
// number of units of 2^-149: w = m 2^s units with an integer m < 2^24 and
// 0 <= s <= 126.  A sum of weights is held as NL limbs of 32-bit digits (limb j
// weighs 2^(32 j) units), each limb in a 64-bit word that may exceed 32 bits until
// it is normalised (carry-save).  A weight adds less than 2^32 to at most two
// adjacent limbs and a row has at most 2^18 tokens, so no word overflows.
constexpr int NL = 5;
struct Wide {
  unsigned long long l[NL];
};

__device__ __forceinline__ Wide wzero() {
  Wide r;
#pragma unroll
  for (int i = 0; i < NL; ++i) r.l[i] = 0ull;
  return r;
}
__device__ __forceinline__ void wadd(Wide& a, const Wide& b) {
#pragma unroll
  for (int i = 0; i < NL; ++i) a.l[i] += b.l[i];
}
// limb-wise difference, for b <= a limb by limb (b a partial sum of a)
__device__ __forceinline__ Wide wsub(Wide a, const Wide& b) {
#pragma unroll
  for (int i = 0; i < NL; ++i) a.l[i] -= b.l[i];
  return a;
}
__device__ __forceinline__ Wide wmul(Wide a, unsigned long long k) {  // k < 2^18, limbs < 2^32
#pragma unroll
  for (int i = 0; i < NL; ++i) a.l[i] *= k;
  return a;
}
// w = m 2^s units: the limb j = s / 32 and the mantissa shifted into it (< 2^56;
// its bits 32 and up belong to limb j + 1)
__device__ __forceinline__ void weight_parts(float w, int& j, unsigned long long& x) {
  const uint32_t u = __float_as_uint(w);
  const uint32_t e = u >> 23;  // w >= 0: no sign bit
  const uint32_t m = e ? ((u & 0x7FFFFFu) | 0x800000u) : u;
  const int s = e ? (int)e - 1 : 0;
  j = s >> 5;
  x = (unsigned long long)m << (s & 31);
}
__device__ __forceinline__ Wide wide_of(float w) {
  int j;
  unsigned long long x;
  weight_parts(w, j, x);
  Wide r;
#pragma unroll
  for (int i = 0; i < NL; ++i)
    r.l[i] = (i == j ? (x & 0xFFFFFFFFull) : 0ull) + (i == j + 1 ? (x >> 32) : 0ull);
  return r;
}
// A normalised sum: NN limbs of 32 bits (192 bits; a row's total is below 2^167)
constexpr int NN = 6;
struct Norm {
  uint32_t l[NN];
};
__device__ __forceinline__ Norm norm_of(const Wide& a) {
  Norm n;
  unsigned long long c = 0ull;
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const unsigned long long v = a.l[i] + c;
    n.l[i] = (uint32_t)v;
    c = v >> 32;
  }
  n.l[NL] = (uint32_t)c;
  return n;
}
__device__ __forceinline__ Norm nzero() {
  Norm r;
#pragma unroll
  for (int i = 0; i < NN; ++i) r.l[i] = 0u;
  return r;
}
__device__ __forceinline__ Norm nadd(const Norm& a, const Norm& b) {
  Norm r;
  unsigned long long c = 0ull;
#pragma unroll
  for (int i = 0; i < NN; ++i) {
    const unsigned long long v = (unsigned long long)a.l[i] + b.l[i] + c;
    r.l[i] = (uint32_t)v;
    c = v >> 32;
  }
  return r;
}
__device__ __forceinline__ bool nge(const Norm& a, const Norm& b) {
  bool gt = false, eq = true;  // decided from the top limb down
#pragma unroll
  for (int i = NN - 1; i >= 0; --i) {
    gt = gt || (eq && a.l[i] > b.l[i]);
    eq = eq && a.l[i] == b.l[i];
  }
  return gt || eq;
}
// a value every lane holds the same copy of: kept in scalar registers
__device__ __forceinline__ Norm nuniform(const Norm& a) {
  Norm r;
#pragma unroll
  for (int i = 0; i < NN; ++i) r.l[i] = (uint32_t)__builtin_amdgcn_readfirstlane((int)a.l[i]);
  return r;
}
__device__ __forceinline__ Norm nshfl_down(const Norm& a, int o) {
  Norm r;
#pragma unroll
  for (int i = 0; i < NN; ++i) r.l[i] = (uint32_t)__shfl_down((int)a.l[i], o, 64);
  return r;
}
__device__ __forceinline__ Wide wshfl_xor(const Wide& a, int m) {
  Wide r;
#pragma unroll
  for (int i = 0; i < NL; ++i) r.l[i] = __shfl_xor(a.l[i], m, 64);
  return r;
}
// t[k] for a run-time k (0 past the end), without indexing registers dynamically
__device__ __forceinline__ unsigned long long limb_at(const unsigned long long (&t)[NN + 1], int k) {
  unsigned long long v = 0ull;
#pragma unroll
  for (int i = 0; i <= NN; ++i) v = i == k ? t[i] : v;
  return v;
}
// ceil(x / 2^q) of NN + 1 limbs of 32 bits (0 <= q < 32 NN; the result fits NN limbs)
__device__ __forceinline__ Norm nshr_ceil(const unsigned long long (&t)[NN + 1], int q) {
  const int ws = q >> 5, bs = q & 31;
  bool sticky = (limb_at(t, ws) & ((1ull << bs) - 1ull)) != 0ull;
#pragma unroll
  for (int i = 0; i < NN; ++i) sticky |= i < ws && t[i] != 0ull;
  Norm r;
#pragma unroll
  for (int i = 0; i < NN; ++i)
    r.l[i] = (uint32_t)((limb_at(t, i + ws) >> bs) | (limb_at(t, i + ws + 1) << (32 - bs)));
  Norm one = nzero();
  one.l[0] = sticky ? 1u : 0u;
  return nadd(r, one);
}
// a float32 x > 0 is m 2^(s - 149) exactly: an integer m < 2^24 and s >= 0
__device__ __forceinline__ void float_parts(float x, unsigned long long& m, int& s) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t e = u >> 23;
  m = e ? ((u & 0x7FFFFFu) | 0x800000u) : u;
  s = e ? (int)e - 1 : 0;
}
// ceil(p z) for a float32 p in (0, 1): an integer cumulative c has c >= p z
// exactly when c >= ceil(p z).  p = m 2^-q with q = 149 - s >= 24.
__device__ __forceinline__ Norm nthreshold(float p, const Norm& z) {
  unsigned long long m;
  int s;
  float_parts(p, m, s);
  unsigned long long t[NN + 1];
  unsigned long long c = 0ull;
#pragma unroll
  for (int i = 0; i < NN; ++i) {  // m z, limb by limb (z's limbs < 2^32, m < 2^24)
    const unsigned long long v = (unsigned long long)z.l[i] * m + c;
    t[i] = v & 0xFFFFFFFFull;
    c = v >> 32;
  }
  t[NN] = c;
  return nshr_ceil(t, 149 - s);
}
// the smallest n >= 1 with above + n c >= thr, for a float32 weight c > 0 and
// above < thr (2^31 - 1 stands for anything larger)
__device__ __forceinline__ int ntie_count(const Norm& thr, const Norm& above, float c) {
  unsigned long long t[NN + 1];
  long long br = 0;
#pragma unroll
  for (int i = 0; i < NN; ++i) {  // t = thr - above, borrows propagated
    const long long v = (long long)thr.l[i] - (long long)above.l[i] - br;
    br = v < 0 ? 1 : 0;
    t[i] = (unsigned long long)(v + (br << 32));
  }
  t[NN] = 0ull;
  // c = m 2^s units: n = ceil(ceil(t / 2^s) / m), the division digit by digit
  unsigned long long m;
  int s;
  float_parts(c, m, s);
  const Norm d = nshr_ceil(t, s);
  unsigned long long rem = 0ull, hiq = 0ull, q0 = 0ull;
#pragma unroll
  for (int i = NN - 1; i >= 0; --i) {
    const unsigned long long cur = (rem << 32) | d.l[i];  // rem < m < 2^24
    const unsigned long long qd = cur / m;
    rem = cur % m;
    if (i > 0) hiq |= qd;
    else q0 = qd;
  }
  if (hiq || q0 >= 0x7FFFFFFFull) return 0x7FFFFFFF;
  const long long n = (long long)q0 + (rem ? 1 : 0);
  return n < 1 ? 1 : (int)n;
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
// the top, with exact totals (counts for top-k; for top-p the exact sums of the
// float32 weights, as Wide integers in units of 2^-149, and the exact threshold
// ceil(top_p x total)).  Equal keys have equal weights; the cut inside a group of
// equal keys is the n-th of them in token order, found by a scan over contiguous
// token ranges.
// --------------------------------------------------------------------------
// NPT > 0: V <= NPT NT and every thread keeps its NPT (key, weight) pairs in
// registers after the first read; NPT = 0: KL: the keys are kept in LDS (V <=
// kKlMaxV), else the logits are re-read on every pass.
// With top-k on and at most kOnDemandK survivors, the weights are formed only
// for the tokens that need one (the survivors), when they need it; otherwise
// every weight is formed once and kept (registers, or the output row).
template <int NT, int NPT, bool KL = false>
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
  __shared__ Wide s_w[NW];
  // radix bins (counts: CSETS sets of 256, shared by the wavefronts w % CSETS; or
  // NL x 256 limbs of weight sums), ballot entries (V / 64), or the survivor list
  constexpr int CSETS = KL ? 4 : NW;
  constexpr int HIST = KL ? NL * 256 : 4096;
  __shared__ unsigned long long s_hist[HIST];
  static_assert(CSETS * 256 <= HIST && NL * 256 <= HIST && NT <= HIST && (!KL || kKlMaxV / 64 <= HIST),
                "radix bins, survivor list and ballot entries fit");
  __shared__ Norm s_abv;
  __shared__ Wide s_wt_total;
  __shared__ unsigned long long s_top[NT];  // the top-k survivors in rank order (top-k fast path)
  __shared__ unsigned long long s_abvc;
  __shared__ int s_pick, s_sel, s_cnt;
  extern __shared__ uint32_t s_key[];  // KL: the order key of token v
  static_assert(!KL || (NPT == 0 && NT == 1024), "keys in LDS: 1024 threads, no register copy");

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
  } else if constexpr (KL) {
    // the whole row in flight at once (up to kKlMaxV / NT = 32 tokens per thread)
    constexpr int J = kKlMaxV / NT;
    float x[J];
#pragma unroll
    for (int j = 0; j < J; ++j) x[j] = tid + j * NT < V ? lr[tid + j * NT] : -INFINITY;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int v = tid + j * NT;
      if (v < V) {
        s_key[v] = logit_key(x[j]);  // read back by this thread only (the same v in every pass)
        best = umax64(best, rank_key(clean_logit(x[j]), (uint32_t)v));
      }
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
  // Weights formed on demand (top-k on with few survivors) or kept: NPT > 0 in
  // registers, NPT = 0 in the output row, where each thread re-reads only the
  // weights it wrote (the same v in every row pass).
  const bool stored = NPT > 0 || !(kk > 1 && kk < V && kk <= kOnDemandK);
  auto wt = [&](uint32_t k, float w) -> float { return stored ? w : weight(k); };
  auto ld_kw = [&](int v) {
    const uint32_t k = KL ? s_key[v] : logit_key(lr[v]);
    return KW{k, stored ? orow[v] : 0.0f};
  };
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
  // the workgroup's sum of one Wide per thread (every thread gets it, carry-save):
  // wavefront totals by butterfly, then the first wavefront adds them
  auto block_wsum = [&](Wide v) -> Wide {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) wadd(v, wshfl_xor(v, o));
    if ((tid & 63) == 0) s_w[tid >> 6] = v;
    __syncthreads();
    if (tid < 64) {
      Wide t = (tid < NW) ? s_w[tid] : wzero();
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) wadd(t, wshfl_xor(t, o));
      if (tid == 0) s_wt_total = t;
    }
    __syncthreads();
    const Wide t = s_wt_total;
    __syncthreads();
    return t;
  };
  const bool with_p = tp < 1.0f;
  Wide w_all = wzero();  // this thread's total weight (only needed for top-p)
  if constexpr (NPT > 0) {
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      reg[j].w = weight(reg[j].k);
      if (with_p && tid + j * NT < V) wadd(w_all, wide_of(reg[j].w));
    }
  } else if (stored) {
    if constexpr (KL) {
      for (int v = tid; v < V; v += NT) {
        const float w = weight(s_key[v]);
        orow[v] = w;
        if (with_p) wadd(w_all, wide_of(w));
      }
    } else {
      row_pass<NT>(V, ld_l, [&](int v, float x) {
        const float w = weight(logit_key(x));
        orow[v] = w;
        if (with_p) wadd(w_all, wide_of(w));
      });
    }
  }

  const int lane = tid & 63, wave = tid >> 6;
  // The n-th token (token order, n >= 1) with key t inside the top-k cut (tk, ck),
  // in one coalesced pass: for each slice of NT consecutive tokens, every
  // wavefront's ballot of its matching tokens goes to LDS, slice-major, so the
  // entries are in token order; the first wavefront then finds the entry holding
  // the n-th match (64 entries per lane at most, a scan over the lanes) and the
  // bit inside it.  With `mass`, also returns the exact total weight of the
  // tokens with key > t (all inside the cut, since t >= tk).
  const int nsl = (V + NT - 1) / NT;  // <= 256 slices, <= 4096 entries
  auto nth_with_key = [&](uint32_t t, int n, uint32_t tk, int ck, bool mass, Wide& mass_above) -> int {
    Wide ma = wzero();
    auto body = [&](int j, uint32_t k, float w) __attribute__((always_inline)) {
      const int v = j * NT + tid;
      const bool f = v < V && k == t && (k > tk || v <= ck);
      const unsigned long long m = __ballot(f);
      if (lane == 0) s_hist[j * NW + wave] = m;
      if (mass && v < V && k > t) wadd(ma, wide_of(wt(k, w)));
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
    mass_above = mass ? block_wsum(ma) : wzero();
    return res;
  };

  // ---- radix selection over the keys, eight bits per pass from the top.  Each
  // pass histograms the tokens whose key matches the digits chosen so far into 256
  // bins of the next digit (LDS integer atomics: the totals are exact, so the
  // order of the additions does not matter), then the first wavefront places the
  // target among the bins (four bins per lane, a suffix sum over the lanes) and
  // the highest bin at which the running total reaches the target is chosen.
  // Counts (top-k): the key of the kk-th ranked token and the number of tokens
  // with larger keys.
  // `visit(f)` calls f(key) for every element counted (each token, or one value per thread).
  auto radix_count = [&](int kk_, uint32_t& t_out, int& above_out, auto visit) {
    uint32_t prefix = 0u, pmask = 0u;
    unsigned long long above = 0ull;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int e = tid; e < CSETS * 256; e += NT) s_hist[e] = 0ull;
      __syncthreads();
      visit([&](uint32_t k) {
        if ((k & pmask) == prefix) atomicAdd(&s_hist[(wave % CSETS) * 256 + ((k >> shift) & 255u)], 1ull);
      });
      __syncthreads();
      if (wave == 0) {
        unsigned long long m[4], g = 0ull;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          m[j] = 0ull;
          for (int w = 0; w < CSETS; ++w) m[j] += s_hist[w * 256 + 4 * lane + j];
          g += m[j];
        }
        unsigned long long suf = g;  // total of this lane's bins and every higher lane's
        for (int o = 1; o < 64; o <<= 1) {
          const unsigned long long y = __shfl_down(suf, o, 64);
          if (lane + o < 64) suf += y;
        }
        unsigned long long run = above + (suf - g);
        int cand = -1;
        unsigned long long cabove = 0ull;
#pragma unroll
        for (int j = 3; j >= 0; --j) {
          if (cand < 0 && run + m[j] >= (unsigned long long)kk_) {
            cand = 4 * lane + j;
            cabove = run;
          }
          run += m[j];
        }
        const unsigned long long hit = __ballot(cand >= 0);
        if (hit && lane == 63 - __builtin_clzll(hit)) {  // the highest digit that reaches the target
          s_sel = cand;
          s_abvc = cabove;
        }
      }
      __syncthreads();
      const int sel = s_sel;  // always found: kk_ < V tokens
      above = s_abvc;
      __syncthreads();
      prefix |= (uint32_t)sel << shift;
      pmask |= 255u << shift;
    }
    t_out = prefix;
    above_out = (int)above;
  };
  // Weights (top-p): over the tokens with pred, the key of the first token at
  // which the exact cumulative weight reaches thr, the exact weight of the tokens
  // with larger keys, and false if thr is never reached.  The bins hold NL
  // carry-save limbs each (limb-major: s_hist[limb 256 + bin]); a token adds to
  // the one or two limbs its weight covers.
  auto radix_mass = [&](auto pred, const Norm& thr, uint32_t& t_out, Norm& above_out) -> bool {
    uint32_t prefix = 0u, pmask = 0u;
    Norm above = nzero();
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int e = tid; e < NL * 256; e += NT) s_hist[e] = 0ull;
      __syncthreads();
      pass([&](int v, KW e) {
        const float w = (e.k & pmask) == prefix && pred(e.k, v) ? wt(e.k, e.w) : 0.0f;
        if (w > 0.0f) {
          int j;
          unsigned long long x;
          weight_parts(w, j, x);
          const int bin = (int)((e.k >> shift) & 255u);
          atomicAdd(&s_hist[j * 256 + bin], x & 0xFFFFFFFFull);
          if (x >> 32) atomicAdd(&s_hist[(j + 1) * 256 + bin], x >> 32);
        }
      });
      __syncthreads();
      if (wave == 0) {
        auto bin_at = [&](int bin) {
          Wide x;
#pragma unroll
          for (int i = 0; i < NL; ++i) x.l[i] = s_hist[i * 256 + bin];
          return x;
        };
        Wide g = wzero();
#pragma unroll
        for (int j = 0; j < 4; ++j) wadd(g, bin_at(4 * lane + j));
        Norm suf = norm_of(g);  // this lane's bins and every higher lane's
        for (int o = 1; o < 64; o <<= 1) {
          const Norm y = nshfl_down(suf, o);
          if (lane + o < 64) suf = nadd(suf, y);
        }
        Norm run = nshfl_down(suf, 1);  // every higher lane's bins
        if (lane == 63) run = nzero();
        run = nadd(run, above);
        int cand = -1;
        Norm cabove = nzero();
#pragma unroll
        for (int j = 3; j >= 0; --j) {  // (unrolled, no early exit: nothing is indexed dynamically)
          const Norm r2 = nadd(run, norm_of(bin_at(4 * lane + j)));
          if (cand < 0 && nge(r2, thr)) {
            cand = 4 * lane + j;
            cabove = run;
          }
          run = r2;
        }
        const unsigned long long hit = __ballot(cand >= 0);
        if (lane == 0) s_sel = -1;
        if (hit && lane == 63 - __builtin_clzll(hit)) {  // the highest digit that reaches thr
          s_sel = cand;
          s_abv = cabove;
        }
      }
      __syncthreads();
      const int sel = s_sel;
      above = nuniform(s_abv);
      __syncthreads();
      if (sel < 0) return false;
      prefix |= (uint32_t)sel << shift;
      pmask |= 255u << shift;
    }
    t_out = prefix;
    above_out = above;
    return true;
  };

  // ---- top-k cut (tk, ck); the default keeps everything (every key is > 0)
  uint32_t tk = 0u;
  int ck = V;
  Norm wk = nzero();  // the survivors' exact total weight (top-p)
  // Fast path, 1 < top_k <= kFastK: at least top_k tokens reach tau, the key of
  // the top_k-th best of the per-thread best tokens (each thread's best is a
  // distinct token), so the top_k survivors are among the tokens whose key
  // reaches tau: usually a few more than top_k.  They are gathered into LDS and
  // ranked exactly by counting, which leaves them in rank order in s_top.  With
  // more candidates than the list holds, the general path below runs instead.
  bool sorted = false;
  if (kk > 1 && kk <= kFastK && kk < V) {
    unsigned long long tm = 0ull;  // this thread's best token as a rank key
    pass([&](int v, KW e) { tm = umax64(tm, ((unsigned long long)e.k << 32) | (0xFFFFFFFFu - (uint32_t)v)); });
    uint32_t tau_k = 0u;
    int above_t = 0;
    const uint32_t mk = (uint32_t)(tm >> 32);  // 0 (below every key) for a thread without tokens
    radix_count(kk, tau_k, above_t, [&](auto f) { f(mk); });
    unsigned long long* s_cand = s_hist;
    if (tid == 0) s_cnt = 0;
    __syncthreads();
    pass([&](int v, KW e) {
      if (e.k >= tau_k) {
        const int pos = atomicAdd(&s_cnt, 1);
        if (pos < HIST) s_cand[pos] = ((unsigned long long)e.k << 32) | (0xFFFFFFFFu - (uint32_t)v);
      }
    });
    __syncthreads();
    const int m = s_cnt;
    if (m <= HIST) {
      for (int t = tid; t < m; t += NT) {
        const unsigned long long my = s_cand[t];
        int rk = 0;
        for (int o = 0; o < m; ++o) rk += s_cand[o] > my;  // (all lanes read the same entry)
        if (rk < kk) s_top[rk] = my;
      }
      __syncthreads();
      const unsigned long long last = s_top[kk - 1];
      tk = (uint32_t)(last >> 32);
      ck = (int)key_index(last);
      sorted = true;
      if (with_p) wk = nuniform(norm_of(block_wsum(tid < kk ? wide_of(weight((uint32_t)(s_top[tid] >> 32)))
                                                               : wzero())));
    }
    __syncthreads();
  }
  if (!sorted) {
    if (with_p) wk = nuniform(norm_of(block_wsum(w_all)));
    if (kk > 1 && kk < V) {
      int above = 0;
      Wide ma = wzero();
      radix_count(kk, tk, above, [&](auto f) { pass([&](int, KW e) { f(e.k); }); });
      const int need = kk - above;
      ck = nth_with_key(tk, need, 0u, V, with_p, ma);
      wadd(ma, wmul(wide_of(weight(tk)), (unsigned long long)need));
      wk = nuniform(norm_of(ma));
    }
  }
  auto in_k = [&](uint32_t k, int v) { return k > tk || (k == tk && v <= ck); };

  // ---- top-p cut (tpk, cp) over the top-k survivors: the shortest rank prefix
  // whose exact cumulative weight c satisfies c >= top_p x total, i.e.
  // c >= thr = ceil(top_p x total) (c is an integer number of units)
  uint32_t tpk = 0u;
  int cp = V;
  const Norm thr = with_p ? nuniform(nthreshold(tp, wk)) : nzero();
  if (with_p && kk > 1 && kk <= NT) {
    // at most NT survivors: gathered into LDS as 64-bit rank keys (key,
    // then token ascending; the order of the appends does not matter), sorted
    // descending by a bitonic network (the fast path has them in order already),
    // then one exact prefix sum of their weights in rank order finds the cut
    unsigned long long* s_list = sorted ? s_top : s_hist;  // NT entries
    const int n = sorted ? kk : min(kk, NT);
    if (!sorted) {
      if (tid == 0) s_cnt = 0;
      __syncthreads();
      pass([&](int v, KW e) {
        if (in_k(e.k, v)) {
          const int pos = atomicAdd(&s_cnt, 1);  // < kk by construction of the cut
          if (pos < NT) s_list[pos] = rank_key(key_float(e.k), (uint32_t)v);
        }
      });
      __syncthreads();
    }
    if (tid >= n) s_list[tid] = 0ull;
    __syncthreads();
    for (int k2 = 2; !sorted && k2 <= NT; k2 <<= 1) {
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
    // inclusive prefix (rank order) of the exact weights: a lane scan, then the
    // totals of the earlier wavefronts
    Wide incl = tid < n ? wide_of(weight((uint32_t)(mine >> 32))) : wzero();
    for (int o = 1; o < 64; o <<= 1) {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const unsigned long long y = __shfl_up(incl.l[i], o, 64);
        if (lane >= o) incl.l[i] += y;
      }
    }
    if (lane == 63) s_w[wave] = incl;
    if (tid == 0) s_pick = n;
    __syncthreads();
    for (int w = 0; w < wave; ++w) wadd(incl, s_w[w]);
    if (tid < n && nge(norm_of(incl), thr)) atomicMin(&s_pick, tid);
    __syncthreads();
    const int cut = s_pick;  // the last kept rank
    if (cut < n) {
      const unsigned long long kc = s_list[cut];
      tpk = (uint32_t)(kc >> 32);
      cp = (int)key_index(kc);
    }
    __syncthreads();
  } else if (with_p) {
    Norm above = nzero();
    Wide unused = wzero();
    if (radix_mass(in_k, thr, tpk, above)) {
      // the survivors with key tpk all weigh ct: in token order, the first n of
      // them bring the cumulative to thr (n = ceil((thr - above) / ct))
      const int n = ntie_count(thr, above, weight(tpk));
      cp = nth_with_key(tpk, n, tk, ck, false, unused);
    } else {
      tpk = 0u;  // never reached: every survivor stays
    }
  }

  // ---- min-p, the kept total and the output
  // the weight of a kept token, 0 for the others (a weight is formed only for the
  // top-k and top-p survivors)
  auto kept_w = [&](uint32_t k, int v, float w) -> float {
    if (!(in_k(k, v) && (k > tpk || (k == tpk && v <= cp)))) return 0.0f;
    const float x = wt(k, w);
    return (!(mp > 0.0f) || x >= mp || v == tok0) ? x : 0.0f;
  };
  double wsum = 0.0;
  pass([&](int v, KW e) { wsum += (double)kept_w(e.k, v, e.w); });
  const double W = block_sum_d<NT>(wsum, s_d);
  pass([&](int v, KW e) {
    const float x = kept_w(e.k, v, e.w);
    orow[v] = x > 0.0f ? (float)((double)x / W) : 0.0f;
  });
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
  // Rows that do not fit the registers but whose keys fit LDS: 1024 threads with
  // the keys in LDS (one row per CU; every pass after the first read stays on chip).
  const bool many = (long long)B * T_max >= 512;
  int nt = many ? 256 : 1024;
  const bool regs = V <= 8 * nt;
  const bool kl = !regs && V <= tv::kKlMaxV;
  if (kl) nt = 1024;
  auto k = kl ? tv::k_sampling_probs<1024, 0, true>
              : many ? (regs ? tv::k_sampling_probs<256, 8> : tv::k_sampling_probs<256, 0>)
                     : (regs ? tv::k_sampling_probs<1024, 8> : tv::k_sampling_probs<1024, 0>);
  const size_t dyn = kl ? (size_t)V * sizeof(uint32_t) : 0;
  if (kl) {
    static bool attr_set = false;  // the LDS a launch may ask for, raised once
    if (!attr_set) {
      if (hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)(tv::kKlMaxV * sizeof(uint32_t))) != hipSuccess)
        return TV_ELAUNCH;
      attr_set = true;
    }
  }
  hipLaunchKernelGGL(k, dim3(T_max, B), dim3(nt), dyn, reinterpret_cast<hipStream_t>(stream), T_max, V, logits,
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
