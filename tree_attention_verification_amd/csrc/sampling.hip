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
// wavefront by a fixed tree of lane moves, the wavefronts in index order), so results do not
// depend on scheduling.  Products and differences that decide an outcome are
// rounded one at a time (no fused multiply-add), as written.
#include <type_traits>

#include "tv_common.h"

namespace tv {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxV = 262144;  // vocabulary limit (the removed-token bitmap is 32 KB of LDS)
constexpr int kKlMaxV = 32768;   // largest row whose keys stay in LDS (128 KB)
constexpr int kFastK = 256;      // top-k up to which the candidates of a threshold are ranked directly

__device__ __forceinline__ double wave_sum_d(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Wavefront reductions by DPP moves (no LDS round trips): an inclusive scan in
// rows of 16 lanes (row_shr 1, 2, 4, 8; lanes without a source read 0), then
// lane 15 of rows 0 and 2 into rows 1 and 3 (row_bcast 15) and lane 31 into
// rows 2 and 3 (row_bcast 31): lane 63 ends with the whole wavefront's value.
template <int CTRL, int ROWS>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long x) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)x, CTRL, ROWS, 0xF, true);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(x >> 32), CTRL, ROWS, 0xF, true);
  return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}
// (every lane ends with the inclusive scan of the lanes up to its own)
template <class Op>
__device__ __forceinline__ unsigned long long wave_scan_dpp(unsigned long long v, Op op) {
  v = op(v, dpp_u64<0x111, 0xF>(v));
  v = op(v, dpp_u64<0x112, 0xF>(v));
  v = op(v, dpp_u64<0x114, 0xF>(v));
  v = op(v, dpp_u64<0x118, 0xF>(v));
  v = op(v, dpp_u64<0x142, 0xA>(v));
  v = op(v, dpp_u64<0x143, 0xC>(v));
  return v;
}
template <class Op>
__device__ __forceinline__ unsigned long long wave_reduce_dpp(unsigned long long v, Op op) {
  return readlane_u64(wave_scan_dpp(v, op), 63);
}
__device__ __forceinline__ double wave_sum_dpp(double v) {
  return __longlong_as_double((long long)wave_reduce_dpp(
      (unsigned long long)__double_as_longlong(v), [](unsigned long long x, unsigned long long y) {
        return (unsigned long long)__double_as_longlong(__longlong_as_double((long long)x) +
                                                        __longlong_as_double((long long)y));
      }));
}
__device__ __forceinline__ unsigned long long wave_max_dpp(unsigned long long v) {
  return wave_reduce_dpp(v, [](unsigned long long x, unsigned long long y) { return x > y ? x : y; });
}
__device__ __forceinline__ int wave_incl_scan_dpp(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr 1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr 2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr 4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr 8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, true);  // row_bcast 15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, true);  // row_bcast 31 into rows 2, 3
  return v;
}

// sum over the workgroup; every thread gets the same value (s: (NT / 64) slots)
template <int NT = kThreads>
__device__ __forceinline__ double block_sum_d(double v, double* s) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum_dpp(v);
  if (lane == 0) s[wave] = v;
  __syncthreads();
  double t = 0.0;
  for (int w = 0; w < (NT / 64); ++w) t += s[w];
  __syncthreads();
  return t;
}

// two sums and two maxima at once (one round of barriers); every thread gets all
template <int NT = kThreads>
__device__ __forceinline__ void block_sum2_max2(double& a, double& c, unsigned long long& m0, unsigned long long& m1,
                                                unsigned long long* s) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  a = wave_sum_dpp(a);
  c = wave_sum_dpp(c);
  m0 = wave_max_dpp(m0);
  m1 = wave_max_dpp(m1);
  if (lane == 0) {
    s[4 * wave] = (unsigned long long)__double_as_longlong(a);
    s[4 * wave + 1] = (unsigned long long)__double_as_longlong(c);
    s[4 * wave + 2] = m0;
    s[4 * wave + 3] = m1;
  }
  __syncthreads();
  double ta = 0.0, tc = 0.0;
  unsigned long long t0 = 0ull, t1 = 0ull;
  for (int w = 0; w < (NT / 64); ++w) {
    ta += __longlong_as_double((long long)s[4 * w]);
    tc += __longlong_as_double((long long)s[4 * w + 1]);
    t0 = umax64(t0, s[4 * w + 2]);
    t1 = umax64(t1, s[4 * w + 3]);
  }
  __syncthreads();
  a = ta;
  c = tc;
  m0 = t0;
  m1 = t1;
}
// two sums at once (one round of barriers); every thread gets both
template <int NT = kThreads>
__device__ __forceinline__ void block_sum_d2(double& a, double& c, double* s) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  a = wave_sum_d(a);
  c = wave_sum_d(c);
  if (lane == 0) {
    s[2 * wave] = a;
    s[2 * wave + 1] = c;
  }
  __syncthreads();
  double ta = 0.0, tc = 0.0;
  for (int w = 0; w < (NT / 64); ++w) {
    ta += s[2 * w];
    tc += s[2 * w + 1];
  }
  __syncthreads();
  a = ta;
  c = tc;
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
  if constexpr (std::is_same_v<T, int>) {
    incl = wave_incl_scan_dpp(v);
  } else if constexpr (std::is_same_v<T, unsigned long long>) {
    incl = wave_scan_dpp(v, [](unsigned long long a, unsigned long long b) { return a + b; });
  } else {
    for (int o = 1; o < 64; o <<= 1) {
      const T y = __shfl_up(incl, o, 64);
      if (lane >= o) incl = incl + y;
    }
  }
  if (lane == 63) s[wave] = incl;
  __syncthreads();
  T off = T(0), tot = T(0);
  for (int w = 0; w < (NT / 64); ++w) {
    if (w < wave) off = off + s[w];
    tot = tot + s[w];
  }
  __syncthreads();
  if constexpr (std::is_same_v<T, int> || std::is_same_v<T, unsigned long long>) {
    lo = off + (incl - v);  // (exact)
  } else {
    const T up = __shfl_up(incl, 1, 64);
    lo = lane > 0 ? off + up : off;
  }
  hi = off + incl;
  total = tot;
}

template <int NT = kThreads>
__device__ __forceinline__ unsigned long long block_max_u64(unsigned long long v, unsigned long long* s) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_max_dpp(v);
  if (lane == 0) s[wave] = v;
  __syncthreads();
  unsigned long long t = 0ull;
  for (int w = 0; w < (NT / 64); ++w) t = umax64(t, s[w]);
  __syncthreads();
  return t;
}

// The workgroup maximum of two values at once (one barrier pair); s holds
// 2 NT / 64 entries.
template <int NT = kThreads>
__device__ __forceinline__ void block_max2_u64(unsigned long long& a, unsigned long long& c, unsigned long long* s) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  a = wave_max_dpp(a);
  c = wave_max_dpp(c);
  if (lane == 0) {
    s[wave] = a;
    s[NT / 64 + wave] = c;
  }
  __syncthreads();
  unsigned long long ta = 0ull, tc = 0ull;
  for (int w = 0; w < (NT / 64); ++w) {
    ta = umax64(ta, s[w]);
    tc = umax64(tc, s[NT / 64 + w]);
  }
  __syncthreads();
  a = ta;
  c = tc;
}

// s_waitcnt immediate (gfx9 encoding) that waits for every vector memory
// operation of the wavefront, stores included, and for nothing else: vmcnt 0
// (bits 3:0 and 15:14), expcnt 7 (bits 6:4), lgkmcnt 15 (bits 11:8)
constexpr int kVmemStoresDone = (7 << 4) | (15 << 8);

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
// ms 2^s units as a Wide, for ms < 2^44 and 0 <= s <= 126 (limbs chosen by
// selects: nothing is indexed at run time)
__device__ __forceinline__ Wide wide_shifted(unsigned long long ms, int s) {
  const int q = s >> 5, r = s & 31;
  const unsigned long long lo = ms << r, hi = r ? ms >> (64 - r) : 0ull;  // ms 2^r; hi < 2^13
  Wide x;
#pragma unroll
  for (int i = 0; i < NL; ++i)
    x.l[i] = (i == q ? (lo & 0xFFFFFFFFull) : 0ull) + (i == q + 1 ? (lo >> 32) : 0ull) + (i == q + 2 ? hi : 0ull) +
             (i == NL - 1 && q + 2 == NL ? (hi << 32) : 0ull);
  return x;
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
// an int / u32 / u64 every lane holds alike, moved to scalar registers
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ uint32_t uni(uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); }
__device__ __forceinline__ unsigned long long uni(unsigned long long x) {
  return ((unsigned long long)uni((uint32_t)(x >> 32)) << 32) | uni((uint32_t)x);
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
__device__ __forceinline__ Norm nshfl(const Norm& a, int src) {
  Norm r;
#pragma unroll
  for (int i = 0; i < NN; ++i) r.l[i] = (uint32_t)__shfl((int)a.l[i], src, 64);
  return r;
}
__device__ __forceinline__ Wide wshfl_down(const Wide& a, int o) {
  Wide r;
#pragma unroll
  for (int i = 0; i < NL; ++i) r.l[i] = __shfl_down(a.l[i], o, 64);
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
// the value of a sum in units of 2^-149, rounded to double
__device__ __forceinline__ double norm_to_double(const Norm& a) {
  double r = 0.0;
#pragma unroll
  for (int i = NN - 1; i >= 0; --i) r = r * 4294967296.0 + (double)a.l[i];
  return r * 0x1p-149;
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
// PF: the next NB loads are issued before the current ones are processed, so
// that neither their latency nor stores in the body hold them up.
constexpr int kNB = 8;
template <int NT = kThreads, bool PF = false, class Load, class Body>
__device__ __forceinline__ void row_pass(int V, Load load, Body body) {
  using T = decltype(load(0));
  if constexpr (PF) {
    T x[kNB];
#pragma unroll
    for (int j = 0; j < kNB; ++j) x[j] = load(min((int)threadIdx.x + j * NT, V - 1));
    for (int base = threadIdx.x; base < V; base += kNB * NT) {
      T y[kNB];
#pragma unroll
      for (int j = 0; j < kNB; ++j) y[j] = load(min(base + (kNB + j) * NT, V - 1));
#pragma unroll
      for (int j = 0; j < kNB; ++j)
        if (base + j * NT < V) body(base + j * NT, x[j]);
#pragma unroll
      for (int j = 0; j < kNB; ++j) x[j] = y[j];
    }
  } else {
    for (int base = threadIdx.x; base < V; base += kNB * NT) {
      T x[kNB];
#pragma unroll
      for (int j = 0; j < kNB; ++j) x[j] = load(min(base + j * NT, V - 1));
#pragma unroll
      for (int j = 0; j < kNB; ++j)
        if (base + j * NT < V) body(base + j * NT, x[j]);
    }
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

// Over a row of 4 n tokens, four consecutive ones per visit: thread t visits
// quads q = t + j NT (tokens 4 q .. 4 q + 3) in increasing q, with the loads of
// kQB quads issued together; indices past the row are clamped for the load and
// skipped for the body.
constexpr int kQB = 4;
template <int NT, class Load, class Body>
__device__ __forceinline__ void quad_pass(int n4, Load load, Body body) {
  using T = decltype(load(0));
  for (int base = threadIdx.x; base < n4; base += kQB * NT) {
    T x[kQB];
#pragma unroll
    for (int j = 0; j < kQB; ++j) x[j] = load(min(base + j * NT, n4 - 1));
#pragma unroll
    for (int j = 0; j < kQB; ++j)
      if (base + j * NT < n4) body(base + j * NT, x[j]);
  }
}
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// logits: NaN ranks as -inf; order_key canonicalises -0.0
__device__ __forceinline__ float clean_logit(float x) { return x != x ? -INFINITY : x; }
__device__ __forceinline__ uint32_t logit_key(float x) { return order_key(clean_logit(x)); }
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// --------------------------------------------------------------------------
// tree_sampling_probs: one workgroup per (node row, request).
//
// Tokens rank by (logit descending, token ascending), with weights
// w = fp32(exp((l - l_max) / temperature)) (exactly 1 at the largest logit).
// Each filter keeps a prefix of the ranking, described by a cut (key t, token c):
// token v with key k is inside iff k > t or (k == t and v <= c).  Both cuts are
// found by radix selection over a 16-bit value code (a monotone map of the logit
// that spreads the tokens over its bins), one byte per level, until the chosen
// bin holds few enough tokens to rank them directly in LDS; key levels over the
// 32-bit order keys take over only for bins of many equal or nearly equal
// logits.  The top-k levels count tokens; the top-p levels sum the float32
// weights exactly, as integers in units of 2^-149, against the exact threshold
// ceil(top_p x total).  For a small top-k, the survivors come instead from the
// few candidates that can make it, ranked directly, and top-p then cuts that
// ranked list.  Equal keys have equal weights; a cut inside a group of equal
// keys is the n-th of them in token order.
// --------------------------------------------------------------------------
// NPT > 0: V <= NPT NT and every thread keeps its NPT (key, weight) pairs in
// registers after the first read; NPT = 0: KL: the keys are kept in LDS (V <=
// kKlMaxV), else the logits are re-read on every pass.  With NPT = 0 the weights
// are formed once, in the pass that does the first top-p level (or sums the kept
// weights), and kept for the later passes: in LDS in place of the keys (KL; the
// few keys still needed afterwards are formed again from the logits), else in the
// output row.
// Rows are launched in order of their cost, so that the rows still starting as
// the grid drains are short ones.  The filter settings decide a row's cost: a
// radix top-p cut (most), then a full pass without top-p (or with a long top-k),
// a short ranked top-k list with top-p, without it, and greedy (least).
template <int NT>
__device__ __forceinline__ int cost_class(int r, int V, const float* __restrict__ temperature,
                                          const int* __restrict__ top_k, const float* __restrict__ top_p) {
  const float t = temperature[r], p = top_p[r];
  const int k = top_k[r];
  if (!(t > 0.0f) || k == 1 || p <= 0.0f) return 4;
  if (p < 1.0f) return (k > 1 && k < V && k <= NT) ? 2 : 0;
  return (k > 1 && k < V && k <= kFastK) ? 3 : 1;
}

// Up to NT requests: the k-th row of all requests' rows in cost order (the
// requests of one class, and each request's rows, keep their order).  A request
// whose status or tree size is invalid has one row.  Sets (b, i) and returns
// true, or returns false for k past the last row.
template <int NT>
__device__ __forceinline__ bool row_by_cost(int k, int B, int V, int T_max, const int* __restrict__ tree_size,
                                            const int* __restrict__ status, const float* __restrict__ temperature,
                                            const int* __restrict__ top_k, const float* __restrict__ top_p,
                                            int& b, int& i) {
  constexpr int NW = NT / 64;
  __shared__ int s_sc[NW], s_b, s_i;
  const int tid = threadIdx.x;
  int c_r = 5, n_r = 0;
  if (tid < B) {
    c_r = cost_class<NT>(tid, V, temperature, top_k, top_p);
    const int T = tree_size[tid];
    n_r = ((status && status[tid] != TV_ST_OK) || T < 1 || T > T_max) ? 1 : T;
  }
  int first = 0, rows = 0;  // this request's first row in the order; all rows
  for (int c = 0; c < 5; ++c) {
    int lo, hi, tot;
    block_scan<int, NT>(c_r == c ? n_r : 0, s_sc, lo, hi, tot);
    first += c < c_r ? tot : (c == c_r ? lo : 0);
    rows += tot;
  }
  if (k >= rows) return false;
  if (tid < B && first <= k && k < first + n_r) {
    s_b = tid;
    s_i = k - first;
  }
  __syncthreads();
  b = __builtin_amdgcn_readfirstlane(s_b);
  i = __builtin_amdgcn_readfirstlane(s_i);
  return true;
}

// The same for up to 64 requests on each wavefront alone (lane r holds request
// r; the five class totals and prefixes are DPP scans over the lanes), so a
// workgroup finds its row without a barrier: the workgroup-wide scans of
// row_by_cost took ~4.7 us of every row's workgroup (measured, 2410 rows).
template <int NT>
__device__ __forceinline__ bool row_by_cost_wave(int k, int B, int V, int T_max, const int* __restrict__ tree_size,
                                                 const int* __restrict__ status,
                                                 const float* __restrict__ temperature,
                                                 const int* __restrict__ top_k, const float* __restrict__ top_p,
                                                 int& b, int& i) {
  const int lane = threadIdx.x & 63;
  int c_r = 5, n_r = 0;
  if (lane < B) {
    c_r = cost_class<NT>(lane, V, temperature, top_k, top_p);
    const int T = tree_size[lane];
    n_r = ((status && status[lane] != TV_ST_OK) || T < 1 || T > T_max) ? 1 : T;
  }
  int first = 0, rows = 0;
#pragma unroll
  for (int c = 0; c < 5; ++c) {
    const int v = c_r == c ? n_r : 0;
    const int incl = wave_incl_scan_dpp(v);
    const int tot = __builtin_amdgcn_readlane(incl, 63);
    first += c < c_r ? tot : (c == c_r ? incl - v : 0);
    rows += tot;
  }
  if (k >= rows) return false;
  const unsigned long long m = __ballot(lane < B && first <= k && k < first + n_r);
  const int bsel = __ffsll((long long)m) - 1;
  b = bsel;
  i = k - __builtin_amdgcn_readlane(first, bsel);
  return true;
}

// More than NT requests: the y-th request in cost order.
template <int NT>
__device__ __forceinline__ int request_by_cost(int y, int B, int V, const float* __restrict__ temperature,
                                               const int* __restrict__ top_k, const float* __restrict__ top_p) {
  constexpr int NW = NT / 64;
  __shared__ int s_cc[5], s_wc[NW], s_req;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  auto cls = [&](int r) { return cost_class<NT>(r, V, temperature, top_k, top_p); };
  if (tid < 5) s_cc[tid] = 0;
  __syncthreads();
  for (int r = tid; r < B; r += NT) atomicAdd(&s_cc[cls(r)], 1);
  __syncthreads();
  int c = 0, base = 0;
  while (c < 4 && y >= base + s_cc[c]) base += s_cc[c++];
  const int pos = y - base;  // the request's place among those of class c
  int seen = 0;
  for (int r0 = 0; r0 < B; r0 += NT) {
    const int r = r0 + tid;
    const bool f = r < B && cls(r) == c;
    const unsigned long long bal = __ballot(f);
    if (lane == 0) s_wc[wave] = __popcll(bal);
    __syncthreads();
    int before = 0, tot = 0;
    for (int w = 0; w < NW; ++w) {
      before += w < wave ? s_wc[w] : 0;
      tot += s_wc[w];
    }
    if (f && seen + before + __popcll(bal & ((1ull << lane) - 1ull)) == pos) s_req = r;
    seen += tot;
    __syncthreads();
  }
  return s_req;
}

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
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // grid (T_max * B): one block per row, rows in cost order; grid (T_max, B):
  // block (i, y) takes row i of the y-th request in cost order
  int i = blockIdx.x, b = 0;
  if ((int)gridDim.x > T_max) {
    const int Bq = (int)gridDim.x / T_max;
    if (Bq <= 64 ? !row_by_cost_wave<NT>(blockIdx.x, Bq, V, T_max, tree_size, status, temperature, top_k, top_p, b, i)
                 : !row_by_cost<NT>(blockIdx.x, Bq, V, T_max, tree_size, status, temperature, top_k, top_p, b, i))
      return;
  } else if (gridDim.y > 1) {
    b = uni(request_by_cost<NT>(blockIdx.y, (int)gridDim.y, V, temperature, top_k, top_p));
  }
  int T = tree_size[b];
  if ((status && status[b] != TV_ST_OK) || T < 1 || T > T_max) T = 1;
  if (i >= T) return;
  const float* lr = logits + ((long long)b * T_max + i) * V;
  float* orow = probs + ((long long)b * T_max + i) * V;
  // keys in LDS, rows of a multiple of 4 tokens on 16-byte boundaries: every pass
  // over the row takes four consecutive tokens per visit (16-byte loads and stores)
  const bool q4 = KL && (V & 3) == 0 && !((reinterpret_cast<uintptr_t>(lr) | reinterpret_cast<uintptr_t>(orow)) & 15);
  __shared__ double s_d[NW * 16];
  __shared__ unsigned long long s_u[NW];
  __shared__ Wide s_w[NW];
  // radix bins (counts: CSETS sets of 256, shared by the wavefronts w % CSETS; or
  // up to 1024 words of weight sums), ballot entries (V / 64), or gathered tokens
  constexpr int CSETS = KL ? 4 : NW;
  constexpr int HIST = KL ? 1536 : 4096;
  __shared__ unsigned long long s_hist[HIST];
  static_assert(CSETS * 256 <= HIST && 1024 <= HIST && NT <= HIST && (!KL || kKlMaxV / 64 <= HIST),
                "radix bins, gathered tokens and ballot entries fit");
  __shared__ Norm s_abv, s_thr, s_kept, s_nw[NW];
  __shared__ unsigned long long s_top[NT];  // ranked tokens, best first
  __shared__ unsigned long long s_abvc;
  __shared__ int s_pick, s_sel, s_cnt, s_fsel;
  __shared__ uint32_t s_kc;
  extern __shared__ __align__(16) uint32_t s_key[];  // KL: the order key of token v
  static_assert(!KL || (NPT == 0 && NT == 1024), "keys in LDS: 1024 threads, no register copy");
  __shared__ double s_exp2[64];  // 2^(j / 64) (visible after the first barrier below)
  if (tid < 64) s_exp2[tid] = exp2((double)tid * 0.015625);

  // a token's 64-bit rank key (key, then token ascending; the larger ranks first)
  auto tok_key = [](uint32_t k, int v) { return ((unsigned long long)k << 32) | (0xFFFFFFFFu - (uint32_t)v); };
  // the first-ranked token, and the smallest key of a finite logit
  struct KW {
    uint32_t k;
    float w;
  };
  KW reg[NPT > 0 ? NPT : 1];
  auto ld_l = [&](int v) { return lr[v]; };
  unsigned long long best = 0ull;
  uint32_t kmin = 0xFFFFFFFFu;
  constexpr uint32_t kNegInfKey = 0x007FFFFFu;  // the order key of -inf
  auto see = [&](uint32_t k, int v) {
    best = umax64(best, tok_key(k, v));
    if (k > kNegInfKey) kmin = min(kmin, k);
  };
  if constexpr (NPT > 0) {
    float x[NPT];
#pragma unroll
    for (int j = 0; j < NPT; ++j) x[j] = lr[min(tid + j * NT, V - 1)];
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      reg[j].k = logit_key(x[j]);
      if (tid + j * NT < V) see(reg[j].k, tid + j * NT);
    }
  } else if constexpr (KL) {
    // the whole row in flight at once (up to kKlMaxV / NT = 32 tokens per thread)
    constexpr int J = kKlMaxV / NT;
    // this thread's tokens come in increasing v, so its first-ranked token is the
    // first one of the largest key (only a strictly larger key replaces it); the
    // smallest finite key is tracked as k - (key(-inf) + 1), which wraps the key
    // of -inf to the top
    uint32_t bk = 0u, kf = 0xFFFFFFFFu;
    int bv = 0;
    auto take = [&](int v, float xv) __attribute__((always_inline)) {
      const uint32_t k = logit_key(xv);
      s_key[v] = k;  // (the later passes read it after the workgroup maxima's barrier)
      if (k > bk) {
        bk = k;
        bv = v;
      }
      kf = min(kf, k - (kNegInfKey + 1u));
    };
    if (q4) {
      // 16-byte loads: thread t takes tokens 4 (t + j NT) .. + 3
      const f32x4* l4 = reinterpret_cast<const f32x4*>(lr);
      f32x4 x4[J / 4];
#pragma unroll
      for (int j = 0; j < J / 4; ++j)
        x4[j] = tid + j * NT < (V >> 2) ? l4[tid + j * NT] : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int j = 0; j < J / 4; ++j) {
        const int v = 4 * (tid + j * NT);
        if (v < V) {
#pragma unroll
          for (int e = 0; e < 4; ++e) take(v + e, x4[j][e]);
        }
      }
    } else {
      float x[J];
#pragma unroll
      for (int j = 0; j < J; ++j) x[j] = tid + j * NT < V ? lr[tid + j * NT] : -INFINITY;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int v = tid + j * NT;
        if (v < V) take(v, x[j]);
      }
    }
    if (bk) best = tok_key(bk, bv);
    if (kf != 0xFFFFFFFFu) kmin = kf + (kNegInfKey + 1u);
  } else {
    row_pass<NT>(V, ld_l, [&](int v, float x) { see(logit_key(x), v); });
  }
  const unsigned long long best_own = best;  // this thread's first-ranked token (0: none)
  {
    unsigned long long nk = (unsigned long long)(~kmin);
    block_max2_u64<NT>(best, nk, s_hist);
    kmin = ~(uint32_t)nk;
  }
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
  // w = fp32(exp(d / tau)), d = l - l_max <= 0.  Fast path (a table-driven
  // exponential in the manner of Tang's method): t = d log2(e) / tau to within a
  // few ulps, 2^t = 2^(k / 64) 2^f with |f| <= 1/128, 2^(j / 64) from a table
  // and 2^f from its degree-4 Taylor polynomial: relative error below 2^-43.  The
  // float32 rounding of that double is the rounding of the exact value unless
  // the double lies within 2^16 ulps of a float32 rounding midpoint (about one
  // value in 4096), or the result would be subnormal; those take the exact path:
  // the quotient d / tau, then exp in double.
  const double c2 = (1.0 / dtau) * 1.4426950408889634;  // log2(e) / tau
  auto weight = [&](uint32_t key) -> float {
    if (key == kmax) return 1.0f;
    const double d = (double)key_float(key) - dmax;
    const double t = d * c2;
    if (t >= -125.0) {
      const double kf = rint(t * 64.0);
      const int ki = (int)kf;
      const double f = fma(kf, -0.015625, t);  // (exact)
      // (fused: a result within the error bound is all the check below needs)
      const double p = fma(f, fma(f, fma(f, fma(f, 0.009618129107628477, 0.05550410866482158), 0.24022650695910072),
                                  0.6931471805599453), 1.0);
      const double y = ldexp(s_exp2[ki & 63] * p, ki >> 6);
      const uint32_t lo = (uint32_t)__double_as_longlong(y) & 0x1FFFFFFFu;  // the bits float32 rounds away
      if (lo - 0x0FFF0000u > 0x20000u) return (float)y;
    }
    return (float)exp(d / dtau);
  };
  // Weights: with NPT > 0 formed once and kept in registers.  Otherwise a row
  // whose survivors are a short ranked list forms their weights per list entry;
  // any other row forms every survivor's weight once and stores it in the output
  // row, where the same thread reads it back (`stored`).
  if constexpr (NPT > 0) {
#pragma unroll
    for (int j = 0; j < NPT; ++j) reg[j].w = weight(reg[j].k);
  }
  bool stored = false;
  // KL: once the weights are formed, each token's LDS slot holds its weight
  // (float bits; 0 outside the top-k cut) in place of its key, so no pass after
  // that touches global memory but the output and the few keys still needed,
  // which come back from the logits (key_at)
  bool lw = false;
  auto key_at = [&](int v) { return logit_key(lr[v]); };
  auto wt = [&](uint32_t k, float w) -> float { return (NPT > 0 || stored) ? w : weight(k); };
  auto ld_k = [&](int v) { return KW{KL ? (lw ? key_at(v) : s_key[v]) : logit_key(lr[v]), 0.0f}; };
  // (only passes after the weight pass read weights: with KL they are in LDS)
  auto ld_kw = [&](int v) {
    if constexpr (KL) return KW{0u, __uint_as_float(s_key[v])};
    else return KW{logit_key(lr[v]), stored ? orow[v] : 0.0f};
  };
  // one pass over the row: body(v, KW) for this thread's tokens in increasing v;
  // pass_k leaves the weight out (0) where it is not in registers
  const u32x4* s_key4 = reinterpret_cast<const u32x4*>(s_key);
  auto pass = [&](auto body) __attribute__((always_inline)) {
    if constexpr (NPT > 0) {
#pragma unroll
      for (int j = 0; j < NPT; ++j)
        if (tid + j * NT < V) body(tid + j * NT, reg[j]);
    } else {
      if (KL && q4) {
        quad_pass<NT>(V >> 2, [&](int q) { return s_key4[q]; }, [&](int q, u32x4 u) {
#pragma unroll
          for (int e = 0; e < 4; ++e) body(4 * q + e, KW{0u, __uint_as_float(u[e])});
        });
      } else {
        row_pass<NT, true>(V, ld_kw, body);
      }
    }
  };
  auto pass_k = [&](auto body) __attribute__((always_inline)) {
    if constexpr (NPT > 0) {
#pragma unroll
      for (int j = 0; j < NPT; ++j)
        if (tid + j * NT < V) body(tid + j * NT, reg[j]);
    } else {
      if (KL && q4 && lw) {
        quad_pass<NT>(V >> 2, [&](int q) { return reinterpret_cast<const f32x4*>(lr)[q]; }, [&](int q, f32x4 x) {
#pragma unroll
          for (int e = 0; e < 4; ++e) body(4 * q + e, KW{logit_key(x[e]), 0.0f});
        });
      } else if (KL && q4) {
        quad_pass<NT>(V >> 2, [&](int q) { return s_key4[q]; }, [&](int q, u32x4 u) {
#pragma unroll
          for (int e = 0; e < 4; ++e) body(4 * q + e, KW{u[e], 0.0f});
        });
      } else {
        row_pass<NT, !KL>(V, ld_k, body);
      }
    }
  };
  const bool with_p = tp < 1.0f;

  // ---- value code: 16 bits, 65535 - floor((l_max - l) 65536 / range) clamped to
  // [0, 65535] and 65535 for the largest logit, in float32, where range spans the
  // finite logits (at most 104 temperatures: weights below that are 0).  Float
  // rounding is monotone, so a larger key never gets a smaller code: each code
  // holds a contiguous range of keys, and the codes spread the tokens by value
  // (the top byte of a key puts nearly all of them into two or three bins).
  const float fmax = key_float(kmax);
  const float range = fminf(fmax - key_float(kmin), 104.0f * tau);
  const float vinv = (range > 0.0f && range <= __FLT_MAX__) ? 65536.0f / range : 0.0f;
  auto vcode = [&](uint32_t k) -> uint32_t {
    if (k == kmax) return 65535u;
    const float d = (fmax - key_float(k)) * vinv;  // >= 0, or NaN (-> 0) from inf * 0
    return d < 65535.0f ? 65535u - (uint32_t)d : 0u;
  };

  // The n-th token (token order, n >= 1) with key t inside the top-k cut (tk, ck),
  // in one coalesced pass: for each slice of NT consecutive tokens, every
  // wavefront's ballot of its matching tokens goes to LDS, slice-major, so the
  // entries are in token order; the first wavefront then finds the entry holding
  // the n-th match (64 entries per lane at most, a scan over the lanes) and the
  // bit inside it.
  const int nsl = (V + NT - 1) / NT;  // <= 256 slices, <= 4096 entries
  auto nth_with_key = [&](uint32_t t, int n, uint32_t tk, int ck) -> int {
    auto body = [&](int j, uint32_t k) __attribute__((always_inline)) {
      const int v = j * NT + tid;
      const bool f = v < V && k == t && (k > tk || v <= ck);
      const unsigned long long m = __ballot(f);
      if (lane == 0) s_hist[j * NW + wave] = m;
    };
    if (tid == 0) s_pick = V;
    if constexpr (NPT > 0) {
#pragma unroll
      for (int j = 0; j < NPT; ++j)
        if (j < nsl) body(j, reg[j].k);
    } else {
      for (int j0 = 0; j0 < nsl; j0 += kNB) {
        KW x[kNB];
#pragma unroll
        for (int jj = 0; jj < kNB; ++jj) x[jj] = ld_k(min((j0 + jj) * NT + tid, V - 1));
#pragma unroll
        for (int jj = 0; jj < kNB; ++jj)
          if (j0 + jj < nsl) body(j0 + jj, x[jj].k);
      }
    }
    __syncthreads();
    if (wave == 0) {
      const int ne = nsl * NW;
      const int per = (ne + 63) / 64;
      const int e0 = min(ne, lane * per), e1 = min(ne, e0 + per);
      int c = 0;
      for (int e = e0; e < e1; ++e) c += __popcll(s_hist[e]);
      const int incl = wave_incl_scan_dpp(c);
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
    const int res = uni(s_pick);
    __syncthreads();
    return res;
  };

  // ---- radix selection by counts (top-k), eight bits per level.  A level counts
  // the tokens with in_level(k, v) into 256 bins of digit(k) (LDS integer atomics),
  // then the first wavefront places the target among the bins (four bins per
  // lane, a suffix sum over the lanes) and the highest digit at which above + the
  // count of that digit and every higher one reaches the target is chosen (-1:
  // never); above gains the count of the higher digits.
  auto count_level = [&](int target, int& above, auto visit, auto digit) -> int {
    for (int e = tid; e < CSETS * 256; e += NT) s_hist[e] = 0ull;
    __syncthreads();
    visit([&](uint32_t k) { atomicAdd(&s_hist[(wave % CSETS) * 256 + digit(k)], 1ull); });
    __syncthreads();
    if (wave == 0) {
      unsigned long long m[4], g = 0ull;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        m[j] = 0ull;
        for (int w = 0; w < CSETS; ++w) m[j] += s_hist[w * 256 + 4 * lane + j];
        g += m[j];
      }
      // the higher lanes' bins: the wavefront's total less the inclusive prefix
      const unsigned long long inc = wave_scan_dpp(g, [](unsigned long long a, unsigned long long b) { return a + b; });
      unsigned long long run = (unsigned long long)above + (readlane_u64(inc, 63) - inc);
      int cand = -1;
      unsigned long long cabove = 0ull;
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        if (cand < 0 && run + m[j] >= (unsigned long long)target) {
          cand = 4 * lane + j;
          cabove = run;
        }
        run += m[j];
      }
      const unsigned long long hit = __ballot(cand >= 0);
      if (lane == 0) s_sel = -1;
      if (hit && lane == 63 - __builtin_clzll(hit)) {  // the highest digit that reaches the target
        s_sel = cand;
        s_abvc = cabove;
      }
    }
    __syncthreads();
    const int sel = uni(s_sel);
    if (sel >= 0) above = uni((int)s_abvc);
    __syncthreads();
    return sel;
  };
  // Gathers the tokens with f(k, v, w) into s_hist as rank keys (in any order)
  // and returns their number; entries past cap (<= HIST) are dropped.  w is the
  // stored weight once the weights are stored (else 0, or the register copy).
  // by_w (KL, once the weights are in LDS): the gathered entries rank by weight,
  // then token, instead of by key, then token
  bool by_w = false;
  auto gather = [&](int cap, auto f) -> int {
    if (tid == 0) s_cnt = 0;
    __syncthreads();
    auto body = [&](int v, KW e) {
      if (f(e.k, v, e.w)) {
        const int pos = atomicAdd(&s_cnt, 1);
        if (pos < cap) s_hist[pos] = tok_key(lw ? (by_w ? __float_as_uint(e.w) : key_at(v)) : e.k, v);
      }
    };
    if (stored) {
      pass(body);
    } else {
      pass_k(body);
    }
    __syncthreads();
    const int m = uni(s_cnt);
    __syncthreads();
    return m;
  };
  // Ranks the m (<= HIST) distinct rank keys of s_hist by counting the larger
  // ones: the first nkeep (<= NT) go in rank order into s_top.  With the keys in
  // LDS and m <= NT / 2, each entry has G = 2..16 adjacent lanes, each counting
  // every G-th entry, and the G counts are added by lane exchanges.
  auto rank_into_top = [&](int m, int nkeep) {
    auto by_one = [&]() {
      for (int t = tid; t < m; t += NT) {
        const unsigned long long my = s_hist[t];
        int rk = 0;
        for (int o = 0; o < m; ++o) rk += s_hist[o] > my;  // (all lanes read the same entry)
        if (rk < nkeep) s_top[rk] = my;
      }
    };
    if constexpr (KL) {
      int G = 1;
      while (G < 16 && m * G * 2 <= NT) G *= 2;
      if (G == 1) {
        by_one();
      } else {
        const int t = tid / G, q = tid % G;  // (m G <= NT: every entry has its lanes)
        const unsigned long long my = t < m ? s_hist[t] : 0ull;
        int rk = 0;
        if (t < m)
          for (int o = q; o < m; o += G) rk += s_hist[o] > my;
        for (int off = 1; off < G; off <<= 1) rk += __shfl_xor(rk, off, 64);  // (G divides 64)
        if (t < m && q == 0 && rk < nkeep) s_top[rk] = my;
      }
    } else {
      by_one();  // (the other variants keep their registers for their own passes)
    }
    __syncthreads();
  };
  // s_top[0..n) in rank order (n <= NT): the first index at which above + the
  // exact inclusive cumulative weight reaches thr (n if none), with that
  // cumulative in `kept`; a lane scan, then the totals of the earlier wavefronts.
  // own_total: thr = ceil(top_p x the list's total) instead (above = 0).
  // Only the wavefronts up to the one holding entry n take part in the sums.
  auto list_cut = [&](int n, const Norm& above, const Norm& thr, bool own_total, Norm& kept) -> int {
    const bool act = wave * 64 <= n;  // (wave-uniform)
    Wide incl = wzero();
    if (act) {
      if (tid < n) incl = wide_of(weight((uint32_t)(s_top[tid] >> 32)));
      // (inclusive prefix of every limb over the lanes, by DPP moves)
#pragma unroll
      for (int i2 = 0; i2 < NL; ++i2)
        incl.l[i2] = wave_scan_dpp(incl.l[i2], [](unsigned long long a, unsigned long long b) { return a + b; });
      if (lane == 63) s_w[wave] = incl;
    }
    if (tid == 0) s_pick = n;
    __syncthreads();
    Norm c = nzero();
    if (act) {
      for (int w = 0; w < wave; ++w) wadd(incl, s_w[w]);
      c = nadd(norm_of(incl), above);
    }
    Norm th = thr;
    if (own_total) {
      if (tid == n - 1) s_thr = nthreshold(tp, c);
      __syncthreads();
      th = nuniform(s_thr);
    }
    if (tid < n && nge(c, th)) atomicMin(&s_pick, tid);
    __syncthreads();
    const int cut = uni(s_pick);
    if (tid == cut) s_kept = c;
    __syncthreads();
    kept = nuniform(s_kept);
    __syncthreads();
    return cut;
  };

  // ---- top-k cut (tk, ck): token v with key k survives iff k > tk or (k == tk
  // and v <= ck); the default keeps everything (every key is > 0)
  uint32_t tk = 0u;
  int ck = V;
  // top-p over at most NT top-k survivors ranks them all in s_top
  const bool listed = with_p && kk > 1 && kk < V && kk <= NT;
  // Fast path, 1 < top_k <= kFastK: take c, the top_k-th largest value code
  // among the per-thread best tokens (distinct tokens, so at least top_k tokens
  // reach c and the top_k survivors all do: codes are monotone).  The tokens whose
  // code reaches c, usually a few more than top_k, are gathered into LDS and
  // ranked exactly by counting, which leaves the survivors in rank order in s_top.
  // With more candidates than the list holds, the general path below runs instead.
  bool sorted = false;
  if (kk > 1 && kk <= kFastK && kk < V) {
    const unsigned long long tm = best_own;  // this thread's best token as a rank key (the first pass's)
    // a thread without tokens has tm = 0: key 0, below every token's key, code 0
    const uint32_t mc = tm ? vcode((uint32_t)(tm >> 32)) : 0u;
    int above_t = 0;
    const uint32_t ch = (uint32_t)max(0, count_level(kk, above_t, [&](auto f) { f(mc); },
                                                     [](uint32_t c) { return c >> 8; }));
    const uint32_t c_k =
        (ch << 8) | (uint32_t)max(0, count_level(kk, above_t, [&](auto f) { if ((mc >> 8) == ch) f(mc); },
                                                 [](uint32_t c) { return c & 255u; }));
    // the tokens whose code reaches c_k are those whose key reaches k_c, the
    // smallest key with that code (codes grow with the key over [key(-inf), kmax],
    // which holds every token's key): a 64-way search on each wavefront's lanes,
    // the same in every wavefront, then one comparison per token
    uint32_t k_c = kNegInfKey;
    // (keys in LDS: the first wavefront searches and the others take k_c from
    // LDS; the other variants search on every wavefront, the same value)
    if (!KL || wave == 0) {
      if (vcode(k_c) < c_k) {
        uint32_t lo = k_c, hi = kmax;  // vcode(lo) < c_k <= vcode(hi)
        while (hi - lo > 1u) {
          const unsigned long long step = ((unsigned long long)(hi - lo) + 63ull) / 64ull;
          const uint32_t p = (uint32_t)min((unsigned long long)lo + step * (unsigned long long)(lane + 1),
                                           (unsigned long long)hi);
          const unsigned long long ok = __ballot(vcode(p) >= c_k);  // (lane 63 probes hi)
          const int f = __ffsll((long long)ok) - 1;
          const uint32_t nh = (uint32_t)__builtin_amdgcn_readlane((int)p, f);
          lo = f ? (uint32_t)__builtin_amdgcn_readlane((int)p, f - 1) : lo;
          hi = nh;
        }
        k_c = hi;
      }
    }
    if constexpr (KL) {
      if (tid == 0) s_kc = k_c;
      __syncthreads();
      k_c = s_kc;
    }
    const int m = gather(HIST, [&](uint32_t k, int, float) { return k >= k_c; });
    if (m <= HIST) {
      rank_into_top(m, kk);
      const unsigned long long last = uni(s_top[kk - 1]);
      tk = (uint32_t)(last >> 32);
      ck = (int)key_index(last);
      sorted = true;
    }
  }
  if (!sorted && kk > 1 && kk < V) {
    // Value levels: the high byte of the code over every token, then the low byte
    // inside the chosen high byte; the tokens of the chosen bin are ranked
    // directly when at most NT, else key levels run inside the chosen code.
    int above = 0;
    auto all = [&](auto f) { pass_k([&](int, KW e) { f(e.k); }); };
    const uint32_t hs = (uint32_t)count_level(kk, above, all, [&](uint32_t k) { return vcode(k) >> 8; });
    uint32_t code = 0u;
    int m = gather(NT, [&](uint32_t k, int, float) { return (vcode(k) >> 8) == hs; });
    if (m > NT) {
      auto in_hs = [&](auto f) { pass_k([&](int, KW e) { if ((vcode(e.k) >> 8) == hs) f(e.k); }); };
      code = (hs << 8) | (uint32_t)count_level(kk, above, in_hs, [&](uint32_t k) { return vcode(k) & 255u; });
      m = gather(NT, [&](uint32_t k, int, float) { return vcode(k) == code; });
    }
    if (m <= NT) {
      // the (kk - above)-th ranked of the bin's m tokens is the last survivor
      const int n = kk - above;
      for (int t = tid; t < m; t += NT) {
        const unsigned long long my = s_hist[t];
        int rk = 0;
        for (int o = 0; o < m; ++o) rk += s_hist[o] > my;
        if (rk == n - 1) s_abvc = my;
      }
      __syncthreads();
      const unsigned long long lastk = uni(s_abvc);
      tk = (uint32_t)(lastk >> 32);
      ck = (int)key_index(lastk);
      __syncthreads();
    } else {
      // key levels over the tokens of the code, then the cut inside the equal keys
      uint32_t prefix = 0u;
      for (int shift = 24; shift >= 0; shift -= 8) {
        const uint32_t pmask = shift == 24 ? 0u : (0xFFFFFFFFu << (shift + 8));
        auto in_code = [&](auto f) {
          pass_k([&](int, KW e) { if (vcode(e.k) == code && (e.k & pmask) == prefix) f(e.k); });
        };
        prefix |= (uint32_t)max(count_level(kk, above, in_code, [&](uint32_t k) { return (k >> shift) & 255u; }), 0)
                  << shift;
      }
      tk = prefix;
      ck = nth_with_key(tk, kk - above, 0u, V);
    }
    if (listed) {
      // all kk survivors, ranked
      const int n = min(NT, gather(NT, [&](uint32_t k, int v, float) { return k > tk || (k == tk && v <= ck); }));
      rank_into_top(n, n);  // (n = kk)
    }
  }
  auto in_k = [&](uint32_t k, int v) { return k > tk || (k == tk && v <= ck); };
  // the survivors are s_top[0..kk) (a small top-k) or are described by the cut
  const bool as_list = sorted || listed;
  if (as_list) {
    // The output row of a list is 0 but for the kept entries: every token 0 now
    // (16-byte stores where the row allows), so that the stores drain while the
    // cut and the kept total are worked out; the kept entries follow at the end.
    if (!(reinterpret_cast<uintptr_t>(orow) & 15)) {
      const float4 z = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      for (int v4 = tid; v4 < (V >> 2); v4 += NT) reinterpret_cast<float4*>(orow)[v4] = z;
      for (int v = (V & ~3) + tid; v < V; v += NT) orow[v] = 0.0f;
    } else {
      for (int v = tid; v < V; v += NT) orow[v] = 0.0f;
    }
  }

  // ---- top-p radix, by the float32 bits u of the survivors' weights (w grows
  // with the key, so the bits order the tokens as the keys do, up to equal
  // weights).  Level 0 bins by u >> 20 (the exponent and 3 mantissa bits, 1024
  // bins), level 1 by the next 8 bits, level 2 by the next 8, level 3 by the
  // last 4.  Every token of a bin has the same exponent, so a bin's exact weight
  // is (the sum of the 24-bit mantissas m) 2^s units: one 64-bit word per bin
  // holds the sum of (m + 2^44), i.e. the mantissa sum (< 2^42: a row has fewer
  // than 2^18 tokens) and, above bit 44, the count, with one atomic per token.
  constexpr unsigned long long kCnt1 = 1ull << 44;
  auto lev_shift = [](int lev) { return lev == 0 ? 20 : lev == 1 ? 12 : lev == 2 ? 4 : 0; };
  auto lev_bins = [](int lev) { return lev == 0 ? 1024 : lev == 3 ? 16 : 256; };
  auto w_word = [](float w) {  // m + 2^44 for a weight w > 0
    const uint32_t u = __float_as_uint(w);
    return ((u >> 23) ? (unsigned long long)((u & 0x7FFFFFu) | 0x800000u) : (unsigned long long)u) + kCnt1;
  };
  Norm above = nzero(), thr = nzero();
  // After a level's sums (the bins of one exponent e, or, at level 0, bin b of
  // exponent b >> 3), every thread takes nb / NT (at least one) consecutive bins:
  // an exact suffix sum over the threads (a lane scan, then the wavefront totals)
  // gives each the weight of all higher bins, and the one bin at which above +
  // that weight first reaches thr is chosen (-1: never), with its count in
  // s_cnt.  `above` gains the weight of the higher bins; level 0 sets thr from
  // the total.
  // The sums run on the first WT threads (the same exact integers whichever
  // threads add them; fewer wavefronts issue fewer of the wide additions).
  constexpr int WT = NT < 256 ? NT : 256, WW = WT / 64;
  auto w_select = [&](int lev, uint32_t prefix) __attribute__((always_inline)) -> int {
    const int nb = lev_bins(lev);
    const int bpt = (nb + WT - 1) / WT;  // 4 at level 0 (1024 bins), else 1
    const bool part = tid < WT;          // (wave-uniform)
    const int e_fix = lev == 1 ? (int)(prefix >> 3) : lev == 2 ? (int)(prefix >> 11) : (int)(prefix >> 19);
    auto bin_at = [&](int bin) {  // the bin's weight as a Wide (0 past the bins)
      const unsigned long long word = bin < nb ? s_hist[bin] : 0ull;
      const int e = lev == 0 ? (bin >> 3) : e_fix;
      return wide_shifted(word & (kCnt1 - 1), e ? e - 1 : 0);
    };
    if (tid == 0) s_sel = -1;
    __syncthreads();
    // carry-save sums: a bin's limbs are below 2^46, so 1024 of them fit a limb
    Wide run = wzero();
    if (part) {
      Wide own = wzero();
#pragma unroll 1
      for (int j = 0; j < bpt; ++j) wadd(own, bin_at(tid * bpt + j));
      // limb by limb: the inclusive prefix over the lanes (DPP moves) and the
      // wavefront's total; the higher lanes' bins are their difference (exact:
      // each limb of a prefix is at most that limb of the total)
      Wide inc, tot;
#pragma unroll
      for (int l = 0; l < NL; ++l) {
        inc.l[l] = wave_scan_dpp(own.l[l], [](unsigned long long a, unsigned long long b) { return a + b; });
        tot.l[l] = readlane_u64(inc.l[l], 63);
      }
      run = wsub(tot, inc);  // the higher lanes' bins
      if (lane == 0) s_w[wave] = tot;
    }
    __syncthreads();
    if (part) {
      for (int w = wave + 1; w < WW; ++w) wadd(run, s_w[w]);  // the higher wavefronts' bins
    }
    if (lev == 0 && tid == 0) {  // thr from the total
      Wide z = wzero();
      for (int w = 0; w < WW; ++w) wadd(z, s_w[w]);
      s_thr = nthreshold(tp, norm_of(z));
    }
    if (lev == 0) __syncthreads();
    const Norm th = lev == 0 ? nuniform(s_thr) : thr;
    if (part) {
#pragma unroll 1
      for (int j = bpt - 1; j >= 0; --j) {
        const int bin = tid * bpt + j;
        const Norm r0 = nadd(norm_of(run), above);
        wadd(run, bin_at(bin));
        const Norm r2 = nadd(norm_of(run), above);
        if (bin < nb && !nge(r0, th) && nge(r2, th)) {  // the one bin where the cumulative crosses thr
          s_sel = bin;
          s_abv = r0;
          s_cnt = (int)(s_hist[bin] >> 44);
        }
      }
    }
    __syncthreads();
    const int sel = uni(s_sel);
    if (sel >= 0) above = nuniform(s_abv);
    thr = th;
    __syncthreads();
    return sel;
  };

  // Level 0 decided by float64 sums first.  A bin's weight (its mantissa sum,
  // < 2^42, times 2^(e - 1) units) is exact in float64; the suffix sums over the
  // bins (4 per thread on the first WT threads, a lane scan, then the wavefront
  // totals) and the threshold top_p x total take at most ~25 roundings of
  // non-negative terms, so each is within total x 2^-48 of its exact value.  A
  // bin whose cumulative before it is below the threshold and after it above it
  // by more than total x 2^-40 on both sides is therefore the exact crossing.
  // Only that bin's exact "above" and the exact threshold are then formed (two
  // workgroup sums of Wide).  Returns -2 when no bin clears the margin (a
  // crossing within it, or none at all): the exact w_select decides then.
  auto w_select0_fast = [&]() -> int {
    const bool part = tid < WT;  // (wave-uniform)
    __syncthreads();  // the bins' sums are complete
    if (tid == 0) s_fsel = -1;
    unsigned long long ms[4];
    double dv[4];
    double S = 0.0;
    // the first WT threads: bins 4 tid .. 4 tid + 3, one exponent e = tid / 2
    const int e = tid >> 1, sx = e ? e - 1 : 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ms[j] = part ? (s_hist[4 * tid + j] & (kCnt1 - 1)) : 0ull;
      dv[j] = ldexp((double)ms[j], sx);
      S += dv[j];
    }
    // inclusive prefix over the lanes by DPP moves (as wave_reduce_dpp), then the
    // wavefront totals: the bins above this thread's = total - prefix
    unsigned long long x = (unsigned long long)__double_as_longlong(S);
    auto addd = [](unsigned long long a, unsigned long long b) {
      return (unsigned long long)__double_as_longlong(__longlong_as_double((long long)a) +
                                                      __longlong_as_double((long long)b));
    };
    x = addd(x, dpp_u64<0x111, 0xF>(x));
    x = addd(x, dpp_u64<0x112, 0xF>(x));
    x = addd(x, dpp_u64<0x114, 0xF>(x));
    x = addd(x, dpp_u64<0x118, 0xF>(x));
    x = addd(x, dpp_u64<0x142, 0xA>(x));
    x = addd(x, dpp_u64<0x143, 0xC>(x));
    const double incl = __longlong_as_double((long long)x);
    if (lane == 63 && part) s_d[wave] = incl;  // the wavefront's total
    __syncthreads();
    double tot = 0.0, above_w = 0.0;
    for (int w = 0; w < WW; ++w) {
      const double v = s_d[w];
      tot += v;
      if (w > wave) above_w += v;
    }
    const double thr_d = (double)tp * tot;
    const double marg = tot * 0x1p-40;
    if (part) {
      double r = (s_d[wave] - incl) + above_w;  // every bin above this thread's
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        const double r0 = r;
        r += dv[j];
        if (r0 + marg < thr_d && r - marg >= thr_d) s_fsel = 4 * tid + j;  // (at most one)
      }
    }
    __syncthreads();
    const int sel = uni(s_fsel);
    if (sel < 0) return -2;
    // exact: the bins above sel and all bins, as carry-save limbs summed by DPP
    // within each wavefront, then the wavefronts' limbs added in LDS
    if (part) {
      unsigned long long ma = 0ull, mz = 0ull;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        mz += ms[j];
        if (4 * tid + j > sel) ma += ms[j];
      }
      const Wide wa = wide_shifted(ma, sx), wz = wide_shifted(mz, sx);  // (mantissa sums < 2^44)
      auto addu = [](unsigned long long a, unsigned long long b) { return a + b; };
#pragma unroll
      for (int l = 0; l < NL; ++l) {
        const unsigned long long ta = wave_reduce_dpp(wa.l[l], addu);
        const unsigned long long tz = wave_reduce_dpp(wz.l[l], addu);
        if (lane == 0) {
          s_hist[1024 + wave * 2 * NL + l] = ta;
          s_hist[1024 + wave * 2 * NL + NL + l] = tz;
        }
      }
    }
    __syncthreads();
    if (tid == 0) {
      Wide wa = wzero(), wz = wzero();
      for (int w = 0; w < WW; ++w)
#pragma unroll
        for (int l = 0; l < NL; ++l) {
          wa.l[l] += s_hist[1024 + w * 2 * NL + l];
          wz.l[l] += s_hist[1024 + w * 2 * NL + NL + l];
        }
      s_abv = norm_of(wa);
      s_thr = nthreshold(tp, norm_of(wz));
      s_cnt = (int)(s_hist[sel] >> 44);
    }
    __syncthreads();
    above = nuniform(s_abv);
    thr = nuniform(s_thr);
    __syncthreads();
    return sel;
  };

  // ---- one pass forming every survivor's weight (unless they are a ranked
  // list): NPT = 0 stores it into the output row (0 for the others), and the pass
  // also does the first top-p level's sums or, without top-p, sums the kept weights
  double wsum = 0.0;
  if (!as_list) {
    if (with_p) {
      for (int e = tid; e < 1024; e += NT) s_hist[e] = 0ull;
      __syncthreads();
    }
    pass_k([&](int v, KW e) {
      const float w = in_k(e.k, v) ? wt(e.k, e.w) : 0.0f;
      if constexpr (KL) s_key[v] = __float_as_uint(w);  // (this thread's own slot, read just above)
      else if constexpr (NPT == 0) orow[v] = w;
      if (with_p) {
        if (w > 0.0f) atomicAdd(&s_hist[__float_as_uint(w) >> 20], w_word(w));
      } else if (!(mp > 0.0f) || w >= mp || v == tok0) {
        wsum += (double)w;
      }
    });
    stored = NPT == 0;  // later passes read the weights back (ld_kw): from LDS (KL) or the output row
    lw = KL;
  }

  // ---- top-p cut (tpk, cp) over the top-k survivors: the shortest rank prefix
  // whose exact cumulative weight c satisfies c >= top_p x total, i.e.
  // c >= thr = ceil(top_p x total) (c is an integer number of units).  kept: the
  // exact weight of the prefix, when the cut is found.
  uint32_t tpk = 0u;
  int cp = V;
  // KL: the cut by weight: a weight above w_cut stays, one below goes, and one
  // equal to it stays if tie_all (every token of that weight is inside the cut)
  // or its key is inside (tpk, cp)
  bool tie_all = false;
  float w_cut = 0.0f;
  int n_list = kk;  // the ranked survivors that stay (as_list)
  bool have_kept = false;
  Norm kept = nzero();
  if (listed) {
    const int cut = list_cut(kk, nzero(), nzero(), true, kept);
    if (cut < kk) n_list = cut + 1;
  } else if (with_p) {
    // levels until the chosen bin holds at most NT tokens, which are then ranked
    // in a list; a bin of more than NT equal weights at the last level is cut by
    // counting: n of its tokens, the first n in rank order
    uint32_t prefix = 0u;  // u >> (the last level's shift)
    int m = 0, sh = 20;
    bool reached = true;
#pragma unroll 1
    for (int lev = 0; lev < 4; ++lev) {
      if (lev > 0) {
        const int sh0 = sh, nb = lev_bins(lev);
        sh = lev_shift(lev);
        for (int e = tid; e < nb; e += NT) s_hist[e] = 0ull;
        __syncthreads();
        pass([&](int v, KW e) {
          const float w = KL ? e.w : (in_k(e.k, v) ? wt(e.k, e.w) : 0.0f);
          const uint32_t u = __float_as_uint(w);
          if (w > 0.0f && (u >> sh0) == prefix) atomicAdd(&s_hist[(u >> sh) & (nb - 1)], w_word(w));
        });
      }
      // (the float64 level 0 on the keys-in-LDS variant only: the others keep
      // their registers for their own passes)
      int sel = -2;
      if constexpr (KL) {
        if (lev == 0) sel = w_select0_fast();
      }
      if (sel == -2) sel = w_select(lev, prefix);
      if (sel < 0) {  // never reached: every survivor stays
        reached = false;
        break;
      }
      m = uni(s_cnt);
      prefix = lev == 0 ? (uint32_t)sel : (prefix << (lev == 3 ? 4 : 8)) | (uint32_t)sel;
      if (m <= NT) break;
    }
    if (reached && m <= NT) {
      __syncthreads();
      // KL: the bin's tokens are ranked by weight (w grows with the key, so only
      // equal weights may be out of key order: they are sorted out below when the
      // cut falls among them), and each entry carries its weight
      by_w = KL;
      gather(NT, [&](uint32_t k, int v, float w) {
        const float x = KL ? w : (in_k(k, v) ? wt(k, w) : 0.0f);
        return x > 0.0f && (__float_as_uint(x) >> sh) == prefix;
      });
      by_w = false;
      rank_into_top(m, m);
      // every weight of the bin is m_t 2^s units (one exponent): the cut is the
      // first rank whose inclusive mantissa sum reaches need = ceil((thr - above)
      // / 2^s) (< 2^43: the bin's total reaches thr)
      const uint32_t e = prefix >> (23 - sh);
      const int sx = e ? (int)e - 1 : 0;
      unsigned long long dt[NN + 1];
      long long br = 0;
#pragma unroll
      for (int i = 0; i < NN; ++i) {  // thr - above, borrows propagated
        const long long d = (long long)thr.l[i] - (long long)above.l[i] - br;
        br = d < 0 ? 1 : 0;
        dt[i] = (unsigned long long)(d + (br << 32));
      }
      dt[NN] = 0ull;
      const Norm nq = nshr_ceil(dt, sx);
      const unsigned long long need = ((unsigned long long)nq.l[1] << 32) | nq.l[0];
      unsigned long long mt = 0ull;
      if (tid < m) {
        const uint32_t u = KL ? (uint32_t)(s_top[tid] >> 32) : __float_as_uint(weight((uint32_t)(s_top[tid] >> 32)));
        mt = (u >> 23) ? ((u & 0x7FFFFFu) | 0x800000u) : u;
      }
      unsigned long long lo_c, hi_c, tot_c;
      block_scan<unsigned long long, NT>(mt, s_u, lo_c, hi_c, tot_c);
      if (tid == 0) s_pick = m;
      __syncthreads();
      if (tid < m && hi_c >= need && lo_c < need) s_pick = tid;  // (exactly one)
      __syncthreads();
      const int cut = uni(s_pick);
      if (cut < m) {
        if (tid == cut) s_kept = nadd(above, norm_of(wide_shifted(hi_c, sx)));
        __syncthreads();
        kept = nuniform(s_kept);
        const unsigned long long ck2 = uni(s_top[cut]);
        if constexpr (KL) {
          // the tokens of the cut's weight are entries first..last; the first
          // cut - first + 1 of them in key order stay
          const uint32_t uc = (uint32_t)(ck2 >> 32);
          w_cut = __uint_as_float(uc);
          if (tid == 0) {
            s_pick = m;
            s_sel = -1;
          }
          __syncthreads();
          if (tid < m && (uint32_t)(s_top[tid] >> 32) == uc) {
            atomicMin(&s_pick, tid);
            atomicMax(&s_sel, tid);
          }
          __syncthreads();
          const int first = uni(s_pick), last = uni(s_sel);
          const int n_t = cut - first + 1, g = last - first + 1;
          __syncthreads();
          tie_all = n_t == g;
          if (!tie_all) {
            // their keys, and the n_t-th of them in (key desc, token asc) order
            if (tid >= first && tid <= last) {
              const int v = (int)key_index(s_top[tid]);
              s_hist[tid - first] = tok_key(key_at(v), v);
            }
            __syncthreads();
            for (int t = tid; t < g; t += NT) {
              const unsigned long long my = s_hist[t];
              int rk = 0;
              for (int o = 0; o < g; ++o) rk += s_hist[o] > my;
              if (rk == n_t - 1) s_abvc = my;
            }
            __syncthreads();
            const unsigned long long lastk = uni(s_abvc);
            tpk = (uint32_t)(lastk >> 32);
            cp = (int)key_index(lastk);
            __syncthreads();
          } else {
            tpk = 1u;  // (a cut exists; equal weights need no key)
          }
        } else {
          tpk = (uint32_t)(ck2 >> 32);
          cp = (int)key_index(ck2);
        }
        have_kept = true;
      }
    } else if (reached) {
      // more than NT survivors of the one weight c = prefix: the first n of them in
      // rank order (n = ceil((thr - above) / c)) keep; key levels find the n-th
      // one's key
      const float c = __uint_as_float(prefix);
      const int n = ntie_count(thr, above, c);
      int ab = 0;
      uint32_t kp = 0u;
      for (int shift = 24; shift >= 0; shift -= 8) {
        const uint32_t pmask = shift == 24 ? 0u : (0xFFFFFFFFu << (shift + 8));
        auto in_c = [&](auto f) {
          pass([&](int v, KW e) {
            if constexpr (KL) {
              if (e.w == c) {  // (c > 0: inside the top-k cut)
                const uint32_t k = key_at(v);
                if ((k & pmask) == kp) f(k);
              }
            } else if (in_k(e.k, v) && wt(e.k, e.w) == c && (e.k & pmask) == kp) {
              f(e.k);
            }
          });
        };
        kp |= (uint32_t)max(count_level(n, ab, in_c, [&](uint32_t k) { return (k >> shift) & 255u; }), 0)
              << shift;
      }
      tpk = kp;
      cp = nth_with_key(tpk, n - ab, tk, ck);
    }
  }

  // ---- min-p, the kept total and the output.  The kept tokens are a rank prefix.
  if (as_list) {
    // s_top[0..n_list) ranked; min-p keeps the entries with w >= min_p (a prefix,
    // the first entry always): their exact total is W, and each kept entry is
    // written by its thread over the zero the row already holds.  The two stores
    // of a kept token come from different wavefronts: each thread waits until its
    // zero stores are done (in this CU's L2) before the barrier, which a
    // workgroup barrier alone does not do for global memory.
    // The total: limbs summed by DPP on the wavefronts holding entries, then
    // their sums in LDS (the barrier in between also orders the stores).
    const float w_t = tid < n_list ? weight((uint32_t)(s_top[tid] >> 32)) : 0.0f;
    const bool keep = tid < n_list && (!(mp > 0.0f) || w_t >= mp || tid == 0);
    const int nwl = (n_list + 63) >> 6;  // (n_list >= 1)
    if (wave < nwl) {
      Wide t = keep ? wide_of(w_t) : wzero();
#pragma unroll
      for (int l = 0; l < NL; ++l)
        t.l[l] = wave_reduce_dpp(t.l[l], [](unsigned long long a, unsigned long long b) { return a + b; });
      if (lane == 0) s_w[wave] = t;
    }
    __builtin_amdgcn_s_waitcnt(kVmemStoresDone);
    __syncthreads();
    Wide tw = wzero();
    for (int w = 0; w < nwl; ++w) wadd(tw, s_w[w]);
    const double W = norm_to_double(norm_of(tw));
    if (keep) orow[key_index(s_top[tid])] = (float)((double)w_t * (1.0 / W));
    return;
  }
  // KL: the top-p cut by weight: w grows with the key, so a weight above the
  // cut's ranks above it and one below ranks below; only equal weights may need
  // the key (tpk = 0: no cut).  A cut set by key alone takes the weight of its key.
  if (KL && tpk && w_cut == 0.0f) w_cut = weight(tpk);
  auto kept_w = [&](uint32_t k, int v, float w) -> float {
    if constexpr (KL) {
      if (!(w > 0.0f)) return 0.0f;  // (outside the top-k cut, or no weight)
      if (tpk && !(w > w_cut)) {
        if (w < w_cut) return 0.0f;
        if (!tie_all) {
          const uint32_t kv = key_at(v);
          if (!(kv > tpk || (kv == tpk && v <= cp))) return 0.0f;
        }
      }
      return (!(mp > 0.0f) || w >= mp || v == tok0) ? w : 0.0f;
    }
    if (!(in_k(k, v) && (k > tpk || (k == tpk && v <= cp)))) return 0.0f;
    const float x = wt(k, w);
    return (!(mp > 0.0f) || x >= mp || v == tok0) ? x : 0.0f;
  };
  double W;
  if (!with_p) {
    W = block_sum_d<NT>(wsum, s_d);
  } else if (have_kept && !(mp > 0.0f)) {
    W = norm_to_double(kept);
  } else {
    double ws = 0.0;
    pass([&](int v, KW e) { ws += (double)kept_w(e.k, v, e.w); });
    W = block_sum_d<NT>(ws, s_d);
  }
  // w / W as w (1 / W) in double: within one double rounding of the quotient
  const double rW = 1.0 / W;
  if (KL && q4) {
    quad_pass<NT>(V >> 2, [&](int q) { return s_key4[q]; }, [&](int q, u32x4 u) {
      f32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = kept_w(0u, 4 * q + e, __uint_as_float(u[e]));
        o[e] = x > 0.0f ? (float)((double)x * rW) : 0.0f;
      }
      reinterpret_cast<f32x4*>(orow)[q] = o;
    });
    return;
  }
  pass([&](int v, KW e) {
    const float x = kept_w(e.k, v, e.w);
    // (NPT = 0 without LDS weights: a token outside the top-k cut already holds 0)
    if (NPT > 0 || KL || x > 0.0f || in_k(e.k, v)) orow[v] = x > 0.0f ? (float)((double)x * rW) : 0.0f;
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
        // other threads read R next (the tests, the correction's ranges): every
        // store is done before the barrier below
        __builtin_amdgcn_s_waitcnt(kVmemStoresDone);
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
    // (a range of no width takes no target; should rounding leave two ranges
    // holding it, the larger token is taken)
    if (lo < hi && lo <= target && target < hi) {
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
      atomicMax(&s_pick, pick >= 0 ? pick : last);
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

// --------------------------------------------------------------------------
// tree_accept_sample_draft, sliced: S workgroups per request, workgroup s owning
// tokens [s L, min(V, (s + 1) L)) with its slice of R (float64) and Q (float32)
// in LDS, so that a pass over the residual streams through S CUs instead of
// one.  The workgroups of a request take the same walk: each computes every
// decision from the same values -- the slice sums, exchanged through the
// workspace and added in slice order, and R(x), Q(x) of the child's token,
// which each re-derives from p(x), q(x) by replaying the node's updates with
// the operations of the slice pass.  Exchange g uses its own slots in the
// workspace (4 words per workgroup, set to an empty mark by k_slice_reset):
// each workgroup stores its words and polls the others' until none is empty.
// Slots and marks are only touched by device-scope atomics, which are performed
// past the per-XCD caches, so no cache is written back or invalidated.  Every
// wait is bounded, and a request whose wait runs out gets accept_len =
// bonus_token = -1.  The host launches at most as many workgroups as the
// device holds at once, so all of a request's workgroups are resident together.
// --------------------------------------------------------------------------
constexpr int kSliceMax = 8;          // workgroups per request
constexpr int kSliceSpin = 1 << 22;   // polls of a slot before a wait gives up
constexpr unsigned long long kSlotEmpty = ~0ull;  // (no exchanged word is all ones)
// exchanges a walk makes at most: one per node entered (<= dcap + 1 <= T_max)
// and one per rejection (< T_max)
__host__ __device__ constexpr int slice_exchanges(int T_max) { return 2 * T_max; }

// slot words of request b: its workspace row, exchange-major, 4 words per slice
__global__ void k_slice_reset(double* __restrict__ ws, int V, int words) {
  unsigned long long* row = reinterpret_cast<unsigned long long*>(ws + (long long)blockIdx.x * V);
  for (int e = threadIdx.x; e < words; e += blockDim.x) row[e] = kSlotEmpty;
}

template <int NT>
__global__ __launch_bounds__(NT) void k_tree_accept_sample_draft_sliced(
    int S, int L, int T_max, int dcap, int V, int without_replacement, const int* __restrict__ draft_tokens,
    const int* __restrict__ parents, const int* __restrict__ tree_size, const float* __restrict__ target_probs,
    const float* __restrict__ draft_probs, const float* __restrict__ uniforms, const int* __restrict__ status,
    int* __restrict__ accept_len, int* __restrict__ accept_path, int* __restrict__ bonus_token,
    double* __restrict__ ws) {
#pragma clang fp contract(off)
  constexpr int NW = NT / 64;
  const int sl = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int v0 = sl * L, n = max(0, min(V, v0 + L) - v0);  // this slice: tokens v0 .. v0 + n - 1
  extern __shared__ double s_R[];                            // L residual values
  float* s_Q = reinterpret_cast<float*>(s_R + L);           // L draft values
  uint32_t* s_rm = reinterpret_cast<uint32_t*>(s_Q + L);    // (L + 31) / 32 words: removed tokens
  __shared__ int s_tok[kTMaxLimit], s_par[kTMaxLimit], s_path[kTMaxLimit], s_gc[kTMaxLimit];
  __shared__ float s_uni[kTMaxLimit], s_px[kTMaxLimit], s_qx[kTMaxLimit];
  __shared__ double s_rc[kTMaxLimit];  // R(x) of each pending child of the current node (s_gc: x removed)
  __shared__ unsigned long long s_km[kTMaxLimit / 64];  // the entered node's children
  __shared__ double s_d[NW * 16];
  __shared__ unsigned long long s_u[NW], s_all[kSliceMax][4], s_r4[4 * NW];
  __shared__ int s_dec, s_fail, s_pick;
  const long long ob = (long long)b * T_max;
  int T = tree_size[b];
  const bool ok = status[b] == TV_ST_OK && T >= 1 && T <= T_max;
  if (!ok) T = 1;
  for (int c = tid; c < T_max; c += NT) {
    s_tok[c] = c < T ? draft_tokens[ob + c] : -1;
    s_par[c] = (c > 0 && c < T) ? parents[ob + c] : -2;
    s_uni[c] = uniforms[ob + c];
  }
  if (tid == 0) {
    s_path[0] = 0;
    s_fail = 0;
  }
  const int nwd = (n + 31) / 32;
  auto removed = [&](int t) { return (s_rm[t >> 5] >> (t & 31)) & 1u; };
  unsigned long long* slots = reinterpret_cast<unsigned long long*>(ws + (long long)b * V);
  int gen = 0;
  // every workgroup publishes 4 words in exchange gen's slots, then waits for
  // the request's others: all S x 4 end in s_all
  auto exchange = [&](unsigned long long a0, unsigned long long a1, unsigned long long a2,
                      unsigned long long a3) __attribute__((always_inline)) {
    __syncthreads();
    unsigned long long* g = slots + (long long)gen * S * 4;
    if (tid < 4)
      __hip_atomic_store(g + sl * 4 + tid, tid == 0 ? a0 : tid == 1 ? a1 : tid == 2 ? a2 : a3, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    if (tid < 4 * S) {
      unsigned long long v;
      int spins = 0;
      while ((v = __hip_atomic_load(g + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) == kSlotEmpty) {
        if (++spins > kSliceSpin || s_fail) {
          s_fail = 1;
          break;
        }
      }
      s_all[tid >> 2][tid & 3] = v;
    }
    __syncthreads();
    ++gen;
  };
  auto dsum = [&](int f) {  // field f of every slice as float64, added in slice order
    double t = 0.0;
    for (int s2 = 0; s2 < S; ++s2) t += __longlong_as_double((long long)s_all[s2][f]);
    return t;
  };
  auto as_u = [](double x) { return (unsigned long long)__double_as_longlong(x); };
  // Node entry: R = p and Q = q on the slice, the removed set cleared, p(x) and
  // q(x) of the node's children gathered; the slice sums of p and q, the last
  // token with p > 0 (+ 1; 0: none) and the best p as a rank key, exchanged.
  auto enter = [&](int nd) {
    const float* p = target_probs + (ob + nd) * (long long)V;
    const float* q = draft_probs + (ob + nd) * (long long)V;
    double a = 0.0, c = 0.0;
    int lastp = 0;
    unsigned long long bst = 0ull;
    row_pass<NT>(n, [&](int t) { return float2{p[v0 + t], q[v0 + t]}; }, [&](int t, float2 e) {
      s_R[t] = (double)e.x;
      s_Q[t] = e.y;
      a += (double)e.x;
      c += (double)e.y;
      if (e.x > 0.0f) lastp = v0 + t + 1;
      bst = umax64(bst, rank_key(e.x, (uint32_t)(v0 + t)));
    });
    for (int w = tid; w < nwd; w += NT) s_rm[w] = 0u;
    for (int c2 = tid; c2 < T; c2 += NT) {
      const int x = s_tok[c2];
      const bool in = c2 > 0 && s_par[c2] == nd && x >= 0 && x < V;
      s_px[c2] = in ? p[x] : 0.0f;
      s_qx[c2] = in ? q[x] : 0.0f;
    }
    {  // the node's children as a bit mask (node c: bit c % 64 of word c / 64)
      const unsigned long long km = __ballot(tid > 0 && tid < T && s_par[tid] == nd);
      if (lane == 0 && wave < kTMaxLimit / 64) s_km[wave] = km;
    }
    unsigned long long lp = (unsigned long long)lastp;
    block_sum2_max2<NT>(a, c, lp, bst, s_r4);
    exchange(as_u(a), as_u(c), lp, bst);
    unsigned long long bb = 0ull;
    for (int s2 = 0; s2 < S; ++s2) bb = umax64(bb, s_all[s2][3]);
    return bb;  // the node's best token over every slice
  };

  int node = 0, len = 0, entered = -1;
  unsigned long long besta = 0ull;  // the entered node's best token (rank key)
  while (ok && len < dcap) {
    besta = enter(node);
    entered = node;
    if (s_fail) break;
    double ZR = dsum(0), ZQ = dsum(1);
    int next = -1;
    // R(x) of every child: p(x) until an update (thread c holds child c)
    if (tid < T) {
      const int xc = s_tok[tid];
      s_rc[tid] = (s_par[tid] == node && xc >= 0 && xc < V) ? (double)s_px[tid] : 0.0;
      s_gc[tid] = 0;
    }
    __syncthreads();
    // the children in ascending id, from the mask
    int kq = 0;
    unsigned long long kmask = s_km[0];
    for (;;) {
      while (kmask == 0ull && kq + 1 < kTMaxLimit / 64 && (kq + 1) * 64 < T) kmask = s_km[++kq];
      if (kmask == 0ull) break;
      const int c = 64 * kq + __ffsll((long long)kmask) - 1;
      kmask &= kmask - 1ull;
      const int x = s_tok[c];
      const bool inside = x >= 0 && x < V;
      bool acc;
      {
        // R(x) and Q(x) now: p(x), q(x) through this node's updates so far, kept
        // up to date by thread c (the same operations as the slice pass that
        // holds x)
        const double r = s_rc[c];
        const double s = (inside && !s_gc[c]) ? (double)s_qx[c] : 0.0;
        const double lhs = ((double)s_uni[c] * s) * ZR;
        const double rhs = r * ZQ;
        acc = r > 0.0 && (s == 0.0 || lhs < rhs);
      }
      if (acc) {
        next = c;
        break;
      }
      const bool rm = without_replacement && inside;
      // the later children's R(x): this rejection's update, then x removed from Q
      // (the barriers of the exchange below order it before their tests)
      if (tid > c && tid < T && s_par[tid] == node) {
        const int xc = s_tok[tid];
        if (xc >= 0 && xc < V) {
          if (ZQ > 0.0) {
            const double qv = s_gc[tid] ? 0.0 : (double)s_qx[tid];
            const double a = s_rc[tid] * ZQ;
            const double bq = qv * ZR;
            s_rc[tid] = fmax(0.0, a - bq);
          }
          if (rm && xc == x) s_gc[tid] = 1;
        }
      }
      if (!(ZQ > 0.0)) __syncthreads();  // (no exchange below to order the update)
      if (ZQ > 0.0) {
        // R <- max(0, R ZQ - Q ZR) on the slice; without replacement Q loses x
        double a = 0.0, c2 = 0.0;
        int lastp = 0;
        // (eight entries' reads in flight together; entries in increasing t)
        for (int t0 = tid; t0 < n; t0 += 8 * NT) {
          double rv[8];
          float qq[8];
          uint32_t rw[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int t = min(t0 + u * NT, n - 1);
            rv[u] = s_R[t];
            qq[u] = s_Q[t];
            rw[u] = s_rm[t >> 5];
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int t = t0 + u * NT;
            if (t < n) {
              const double qv = ((rw[u] >> (t & 31)) & 1u) ? 0.0 : (double)qq[u];
              const double ra = rv[u] * ZQ;
              const double rb = qv * ZR;
              const double nr = fmax(0.0, ra - rb);
              s_R[t] = nr;
              a += nr;
              c2 += (rm && v0 + t == x) ? 0.0 : qv;
              if (nr > 0.0) lastp = v0 + t + 1;
            }
          }
        }
        unsigned long long lp = (unsigned long long)lastp, unused = 0ull;
        block_sum2_max2<NT>(a, c2, lp, unused, s_r4);
        if (rm && x >= v0 && x < v0 + n && tid == 0) s_rm[(x - v0) >> 5] |= 1u << ((x - v0) & 31);
        exchange(as_u(a), as_u(c2), lp, 0ull);
        if (s_fail) break;
        ZR = dsum(0);
        if (rm) ZQ = dsum(1);
      }
    }
    if (s_fail || next < 0) break;
    ++len;
    node = next;
    if (tid == 0) s_path[len] = node;
  }

  // ---- the correction token at `node`, from R on the slices (p when nothing was
  // rejected there, or when the walk stopped before entering it).  The last
  // exchange holds every slice's sum of R and its last token with R > 0.
  if (!s_fail && entered != node) besta = enter(node);
  // this slice: each thread a contiguous range of it, in token order
  const int Lt = (n + NT - 1) / NT;
  const int c0 = min(n, tid * Lt), c1 = min(n, c0 + Lt);
  double cs = 0.0;
  for (int t = c0; t < c1; ++t) cs += s_R[t];
  double lo, hi, tot;
  block_scan<double, NT>(cs, s_d, lo, hi, tot);
  if (tid == 0) s_pick = -1;
  __syncthreads();
  if (!s_fail) {
    double total = 0.0;
    unsigned long long lpa = 0ull;
    for (int s2 = 0; s2 < S; ++s2) {
      total += __longlong_as_double((long long)s_all[s2][0]);
      lpa = s_all[s2][2] > lpa ? s_all[s2][2] : lpa;
    }
    int writer = 0, fallback;  // the workgroup that writes the bonus token, and its value if no pick
    double pre = 0.0;
    if (total > 0.0) {
      const double target = (double)s_uni[0] * total;
      fallback = (int)lpa - 1;  // the last token with mass (rounding past every cumulative)
      bool found = false;
      for (int s2 = 0; s2 < S && !found; ++s2) {
        const double z = __longlong_as_double((long long)s_all[s2][0]);
        if (pre <= target && target < pre + z) {
          writer = s2;
          found = true;
        } else {
          pre += z;
        }
      }
      if (found && writer == sl) {
        // inside this slice: cumulative = (the earlier slices) + the in-slice prefix
        const double tl = target - pre;
        // (a range of no width takes no target; should rounding leave two
        // ranges holding it, the larger token is taken)
        if (lo < hi && lo <= tl && tl < hi) {
          double cum = pre + lo;
          int pick = -1;
          for (int t = c0; t < c1; ++t) {
            cum += s_R[t];
            if (cum > target) {
              pick = v0 + t;
              break;
            }
          }
          if (pick >= 0) atomicMax(&s_pick, pick);
        }
      }
    } else {
      fallback = (int)key_index(besta);  // no residual mass: the node's best token
    }
    __syncthreads();
    if (sl == writer && tid == 0) bonus_token[b] = s_pick >= 0 ? s_pick : fallback;
  }
  if (sl == 0) {
    for (int t = tid; t <= dcap; t += NT)
      accept_path[(long long)b * (dcap + 1) + t] = (!s_fail && t <= len) ? s_path[t] : -1;
    if (tid == 0) accept_len[b] = s_fail ? -1 : len;
  }
  if (s_fail && tid == 0) bonus_token[b] = -1;
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
  // up to nt requests: blocks walk the rows in cost order, those past the last
  // row end at once; more: one block per (row, request)
  const dim3 grid = B > 1 && B <= nt ? dim3(T_max * B) : dim3(T_max, B);
  hipLaunchKernelGGL(k, grid, dim3(nt), dyn, reinterpret_cast<hipStream_t>(stream), T_max, V, logits,
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
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  double* ws = reinterpret_cast<double*>(workspace);
  // Few requests over a large vocabulary: S workgroups per request (the sliced
  // kernel), S as large as the device holds all B x S of them at once (at most
  // kSliceMax, slices of at least 1024 tokens and at most 5120).
  constexpr int kSliceNT = 512;
  constexpr int kSliceLdsCap = 5120 * 12 + 5120 / 8;  // the LDS the residency count assumes
  static int cap[8];  // per device: sliced workgroups resident at once, 0 = not yet known
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return TV_ELAUNCH;
  int& cp = cap[dev & 7];
  if (cp == 0) {
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per, reinterpret_cast<const void*>(tv::k_tree_accept_sample_draft_sliced<kSliceNT>), kSliceNT,
            kSliceLdsCap) != hipSuccess)
      return TV_ELAUNCH;
    cp = max(1, cus * per);
  }
  // (the exchange slots live in each request's workspace row: 4 words per slice
  // and exchange)
  const int S = std::min(std::min(std::min(tv::kSliceMax, cp / B), V / 1024), V / (4 * tv::slice_exchanges(T_max)));
  const int L = S >= 2 ? ((V + S - 1) / S + 63) / 64 * 64 : 0;
  if (S >= 2 && L <= 5120) {
    const size_t dyn = (size_t)L * 12 + (size_t)(L + 31) / 32 * 4;
    hipLaunchKernelGGL(tv::k_slice_reset, dim3(B), dim3(256), 0, st, ws, V, 4 * S * tv::slice_exchanges(T_max));
    TV_CHECK_LAUNCH();
    hipLaunchKernelGGL(tv::k_tree_accept_sample_draft_sliced<kSliceNT>, dim3(S, B), dim3(kSliceNT), dyn, st, S, L,
                       T_max, dcap, V, without_replacement ? 1 : 0, draft_tokens, parents, tree_size, target_probs,
                       draft_probs, uniforms, status, accept_len, accept_path, bonus_token, ws);
    TV_CHECK_LAUNCH();
    return TV_OK;
  }
  hipLaunchKernelGGL(tv::k_tree_accept_sample_draft, dim3(B), dim3(tv::kThreads), 0, st, T_max, dcap, V,
                     without_replacement ? 1 : 0, draft_tokens, parents, tree_size, target_probs, draft_probs,
                     uniforms, status, accept_len, accept_path, bonus_token, ws);
  TV_CHECK_LAUNCH();
  return TV_OK;
}
