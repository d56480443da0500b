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
__device__ __forceinline__ int wave_sum_i(int v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// sum over the workgroup; every thread gets the same value (s: kWaves slots)
__device__ __forceinline__ double block_sum_d(double v, double* s) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum_d(v);
  if (lane == 0) s[wave] = v;
  __syncthreads();
  double t = 0.0;
  for (int w = 0; w < kWaves; ++w) t += s[w];
  __syncthreads();
  return t;
}
__device__ __forceinline__ int block_sum_i(int v, int* s) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum_i(v);
  if (lane == 0) s[wave] = v;
  __syncthreads();
  int t = 0;
  for (int w = 0; w < kWaves; ++w) t += s[w];
  __syncthreads();
  return t;
}

// Exclusive / inclusive prefix of per-thread values in thread order: lo = sum of
// the earlier threads' values, hi = lo + own.  hi of thread t and lo of thread
// t + 1 are the same stored number.  total = sum of all.
template <typename T>
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
  for (int w = 0; w < kWaves; ++w) {
    if (w < wave) off = off + s[w];
    tot = tot + s[w];
  }
  __syncthreads();
  const T up = __shfl_up(incl, 1, 64);
  lo = lane > 0 ? off + up : off;
  hi = off + incl;
  total = tot;
}

__device__ __forceinline__ unsigned long long block_max_u64(unsigned long long v, unsigned long long* s) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_max_u64(v);
  if (lane == 0) s[wave] = v;
  __syncthreads();
  unsigned long long t = 0ull;
  for (int w = 0; w < kWaves; ++w) t = umax64(t, s[w]);
  __syncthreads();
  return t;
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
// found by radix selection over the 32-bit order keys, four bits per pass from
// the top: per pass every thread accumulates sixteen digit counters (counts for
// top-k, float64 weight for top-p) over the tokens that match the digits chosen
// so far, the workgroup sums them, and the digit holding the cut is taken.  Equal
// keys have equal weights; the cut inside a group of equal keys is the n-th of
// them in token order, found by a scan over contiguous token ranges.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_sampling_probs(int T_max, int V, const float* __restrict__ logits,
                                                             const int* __restrict__ tree_size,
                                                             const int* __restrict__ status,
                                                             const float* __restrict__ temperature,
                                                             const int* __restrict__ top_k,
                                                             const float* __restrict__ top_p,
                                                             const float* __restrict__ min_p,
                                                             float* __restrict__ probs) {
#pragma clang fp contract(off)
  const int i = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  int T = tree_size[b];
  if ((status && status[b] != TV_ST_OK) || T < 1 || T > T_max) T = 1;
  if (i >= T) return;
  const float* lr = logits + ((long long)b * T_max + i) * V;
  float* orow = probs + ((long long)b * T_max + i) * V;
  __shared__ double s_d[kWaves * 16];
  __shared__ int s_i[kWaves * 16];
  __shared__ unsigned long long s_u[kWaves];
  __shared__ int s_pick;

  // the first-ranked token
  unsigned long long best = 0ull;
  for (int v = tid; v < V; v += kThreads) best = umax64(best, rank_key(clean_logit(lr[v]), (uint32_t)v));
  best = block_max_u64(best, s_u);
  const uint32_t kmax = (uint32_t)(best >> 32);
  const int tok0 = (int)key_index(best);
  const float tau = temperature[b];
  const int kk = top_k[b];
  const float tp = top_p[b], mp = min_p[b];
  // greedy (NaN temperature included); top_k = 1 and top_p <= 0 keep the first token alone
  if (!(tau > 0.0f) || kk == 1 || tp <= 0.0f) {
    for (int v = tid; v < V; v += kThreads) orow[v] = v == tok0 ? 1.0f : 0.0f;
    return;
  }
  const double dmax = (double)key_float(kmax), dtau = (double)tau;
  auto weight = [&](uint32_t key) -> float {
    return key == kmax ? 1.0f : (float)exp(((double)key_float(key) - dmax) / dtau);
  };
  for (int v = tid; v < V; v += kThreads) orow[v] = weight(logit_key(lr[v]));

  // the n-th token (token order) with key t that satisfies pred, n >= 1: each
  // thread counts its contiguous range, a scan finds the range holding it
  const int L = (V + kThreads - 1) / kThreads;
  const int c0 = min(V, tid * L), c1 = min(V, c0 + L);
  auto nth_with_key = [&](uint32_t t, int n, uint32_t tk, int ck) -> int {
    int c = 0;
    for (int v = c0; v < c1; ++v) {
      const uint32_t k = logit_key(lr[v]);
      c += (k == t && (k > tk || v <= ck)) ? 1 : 0;
    }
    if (tid == 0) s_pick = V;
    int lo, hi, tot;
    block_scan<int>(c, s_i, lo, hi, tot);
    if (lo < n && n <= hi) {
      int r = n - lo;
      for (int v = c0; v < c1; ++v) {
        const uint32_t k = logit_key(lr[v]);
        if (k == t && (k > tk || v <= ck) && --r == 0) {
          s_pick = v;
          break;
        }
      }
    }
    __syncthreads();
    const int res = s_pick;
    __syncthreads();
    return res;
  };

  // ---- top-k cut (tk, ck); the default keeps everything (every key is > 0)
  uint32_t tk = 0u;
  int ck = V;
  if (kk > 1 && kk < V) {
    uint32_t prefix = 0u, pmask = 0u;
    int need = kk;  // ranks still to place at or below the digits chosen so far
    for (int shift = 28; shift >= 0; shift -= 4) {
      int cnt[16];
#pragma unroll
      for (int d = 0; d < 16; ++d) cnt[d] = 0;
      for (int v = tid; v < V; v += kThreads) {
        const uint32_t k = logit_key(lr[v]);
        if ((k & pmask) == prefix) {
          const uint32_t dg = (k >> shift) & 15u;
#pragma unroll
          for (int d = 0; d < 16; ++d) cnt[d] += dg == (uint32_t)d ? 1 : 0;
        }
      }
      const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
      for (int d = 0; d < 16; ++d) {
        const int x = wave_sum_i(cnt[d]);
        if (lane == 0) s_i[wave * 16 + d] = x;
      }
      __syncthreads();
      int sel = 0;
      for (int d = 15; d >= 0; --d) {
        int c = 0;
        for (int w = 0; w < kWaves; ++w) c += s_i[w * 16 + d];
        if (c >= need) {
          sel = d;
          break;
        }
        need -= c;
      }
      __syncthreads();
      prefix |= (uint32_t)sel << shift;
      pmask |= 15u << shift;
    }
    tk = prefix;
    ck = nth_with_key(tk, need, 0u, V);
  }
  auto in_k = [&](uint32_t k, int v) { return k > tk || (k == tk && v <= ck); };

  // ---- top-p cut (tp_key, cp) over the top-k survivors
  uint32_t tpk = 0u;
  int cp = V;
  if (tp < 1.0f) {
    double wk = 0.0;
    for (int v = tid; v < V; v += kThreads) {
      const uint32_t k = logit_key(lr[v]);
      if (in_k(k, v)) wk += (double)orow[v];
    }
    const double target = (double)tp * block_sum_d(wk, s_d);
    uint32_t prefix = 0u, pmask = 0u;
    double above = 0.0;  // weight of the survivors ranked above the digits chosen so far
    bool found = true;
    for (int shift = 28; shift >= 0 && found; shift -= 4) {
      double m[16];
#pragma unroll
      for (int d = 0; d < 16; ++d) m[d] = 0.0;
      for (int v = tid; v < V; v += kThreads) {
        const uint32_t k = logit_key(lr[v]);
        if ((k & pmask) == prefix && in_k(k, v)) {
          const uint32_t dg = (k >> shift) & 15u;
          const double w = (double)orow[v];
#pragma unroll
          for (int d = 0; d < 16; ++d) m[d] += dg == (uint32_t)d ? w : 0.0;
        }
      }
      const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
      for (int d = 0; d < 16; ++d) {
        const double x = wave_sum_d(m[d]);
        if (lane == 0) s_d[wave * 16 + d] = x;
      }
      __syncthreads();
      int sel = -1;
      for (int d = 15; d >= 0; --d) {
        double md = 0.0;
        for (int w = 0; w < kWaves; ++w) md += s_d[w * 16 + d];
        if (above + md >= target) {
          sel = d;
          break;
        }
        above += md;
      }
      __syncthreads();
      if (sel < 0) {
        found = false;  // rounding never reaches the target: every survivor stays
      } else {
        prefix |= (uint32_t)sel << shift;
        pmask |= 15u << shift;
      }
    }
    if (found) {
      tpk = prefix;
      // tokens with key tpk among the survivors, each of weight wt, join in token
      // order until the cumulative weight reaches the target
      int na = 0;
      for (int v = tid; v < V; v += kThreads) {
        const uint32_t k = logit_key(lr[v]);
        na += (k == tpk && in_k(k, v)) ? 1 : 0;
      }
      na = block_sum_i(na, s_i);
      const double wt = (double)weight(tpk);
      double acc = above;
      int n = 0;
      do {
        acc += wt;
        ++n;
      } while (acc < target && n < na);
      cp = nth_with_key(tpk, n, tk, ck);
    }
  }

  // ---- min-p, the kept total and the output
  auto keep = [&](uint32_t k, int v, float w) {
    return in_k(k, v) && (k > tpk || (k == tpk && v <= cp)) && (!(mp > 0.0f) || w >= mp || v == tok0);
  };
  double wsum = 0.0;
  for (int v = tid; v < V; v += kThreads) {
    const float w = orow[v];
    if (keep(logit_key(lr[v]), v, w)) wsum += (double)w;
  }
  const double W = block_sum_d(wsum, s_d);
  for (int v = tid; v < V; v += kThreads) {
    const float w = orow[v];
    orow[v] = keep(logit_key(lr[v]), v, w) ? (float)((double)w / W) : 0.0f;
  }
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
    for (int v = tid; v < V; v += kThreads) {
      zp += (double)p[v];
      zq += (double)q[v];
    }
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
        for (int v = tid; v < V; v += kThreads) {
          const double qv = removed(v) ? 0.0 : (double)q[v];
          const double rv = r_ws ? R[v] : (double)p[v];
          const double a = rv * ZQ;
          const double bq = qv * ZR;
          const double nr = fmax(0.0, a - bq);
          R[v] = nr;
          zr += nr;
          zq2 += (rm && v == x) ? 0.0 : qv;
        }
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
  for (int v = c0; v < c1; ++v) cs += X(v);
  double lo, hi, total;
  block_scan<double>(cs, s_d, lo, hi, total);
  if (tid == 0) s_pick = -1;
  __syncthreads();
  if (total > 0.0) {
    const double target = (double)s_uni[0] * total;
    if (lo <= target && target < hi) {
      double cum = lo;
      int pick = -1, last = -1;
      for (int v = c0; v < c1; ++v) {
        const double x = X(v);
        if (x > 0.0) last = v;
        cum += x;
        if (cum > target) {
          pick = v;
          break;
        }
      }
      s_pick = pick >= 0 ? pick : last;
    }
    __syncthreads();
    if (s_pick < 0) {  // rounding left the target past the total: the last token with mass
      int last = -1;
      for (int v = c0; v < c1; ++v)
        if (X(v) > 0.0) last = v;
      if (last >= 0) atomicMax(&s_pick, last);
      __syncthreads();
    }
  } else {
    // no residual mass: the node's best token (probability desc, token asc)
    unsigned long long best = 0ull;
    for (int v = tid; v < V; v += kThreads) best = umax64(best, rank_key(prow[v], (uint32_t)v));
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
  hipLaunchKernelGGL(tv::k_sampling_probs, dim3(T_max, B), dim3(tv::kThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), T_max, V, logits, tree_size, status, temperature, top_k,
                     top_p, min_p, probs);
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
