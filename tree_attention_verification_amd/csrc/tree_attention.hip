// tree_attention: tree-masked grouped-query attention of every draft-tree node
// over the committed prefix K/V plus the node's own ancestors, for gfx950.
//
// What is computed follows the handbook's forward_with_mask (tree_spec.py): the
// full mask is all-visible over the P prefix columns followed by the T x T tree
// mask, the KV heads are repeated over each query-head group, and the softmax
// uses the default 1/sqrt(d) scale; the EAGLE v2 walkthrough's tree_decoding
// (section 4) verifies the whole tree in one forward this way, and the
// TensorRT-LLM dissection keeps that mask bit-packed, 32 nodes per uint32.
//
// bf16 path (k_attn_bf16).  For one (request b, kv head g) the query rows are
// the rep*T (node, head-in-group) pairs, which share every prefix key, so the
// work is a dense (rep*T) x (P+T) tile: QK^T and PV run on the 32x32x16 bf16
// MFMA with fp32 accumulation.
//   * A workgroup is 4 or 8 wavefronts; each wavefront owns one block of 32 query
//     rows and keeps its Q fragments in registers for the whole kernel.
//   * Keys are streamed in tiles of 64 through double-buffered LDS: K rows are
//     copied with coalesced 16-byte loads into an XOR-swizzled layout; V rows are
//     transposed in registers (v_perm) on the way in, so the PV operand is one
//     16-byte LDS read.  The next tile's global loads are in flight while the
//     current tile is computed.
//   * S^T = K Q^T is formed so that each lane holds 16 keys of one query row:
//     the row max needs one cross-half exchange, and the accumulator becomes the
//     PV B-operand directly (keys are permuted consistently in the V^T tile).
//   * Softmax is online in fp32 in the exp2 domain (scale*log2(e) folded into one
//     FMA); the running max is only raised when a tile exceeds it by more than
//     8 (log2 units), so rescaling the accumulators is rare.
//   * The tree mask is read once per row (one 64-bit word) and only the tile(s)
//     reaching past the prefix apply it; no T x T boolean is formed.
//   * Long key ranges are split across workgroups (split-KV); each split writes
//     (max, sum, unnormalised output) partials and k_attn_combine merges them
//     with a log-sum-exp weighting.  Workgroups that share a (request, head,
//     split) but hold different row blocks are placed on the same XCD (the
//     dispatcher assigns workgroups round-robin to the 8 XCDs), so their K/V
//     tiles are fetched from HBM once and hit the shared L2 afterwards.
// fp32 path (k_attn_fp32): one wavefront per (request, head, node), keys spread
// over lanes with a per-lane online softmax, merged through LDS.
#include "tv_common.h"

namespace tv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int KT = 64;  // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSlack = 8.0f;  // lazy running-max threshold, log2 units (p <= 256)

struct Plan {
  int nw;          // wavefronts per workgroup (each owns 32 query rows)
  int rows_wg;     // query rows per workgroup
  int n_rowblk;    // row blocks per (request, kv head)
  int n_split;     // key splits per (request, kv head)
  int chunk_keys;  // keys per split (multiple of KT)
  long long m_pad; // padded rows per (request, kv head) in the workspace
  int n_units;     // B * Hkv * n_split
  int grid;
};

Plan make_plan(int B, int T_max, int Hq, int Hkv, long long S_cap) {
  Plan p{};
  const int rep = Hq / Hkv;
  const long long m_max = (long long)rep * T_max;
  p.nw = m_max <= 128 ? 4 : 8;
  p.rows_wg = 32 * p.nw;
  p.n_rowblk = (int)((m_max + p.rows_wg - 1) / p.rows_wg);
  const long long base = (long long)B * Hkv * p.n_rowblk;
  const long long target = 512;  // two workgroups per CU
  long long max_split = (S_cap + 4 * KT - 1) / (4 * KT);  // >= 256 keys per split
  if (max_split < 1) max_split = 1;
  long long ns = (target + base - 1) / base;
  if (ns > max_split) ns = max_split;
  if (ns < 1) ns = 1;
  long long chunk = (S_cap + ns - 1) / ns;
  chunk = (chunk + KT - 1) / KT * KT;
  ns = (S_cap + chunk - 1) / chunk;
  p.n_split = (int)ns;
  p.chunk_keys = (int)chunk;
  p.m_pad = (long long)p.n_rowblk * p.rows_wg;
  p.n_units = (int)((long long)B * Hkv * ns);
  p.grid = 8 * p.n_rowblk * ((p.n_units + 7) / 8);
  return p;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

template <int D, int NW>
__global__ __launch_bounds__(NW * 64, 8 / NW) void k_attn_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ Kc, const uint16_t* __restrict__ Vc,
    long long S_cap, const int* __restrict__ prefix_len, const int* __restrict__ tree_size,
    const uint32_t* __restrict__ tree_mask, const int* __restrict__ status, int T_max, int Hq, int Hkv, int W,
    float sl2, uint16_t* __restrict__ O, float* __restrict__ ws_o, float* __restrict__ ws_ml, int n_split,
    int chunk_keys, int n_rowblk, int n_units, long long m_pad) {
  constexpr int RB = 1;           // 32-row blocks per wavefront
  constexpr int NT = NW * 64;
  constexpr int KSTEPS = D / 16;  // 16-wide k-steps of QK^T (8 per half of d)
  constexpr int DB = D / 32;      // 32-wide d blocks of the output
  constexpr int CH = D / 8;       // 16-byte chunks per K/V row
  constexpr int VTS = KT + 8;     // padded V^T row (elements): 144 B for KT = 64
  constexpr int KLD = KT * CH / NT;
  constexpr int VITEMS = (KT / 4) * CH;  // (run of 4 keys, chunk) pairs per tile (<= NT)
  __shared__ __attribute__((aligned(16))) uint16_t s_k[2][KT * D];
  __shared__ __attribute__((aligned(16))) uint16_t s_vt[2][D * VTS];

  // ---- which (request, kv head, split, row block) this workgroup owns
  const int wg = blockIdx.x;
  const int slot = wg >> 3;
  const int rbk = slot % n_rowblk;
  const int u = (slot / n_rowblk) * 8 + (wg & 7);
  if (u >= n_units) return;
  const int split = u % n_split;
  const int bg = u / n_split;
  const int g = bg % Hkv, b = bg / Hkv;
  const int rep = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;

  int T = tree_size[b];
  const int P = prefix_len[b];
  if (status[b] != TV_ST_OK || T < 1 || T > T_max) T = 1;
  const int M = rep * T;
  const int row0 = rbk * NW * 32 * RB;
  if (row0 >= M) return;
  if (P < 0 || (long long)P + T > S_cap) {
    // the prefix does not fit the cache: zero this block's output rows once
    if (split == 0) {
      for (int q = tid; q < NW * 32 * RB * CH; q += NT) {
        const int r = row0 + q / CH;
        if (r < M) {
          const int i = r / rep, head = g * rep + r % rep;
          reinterpret_cast<u32x4*>(O + (((long long)b * T_max + i) * Hq + head) * D)[q % CH] = u32x4{0, 0, 0, 0};
        }
      }
    }
    return;
  }
  const int nkeys = P + T;
  const int k_begin = split * chunk_keys;
  if (k_begin >= nkeys) return;
  const int k_end = min(nkeys, k_begin + chunk_keys);
  const int n_tiles = (k_end - k_begin + KT - 1) / KT;

  const uint16_t* Kb = Kc + ((long long)b * Hkv + g) * S_cap * D;
  const uint16_t* Vb = Vc + ((long long)b * Hkv + g) * S_cap * D;

  // ---- Q fragments and mask rows of this wavefront's query rows
  bf16x8 qf[RB][KSTEPS];
  unsigned long long mrow[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = row0 + (wave * RB + rb) * 32 + l32;
    if (r < M) {
      const int i = r / rep, head = g * rep + r % rep;
      const u32x4* qp = reinterpret_cast<const u32x4*>(Q + (((long long)b * T_max + i) * Hq + head) * D + h * (D / 2));
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) qf[rb][kk] = as_bf16x8(qp[kk]);
      const uint32_t* mp = tree_mask + ((long long)b * T_max + i) * W;
      mrow[rb] = (unsigned long long)mp[0] | (W > 1 ? ((unsigned long long)mp[1] << 32) : 0ull);
    } else {
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) qf[rb][kk] = as_bf16x8(u32x4{0, 0, 0, 0});
      mrow[rb] = 0ull;
    }
  }

  f32x16 acc[RB][DB];
  float m_run[RB], l_part[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = -INFINITY;
    l_part[rb] = 0.0f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rb][db][v] = 0.0f;
  }

  // ---- tile staging: global -> registers -> LDS
  u32x4 kreg[KLD];
  u32x4 vreg[4];
  const int v_run = tid / CH, v_c = tid % CH;  // V item of this thread (if tid < VITEMS)
  auto load_tile = [&](int kt0) {
#pragma unroll
    for (int j = 0; j < KLD; ++j) {
      const int q = tid + j * NT;
      const int row = q / CH, c = q % CH;
      const int key = min(kt0 + row, nkeys - 1);
      kreg[j] = reinterpret_cast<const u32x4*>(Kb + (long long)key * D)[c];
    }
    if (tid < VITEMS) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = min(kt0 + 4 * v_run + e, nkeys - 1);
        vreg[e] = reinterpret_cast<const u32x4*>(Vb + (long long)key * D)[v_c];
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int j = 0; j < KLD; ++j) {
      const int q = tid + j * NT;
      const int row = q / CH, c = q % CH;
      *reinterpret_cast<u32x4*>(&s_k[buf][row * D + ((c ^ (row & 7)) * 8)]) = kreg[j];
    }
    if (tid < VITEMS) {
      // keys 4*v_run .. +3 sit at permuted positions p..p+3 of their 16-key group:
      // key k of a group goes to 8*((k/4)%2) + 4*(k/8) + k%4 (bits 2 and 3 swapped)
      const int s4 = v_run & 3;
      const int pos = 16 * (v_run >> 2) + 8 * (s4 & 1) + 4 * (s4 >> 1);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t lo = __builtin_amdgcn_perm(vreg[1][e >> 1], vreg[0][e >> 1], sel);
        const uint32_t hi = __builtin_amdgcn_perm(vreg[3][e >> 1], vreg[2][e >> 1], sel);
        *reinterpret_cast<u32x2*>(&s_vt[buf][(8 * v_c + e) * VTS + pos]) = u32x2{lo, hi};
      }
    }
  };

  load_tile(k_begin);
  store_tile(0);
  __syncthreads();
  int buf = 0;
  for (int t = 0; t < n_tiles; ++t) {
    const int kt0 = k_begin + t * KT;
    const bool more = t + 1 < n_tiles;
    if (more) load_tile(kt0 + KT);

    const uint16_t* sk = s_k[buf];
    const uint16_t* svt = s_vt[buf];
    // S^T = K Q^T for two 32-key blocks
    f32x16 s[RB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) s[rb][kb][v] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int krow = 32 * kb + l32;
        const int c = h * KSTEPS + kk;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sk[krow * D + ((c ^ (krow & 7)) * 8)]);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          s[rb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[rb][kk], s[rb][kb], 0, 0, 0);
      }
    }

    // tree mask (only tiles that reach past the prefix) and online softmax
    const bool tail = kt0 + KT > P;
    bf16x8 pt[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (tail) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = kt0 + 32 * kb + 8 * (v >> 2) + 4 * h + (v & 3);
            const bool vis = key < P || (key < nkeys && ((mrow[rb] >> (key - P)) & 1ull));
            if (!vis) s[rb][kb][v] = -INFINITY;
          }
      }
      float mx = s[rb][0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[rb][kb][v]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float tmax = mx * sl2;
      const bool need = tmax > m_run[rb] + kSlack;
      if (__ballot(need)) {
        const float alpha = need ? __builtin_amdgcn_exp2f(m_run[rb] - tmax) : 1.0f;
        if (need) m_run[rb] = tmax;
        l_part[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[rb][db][v] *= alpha;
      }
      const float mb = m_run[rb] == -INFINITY ? 0.0f : m_run[rb];
      float lsum = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[rb][kb][v], sl2, -mb));
          s[rb][kb][v] = p;
          lsum += p;
        }
      l_part[rb] += lsum;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int kb = ks >> 1, o = 8 * (ks & 1);
        u32x4 w4;
        w4[0] = pack_bf16(s[rb][kb][o + 0], s[rb][kb][o + 1]);
        w4[1] = pack_bf16(s[rb][kb][o + 2], s[rb][kb][o + 3]);
        w4[2] = pack_bf16(s[rb][kb][o + 4], s[rb][kb][o + 5]);
        w4[3] = pack_bf16(s[rb][kb][o + 6], s[rb][kb][o + 7]);
        pt[rb][ks] = as_bf16x8(w4);
      }
    }

    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&svt[(32 * db + l32) * VTS + 16 * ks + 8 * h]);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          acc[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pt[rb][ks], acc[rb][db], 0, 0, 0);
      }
    }

    if (more) store_tile(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  // ---- epilogue
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float l_tot = l_part[rb] + __shfl_xor(l_part[rb], 32, 64);
    const int r = row0 + (wave * RB + rb) * 32 + l32;
    if (r >= M) continue;
    if (n_split == 1) {
      const int i = r / rep, head = g * rep + r % rep;
      uint16_t* op = O + (((long long)b * T_max + i) * Hq + head) * D;
      const float inv = 1.0f / l_tot;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const int d0 = 32 * db + 8 * v4 + 4 * h;
          u32x2 w2;
          w2[0] = pack_bf16(acc[rb][db][4 * v4 + 0] * inv, acc[rb][db][4 * v4 + 1] * inv);
          w2[1] = pack_bf16(acc[rb][db][4 * v4 + 2] * inv, acc[rb][db][4 * v4 + 3] * inv);
          *reinterpret_cast<u32x2*>(op + d0) = w2;
        }
    } else {
      const long long prow = ((long long)bg * n_split + split) * m_pad + r;
      float* wp = ws_o + prow * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const int d0 = 32 * db + 8 * v4 + 4 * h;
          *reinterpret_cast<f32x4*>(wp + d0) =
              f32x4{acc[rb][db][4 * v4 + 0], acc[rb][db][4 * v4 + 1], acc[rb][db][4 * v4 + 2], acc[rb][db][4 * v4 + 3]};
        }
      if (h == 0) {
        ws_ml[2 * prow] = m_run[rb];
        ws_ml[2 * prow + 1] = l_tot;
      }
    }
  }
}

// Merge split partials: weights exp2(m_s - max m), output sum(w o_s) / sum(w l_s).
template <int D>
__global__ __launch_bounds__(256) void k_attn_combine(const float* __restrict__ ws_o, const float* __restrict__ ws_ml,
                                                      const int* __restrict__ prefix_len,
                                                      const int* __restrict__ tree_size,
                                                      const int* __restrict__ status, long long S_cap, int T_max,
                                                      int Hq, int Hkv, int n_split, int chunk_keys, long long m_pad,
                                                      uint16_t* __restrict__ O) {
  constexpr int TPR = D / 4;          // threads per row, 4 outputs each
  constexpr int RPB = 256 / TPR;      // rows per block
  const int bg = blockIdx.x;
  const int b = bg / Hkv, g = bg % Hkv;
  const int rep = Hq / Hkv;
  int T = tree_size[b];
  const int P = prefix_len[b];
  if (status[b] != TV_ST_OK || T < 1 || T > T_max) T = 1;
  if (P < 0 || (long long)P + T > S_cap) return;
  const int M = rep * T;
  const int r = blockIdx.y * RPB + threadIdx.x / TPR;
  if (r >= M) return;
  const int d0 = 4 * (threadIdx.x % TPR);
  const int nkeys = P + T;
  const int n_act = (nkeys + chunk_keys - 1) / chunk_keys;
  const long long base = (long long)bg * n_split * m_pad + r;
  float mx = -INFINITY;
  for (int s = 0; s < n_act; ++s) mx = fmaxf(mx, ws_ml[2 * (base + s * m_pad)]);
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  float l = 0.0f;
  for (int s = 0; s < n_act; ++s) {
    const long long pr = base + s * m_pad;
    const float ms = ws_ml[2 * pr];
    const float w = ms == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ms - mx);
    l += w * ws_ml[2 * pr + 1];
    const f32x4 x = *reinterpret_cast<const f32x4*>(ws_o + pr * D + d0);
    o += w * x;
  }
  const float inv = 1.0f / l;
  const int i = r / rep, head = g * rep + r % rep;
  uint16_t* op = O + (((long long)b * T_max + i) * Hq + head) * D + d0;
  *reinterpret_cast<u32x2*>(op) = u32x2{pack_bf16(o[0] * inv, o[1] * inv), pack_bf16(o[2] * inv, o[3] * inv)};
}

// fp32 path: one wavefront per (node, query head, request).
template <int D>
__global__ __launch_bounds__(64) void k_attn_fp32(const float* __restrict__ Q, const float* __restrict__ Kc,
                                                  const float* __restrict__ Vc, long long S_cap,
                                                  const int* __restrict__ prefix_len,
                                                  const int* __restrict__ tree_size,
                                                  const uint32_t* __restrict__ tree_mask,
                                                  const int* __restrict__ status, int T_max, int Hq, int Hkv, int W,
                                                  float scale, float* __restrict__ O) {
  const int i = blockIdx.x, hq = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  int T = tree_size[b];
  const int P = prefix_len[b];
  if (status[b] != TV_ST_OK || T < 1 || T > T_max) T = 1;
  if (i >= T) return;
  float* op = O + (((long long)b * T_max + i) * Hq + hq) * D;
  if (P < 0 || (long long)P + T > S_cap) {
    for (int d = lane; d < D; d += 64) op[d] = 0.0f;
    return;
  }
  const int g = hq / (Hq / Hkv);
  const int nkeys = P + T;
  const float* qp = Q + (((long long)b * T_max + i) * Hq + hq) * D;
  const float* Kb = Kc + ((long long)b * Hkv + g) * S_cap * D;
  const float* Vb = Vc + ((long long)b * Hkv + g) * S_cap * D;
  const uint32_t* mp = tree_mask + ((long long)b * T_max + i) * W;
  const unsigned long long mrow = (unsigned long long)mp[0] | (W > 1 ? ((unsigned long long)mp[1] << 32) : 0ull);
  __shared__ float s_q[D];
  for (int d = lane; d < D; d += 64) s_q[d] = qp[d];
  __syncthreads();
  float m = -INFINITY, l = 0.0f, acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.0f;
  for (int key = lane; key < nkeys; key += 64) {
    if (!(key < P || ((mrow >> (key - P)) & 1ull))) continue;
    const float* kr = Kb + (long long)key * D;
    float sc = 0.0f;
#pragma unroll
    for (int d = 0; d < D; ++d) sc = fmaf(s_q[d], kr[d], sc);
    sc *= scale;
    const float mn = fmaxf(m, sc);
    const float a = expf(m - mn);  // m = -inf -> 0
    const float p = expf(sc - mn);
    const float* vr = Vb + (long long)key * D;
    l = l * a + p;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = fmaf(p, vr[d], acc[d] * a);
    m = mn;
  }
  __shared__ float s_m[64], s_l[64];
  __shared__ float s_acc[64][D + 1];
  s_m[lane] = m;
  __syncthreads();
  float mx = -INFINITY;
  for (int j = 0; j < 64; ++j) mx = fmaxf(mx, s_m[j]);
  const float f = m == -INFINITY ? 0.0f : expf(m - mx);
  s_l[lane] = l * f;
#pragma unroll
  for (int d = 0; d < D; ++d) s_acc[lane][d] = acc[d] * f;
  __syncthreads();
  float lt = 0.0f;
  for (int j = 0; j < 64; ++j) lt += s_l[j];
  for (int d = lane; d < D; d += 64) {
    float o = 0.0f;
    for (int j = 0; j < 64; ++j) o += s_acc[j][d];
    op[d] = o / lt;
  }
}

template <int D, int NW>
void launch_bf16(const Plan& p, hipStream_t s, const void* Q, const void* Kc, const void* Vc, long long S_cap,
                 const int* prefix_len, const int* tree_size, const uint32_t* tree_mask, const int* status,
                 int T_max, int Hq, int Hkv, int W, float sl2, void* O, float* ws_o, float* ws_ml) {
  hipLaunchKernelGGL((k_attn_bf16<D, NW>), dim3(p.grid), dim3(NW * 64), 0, s, (const uint16_t*)Q, (const uint16_t*)Kc,
                     (const uint16_t*)Vc, S_cap, prefix_len, tree_size, tree_mask, status, T_max, Hq, Hkv, W, sl2,
                     (uint16_t*)O, ws_o, ws_ml, p.n_split, p.chunk_keys, p.n_rowblk, p.n_units, p.m_pad);
}

size_t ws_bytes_for(const Plan& p, int B, int Hkv, int d) {
  if (p.n_split <= 1) return 0;
  return (size_t)B * Hkv * p.n_split * p.m_pad * (size_t)(d + 2) * sizeof(float) + 256;
}

}  // namespace
}  // namespace tv

extern "C" size_t tree_attention_workspace_bytes(int dtype, int B, int T_max, int Hq, int Hkv, int d,
                                                 long long S_cap) {
  if (dtype != TV_DTYPE_BF16 || B <= 0 || T_max <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || S_cap <= 0) return 0;
  const tv::Plan p = tv::make_plan(B, T_max, Hq, Hkv, S_cap);
  return tv::ws_bytes_for(p, B, Hkv, d);
}

extern "C" int tree_attention(int dtype, int B, int T_max, int Hq, int Hkv, int d, const void* Q, const void* Kc,
                              const void* Vc, long long S_cap, const int* prefix_len, const int* tree_size,
                              const uint32_t* tree_mask, const int* status, float scale, void* O, void* workspace,
                              size_t ws_bytes, void* stream) {
  using namespace tv;
  if (B <= 0 || T_max <= 0 || Hq <= 0 || Hkv <= 0 || S_cap <= 0) return TV_EINVAL;
  if (Hq % Hkv != 0) return TV_EINVAL;
  if (!Q || !Kc || !Vc || !prefix_len || !tree_size || !tree_mask || !status || !O) return TV_EINVAL;
  if (dtype != TV_DTYPE_BF16 && dtype != TV_DTYPE_FP32) return TV_EUNSUPPORTED;
  if (d != 64 && d != 128) return TV_EUNSUPPORTED;
  if (T_max > kTMaxLimit) return TV_EUNSUPPORTED;
  if ((long long)B * T_max * Hq > (1LL << 31) || (long long)B * Hkv > (1LL << 24)) return TV_EINVAL;
  const uintptr_t mis = reinterpret_cast<uintptr_t>(Q) | reinterpret_cast<uintptr_t>(Kc) |
                        reinterpret_cast<uintptr_t>(Vc) | reinterpret_cast<uintptr_t>(O);
  if (mis & 15) return TV_EINVAL;
  if (!(scale > 0.0f)) scale = 1.0f / sqrtf((float)d);
  const int W = (T_max + 31) / 32;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dtype == TV_DTYPE_FP32) {
    dim3 grid(T_max, Hq, B);
    if (B > 65535 || Hq > 65535) return TV_EUNSUPPORTED;
    if (d == 64)
      hipLaunchKernelGGL(k_attn_fp32<64>, grid, dim3(64), 0, s, (const float*)Q, (const float*)Kc, (const float*)Vc,
                         S_cap, prefix_len, tree_size, tree_mask, status, T_max, Hq, Hkv, W, scale, (float*)O);
    else
      hipLaunchKernelGGL(k_attn_fp32<128>, grid, dim3(64), 0, s, (const float*)Q, (const float*)Kc,
                         (const float*)Vc, S_cap, prefix_len, tree_size, tree_mask, status, T_max, Hq, Hkv, W, scale,
                         (float*)O);
    TV_CHECK_LAUNCH();
    return TV_OK;
  }
  const Plan p = make_plan(B, T_max, Hq, Hkv, S_cap);
  const size_t need = ws_bytes_for(p, B, Hkv, d);
  if (need && (!workspace || ws_bytes < need)) return TV_EWORKSPACE;
  float* ws_o = reinterpret_cast<float*>(workspace);
  float* ws_ml = need ? ws_o + (size_t)B * Hkv * p.n_split * p.m_pad * d : nullptr;
  const float sl2 = scale * kLog2e;
  if (d == 128) {
    if (p.nw == 4)
      launch_bf16<128, 4>(p, s, Q, Kc, Vc, S_cap, prefix_len, tree_size, tree_mask, status, T_max, Hq, Hkv, W, sl2,
                          O, ws_o, ws_ml);
    else
      launch_bf16<128, 8>(p, s, Q, Kc, Vc, S_cap, prefix_len, tree_size, tree_mask, status, T_max, Hq, Hkv, W, sl2,
                          O, ws_o, ws_ml);
  } else {
    if (p.nw == 4)
      launch_bf16<64, 4>(p, s, Q, Kc, Vc, S_cap, prefix_len, tree_size, tree_mask, status, T_max, Hq, Hkv, W, sl2,
                         O, ws_o, ws_ml);
    else
      launch_bf16<64, 8>(p, s, Q, Kc, Vc, S_cap, prefix_len, tree_size, tree_mask, status, T_max, Hq, Hkv, W, sl2,
                         O, ws_o, ws_ml);
  }
  TV_CHECK_LAUNCH();
  if (p.n_split > 1) {
    const int rpb = 256 / (d / 4);
    dim3 grid(B * Hkv, (unsigned)((p.m_pad + rpb - 1) / rpb));
    if (d == 128)
      hipLaunchKernelGGL(k_attn_combine<128>, grid, dim3(256), 0, s, ws_o, ws_ml, prefix_len, tree_size, status, S_cap,
                         T_max, Hq, Hkv, p.n_split, p.chunk_keys, p.m_pad, (uint16_t*)O);
    else
      hipLaunchKernelGGL(k_attn_combine<64>, grid, dim3(256), 0, s, ws_o, ws_ml, prefix_len, tree_size, status, S_cap,
                         T_max, Hq, Hkv, p.n_split, p.chunk_keys, p.m_pad, (uint16_t*)O);
    TV_CHECK_LAUNCH();
  }
  return TV_OK;
}
