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
//   * Keys are streamed in tiles of 64 straight from HBM into LDS with gfx950's
//     global_load_lds_dwordx4 (no registers), into row-major, XOR-swizzled tile
//     buffers; one tile is in flight while the previous one is computed.  The PV
//     operand is read with the gfx950 transpose read (ds_read_b64_tr_b16), so V
//     is never transposed in registers.
//   * S^T = K Q^T is formed so that each lane holds 16 keys of one query row:
//     the row max needs one cross-half exchange, and the accumulator becomes the
//     PV B-operand directly (keys are permuted consistently in the V^T tile).
//   * Softmax is online in fp32 in the exp2 domain (scale*log2(e) folded into one
//     FMA); the running max is only raised when a tile exceeds it by more than
//     8 (log2 units), so rescaling the accumulators is rare; row sums add the
//     bf16-rounded P that the PV product uses, two at a time with v_dot2.
//   * The tree mask is read once per row (one 64-bit word) and only the tile(s)
//     reaching past the prefix apply it; no T x T boolean is formed.
//   * Long key ranges are split across workgroups (split-KV); each split writes
//     its running max and row sum (fp32) and its normalised output (bf16: half
//     the bytes of fp32 with fp32's exponent range, so any finite bf16 V stays
//     finite and small outputs keep their relative precision), and k_attn_combine
//     merges them with a log-sum-exp weighting.  With several requests the splits
//     follow each request's own length and the longest requests start first.
//   * K/V tile 0, the Q fragments and the mask row are requested before the
//     request's tree size and prefix length arrive (keys clamped to the cache
//     slab, nodes to T_max - 1), so the kernel waits for one memory round trip
//     instead of two before its first tile.  Workgroups that share a (request,
//     head, split) but hold different row blocks are placed on the same XCD (the
//     dispatcher assigns workgroups round-robin to the 8 XCDs), so their K/V tiles
//     are fetched from HBM once and hit the shared L2 afterwards.
// fp32 path (k_attn_fp32): one wavefront per (request, head, node), keys spread
// over lanes with a per-lane online softmax, merged through LDS.
#include "tv_common.h"

#include <mutex>

namespace tv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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
  int rel;         // splits relative to each request's own length, longest request first
};

// Rotary embedding of the queries inside the attention kernel ([HB]
// forward_with_mask rotates the tree's queries at position prefix + depth):
// pair (i, i + d/2) turns by pos * f_i revolutions, f_i = theta^(-2i/d) / 2 pi,
// given as a float pair (f_hi + f_lo) so that pos * f_i keeps ~1e-7 revolutions
// of accuracy at any position below 2^24.
struct Rope {
  float f_hi[64];
  float f_lo[64];
};

Plan plan_with(int B, int T_max, int Hq, int Hkv, long long S_cap, int nw, long long min_keys) {
  Plan p{};
  const int rep = Hq / Hkv;
  const long long m_max = (long long)rep * T_max;
  p.nw = nw;
  p.rows_wg = 32 * p.nw;
  p.n_rowblk = (int)((m_max + p.rows_wg - 1) / p.rows_wg);
  const long long base = (long long)B * Hkv * p.n_rowblk;
  // 512 workgroups: two per CU over the run (256 CUs), which leaves room to
  // balance unequal splits (measured: 256 was 2% faster for equal-length
  // requests, 30% slower for the ragged batch of 16)
  const long long target = 512;
  long long max_split = (S_cap + min_keys - 1) / min_keys;
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
  p.rel = B > 1 && B <= 64;
  return p;
}

// Launch shape: 8-wavefront workgroups (two per SIMD, so one wavefront's softmax
// overlaps the other's MFMAs) with splits of >= 256 keys, aiming at 512
// workgroups.  When that leaves most of the chip idle (a single request: 8 kv
// heads x ~9 splits = 72 workgroups), 4-wavefront workgroups (half the rows
// each, one wavefront per SIMD) with splits of >= 320 keys spread the work over
// more CUs.  Measured on MI355X for 61 nodes x 32 heads over a 2048-token prefix
// (one call, combine included, the step's tree build between calls): splits of
// 3, 4 or 5 tiles all take 19.4 us, so the longest (7 splits, 112 workgroups)
// is kept for its fewer partials (11 -> 7 per row); 6 tiles 20.1 us, 8 tiles
// 20.8 us; 8-wavefront workgroups over all 256 rows 22.6-23.8 us.
Plan make_plan(int B, int T_max, int Hq, int Hkv, long long S_cap) {
  const long long m_max = (long long)(Hq / Hkv) * T_max;
  if (m_max <= 128) return plan_with(B, T_max, Hq, Hkv, S_cap, 4, 4 * KT);
  const Plan p = plan_with(B, T_max, Hq, Hkv, S_cap, 8, 4 * KT);
  if (p.grid < 128) return plan_with(B, T_max, Hq, Hkv, S_cap, 4, 5 * KT);
  return p;
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }
#define kOnes2 (bf16x2{(__bf16)1.0f, (__bf16)1.0f})

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

__device__ __forceinline__ bf16x4 ds_read_tr16(const lds_char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
}

// s_waitcnt immediate that waits for lgkmcnt == 0 only (gfx9 encoding: vmcnt bits
// 3:0 and 15:14 at their maximum, expcnt 6:4 at its maximum, lgkmcnt 11:8 = 0)
constexpr int kLgkmOnlyZero = 15 | (3 << 14) | (7 << 4);

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// One 16-byte global -> LDS copy per lane (global_load_lds_dwordx4): lane l's
// 16 bytes land at LDS byte address m0 + 16 l; each lane supplies its own global
// address.  Written as inline assembly so that the compiler does not track it:
// its own wait placement cannot tell the stage buffers apart and would wait for
// every copy in flight before each tile.  The kernel waits explicitly instead
// (vm_wait_imm), counting these copies; the compiler's waits for its own loads
// can only be stricter than needed, since it does not see the younger copies.
__device__ __forceinline__ void dma16(const uint16_t* g, uint32_t lds_byte_addr) {
  // (one wait state between the m0 write and the LDS-DMA instruction that reads it)
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_byte_addr)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const uint16_t* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint16_t*)p;
}

// s_waitcnt immediate that waits until at most n vector-memory operations of this
// wavefront are outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt
// and lgkmcnt left at their maximum)
constexpr int vm_wait_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

template <int D, int NW, int NSTAGE, bool PAGED, bool ROPE>
__global__ __launch_bounds__(NW * 64, (NSTAGE == 2 && NW == 4) ? 2 : 1) void k_attn_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ Kc, const uint16_t* __restrict__ Vc,
    long long S_cap, const int* __restrict__ prefix_len, const int* __restrict__ tree_size,
    const uint32_t* __restrict__ tree_mask, const int* __restrict__ status, int T_max, int Hq, int Hkv, int W,
    float sl2, uint16_t* __restrict__ O, uint16_t* __restrict__ ws_o, float* __restrict__ ws_ml, int n_split,
    int chunk_keys, int n_rowblk, int n_units, long long m_pad, int B, int rel, Paging pg, Rope rope) {
  constexpr int NT = NW * 64;
  constexpr int KSTEPS = D / 16;     // 16-wide k-steps of QK^T (KSTEPS/2 per half of d)
  constexpr int DB = D / 32;         // 32-wide d blocks of the output
  constexpr int CH = D / 8;          // 16-byte chunks per K/V row
  // NSTAGE LDS tile buffers: NSTAGE - 1 tiles in flight while one is computed.
  // Two are used (64 KB at d = 128; with 4-wavefront workgroups two fit on a CU):
  // measured on MI355X, one tile in flight beat three at every configuration
  // (one request over a 2048-token prefix 18.3 -> 16.4 us, 16 ragged requests
  // 93.6 -> 89.6, 4 requests over 32768 tokens 284 -> 279, 64 requests over
  // 4096 tokens 264 -> 256).
  static_assert(NSTAGE == 2 || NSTAGE == 4, "two or four stage buffers");
  static_assert(!PAGED || NSTAGE == 2, "the paged cache's block numbers are fetched one tile ahead");
  constexpr int kAhead = 5;         // LDS fragment reads issued ahead of the MFMAs that use them
  constexpr int INSTR = KT * CH / 64;  // 64-lane DMA instructions per tensor per tile
  static_assert(INSTR % NW == 0, "DMA instructions split evenly over the wavefronts");
  constexpr int DMA_WAVE = 2 * INSTR / NW;  // DMA instructions per wavefront per tile (K and V)
  // K and V tiles are row-major (key rows of D elements) in LDS with their 16-byte
  // chunks XOR-swizzled per row: chunk c of K row r sits at c ^ kswz(r), so the 16
  // consecutive rows that one 16-byte read serves land on distinct banks; chunk c
  // of V row r sits at c ^ vswz(r), which spreads the 4-row x 32-byte footprint of
  // a transpose read over the banks.
  auto kswz = [](int r) { return CH == 16 ? (r & 15) : ((r >> 1) & 7); };
  auto vswz = [](int r) { return CH == 16 ? 4 * (r & 3) : 2 * (r & 3); };
  // NSTAGE K tile buffers followed by NSTAGE V tile buffers (TB bytes each)
  constexpr int ROWB = 2 * D;        // bytes per K/V row
  constexpr int TB = KT * ROWB;      // bytes per tile buffer
  __shared__ __attribute__((aligned(1024))) uint16_t s_kv[2 * NSTAGE * KT * D];
  lds_char* const kv_lds = (lds_char*)(__attribute__((address_space(3))) uint16_t*)s_kv;
  const uint32_t kv_base = lds_addr(s_kv);

  // ---- which (request, kv head, split, row block) this workgroup owns
  const int wg = blockIdx.x;
  const int slot = wg >> 3;
  const int rbk = slot % n_rowblk;
  const int u = (slot / n_rowblk) * 8 + (wg & 7);
  if (u >= n_units) return;
  const int split = u % n_split;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int bg = u / n_split;
  // Several requests (rel): their sizes are read first, one lane per request, and
  // the requests are taken in descending order of key count (ties: lower index
  // first), so the longest ones start first; each request's keys are then split
  // into n_split nearly equal parts (below).
  int rel_T = 0, rel_P = 0, rel_st = 0;
  if (rel) {
    int nk = -1, Tl = 0, Pl = 0, sl = 0;
    if (lane < B) {
      Tl = tree_size[lane];
      Pl = prefix_len[lane];
      sl = status[lane];
      const int Te = (sl != TV_ST_OK || Tl < 1 || Tl > T_max) ? 1 : Tl;
      nk = (Pl < 0 || (long long)Pl + Te > S_cap) ? 0 : Pl + Te;
    }
    // the rank, counted by every wavefront over its share of the requests and
    // added up through LDS (one barrier; the whole count repeated on every
    // wavefront took ~4 us of each workgroup's prologue with 64 requests)
    __shared__ int s_rank[NW][64];
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int per = (B + NW - 1) / NW;
    const int o0 = min(B, wv * per), o1 = min(B, o0 + per);
    int part = 0;
    for (int o = o0; o < o1; ++o) {
      const int x = __builtin_amdgcn_readlane(nk, o);
      part += (x > nk) || (x == nk && o < lane);
    }
    s_rank[wv][lane] = part;
    __syncthreads();
    int rank = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) rank += s_rank[w][lane];
    const unsigned long long m = __ballot(lane < B && rank == bg / Hkv);
    const int bsel = __ffsll((long long)m) - 1;
    bg = bsel * Hkv + bg % Hkv;
    rel_T = __builtin_amdgcn_readlane(Tl, bsel);
    rel_P = __builtin_amdgcn_readlane(Pl, bsel);
    rel_st = __builtin_amdgcn_readlane(sl, bsel);
  }
  const int g = bg % Hkv, b = bg / Hkv;
  const int rep = Hq / Hkv;
  const int l32 = lane & 31, h = lane >> 5;
  const int row0 = rbk * NW * 32;
  int k_begin = split * chunk_keys;  // (rel: set once the request's size is known)

  // linear cache: row `key` of (b, g) is Kb + key D.  Paged cache: it is row
  // ((blk Hkv + g) << lbs) + key % tokens_per_block of the pool, blk the request's
  // block-table entry for key >> lbs, so Kb holds the g << lbs part.
  const uint16_t* Kb = Kc + (PAGED ? ((long long)g << pg.lbs) : ((long long)b * Hkv + g) * S_cap) * D;
  const uint16_t* Vb = Vc + (PAGED ? ((long long)g << pg.lbs) : ((long long)b * Hkv + g) * S_cap) * D;
  const int* const bt = PAGED ? pg.table + (long long)b * pg.max_blocks : nullptr;

  // ---- tile staging: K/V tiles go straight from global memory into LDS (no
  // registers) through NSTAGE stage buffers; tile t + NSTAGE - 1 is requested
  // while tile t is computed.  The 64 lanes of one DMA instruction fill 1 KB of LDS
  // in order, so the XOR swizzle is applied on the global side: LDS slot (row, c)
  // receives chunk c ^ swz(row).  Only tiles inside the split are requested; the
  // wait before tile t allows exactly the younger tiles that were requested (up to
  // NSTAGE - 2) to stay in flight.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform (LDS base goes to m0)
  // paged cache: the block numbers of this lane's rows of the next tile to be
  // requested, loaded one tile ahead.  They are kept as loaded and only clamped
  // into the pool (so a bad table cannot make the kernel read outside it) where
  // the copy uses them: arithmetic on them here would make the wavefront wait
  // for the load, and with it for the tile copy issued just before.
  int pblk[PAGED ? INSTR / NW : 1];
  auto load_tbl = [&](int kt0, int last_key) __attribute__((always_inline)) {
    if constexpr (PAGED) {
#pragma unroll
      for (int ii = 0; ii < INSTR / NW; ++ii) {
        const int row = (64 * (wave_u + ii * NW) + lane) / CH;
        pblk[ii] = bt[min(kt0 + row, last_key) >> pg.lbs];
      }
    }
  };
  auto dma_tile = [&](int kt0, int last_key, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int ii = 0; ii < INSTR / NW; ++ii) {
      const int i = wave_u + ii * NW;
      const int idx = 64 * i + lane;
      const int row = idx / CH, cs = idx % CH;
      const int key = min(kt0 + row, last_key);
      long long roff = key;
      if constexpr (PAGED) {
        const long long blk = min(max((long long)pblk[ii], 0ll), pg.n_blocks - 1);
        roff = ((blk * Hkv) << pg.lbs) + (key & ((1 << pg.lbs) - 1));
      }
      dma16(Kb + roff * D + 8 * (cs ^ kswz(row)), kv_base + buf * TB + 1024u * i);
      dma16(Vb + roff * D + 8 * (cs ^ vswz(row)), kv_base + (NSTAGE + buf) * TB + 1024u * i);
    }
  };

  // ---- first loads, issued before the request's tree size and prefix length are
  // known (they only decide what is kept): K/V tile 0 with keys clamped to the
  // cache slab, then this lane's Q row and packed mask row with the node clamped
  // to T_max - 1.  What lies past the request is neutralised below.
  const int r = row0 + wave * 32 + l32;
  const int i_row = min(r / rep, T_max - 1);
  // (paged: the first tile's block numbers wait for the request's sizes)
  if (!PAGED && !rel) dma_tile(k_begin, (int)S_cap - 1, 0);
  bf16x8 qf[KSTEPS];
  {
    const int head = g * rep + r % rep;
    const u32x4* qp =
        reinterpret_cast<const u32x4*>(Q + (((long long)b * T_max + i_row) * Hq + head) * D + h * (D / 2));
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) qf[kk] = as_bf16x8(qp[kk]);
  }
  // the packed mask row: nodes 0..63 in mrow, all W words (W <= 8, up to 256
  // nodes) in mw; words past W read as zero
  const uint32_t* mp = tree_mask + ((long long)b * T_max + i_row) * W;
  uint32_t mw[8];
#pragma unroll
  for (int w = 0; w < 8; ++w) mw[w] = w < W ? mp[w] : 0u;
  unsigned long long mrow = (unsigned long long)mw[0] | ((unsigned long long)mw[1] << 32);

  int T = rel ? rel_T : tree_size[b];
  const int P = rel ? rel_P : prefix_len[b];
  if ((rel ? rel_st : status[b]) != TV_ST_OK || T < 1 || T > T_max) T = 1;
  const int M = rep * T;
  if (row0 >= M) {
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));  // no LDS DMA may outlive the workgroup
    return;
  }
  if (P < 0 || (long long)P + T > S_cap) {
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
    // the prefix does not fit the cache: zero this block's output rows once
    if (split == 0) {
      for (int q = tid; q < NW * 32 * CH; q += NT) {
        const int rr = row0 + q / CH;
        if (rr < M) {
          const int i = rr / rep, head = g * rep + rr % rep;
          reinterpret_cast<u32x4*>(O + (((long long)b * T_max + i) * Hq + head) * D)[q % CH] = u32x4{0, 0, 0, 0};
        }
      }
    }
    return;
  }
  const int nkeys = P + T;
  int k_end, n_tiles;
  if (rel) {
    // split `split` of min(n_split, tiles) nearly equal parts of the request's
    // tiles; the later splits of a short request are empty
    const int tiles = (nkeys + KT - 1) / KT;
    const int n_eff = min(n_split, tiles);
    if (split >= n_eff) return;  // nothing requested yet
    const int t0 = (int)((long long)split * tiles / n_eff), t1 = (int)((long long)(split + 1) * tiles / n_eff);
    k_begin = t0 * KT;
    k_end = min(nkeys, t1 * KT);
    n_tiles = t1 - t0;
    load_tbl(k_begin, nkeys - 1);
    dma_tile(k_begin, nkeys - 1, 0);
  } else {
    if (k_begin >= nkeys) {
      __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
      return;
    }
    k_end = min(nkeys, k_begin + chunk_keys);
    n_tiles = (k_end - k_begin + KT - 1) / KT;
    // A tile 0 that reaches past the last key was fetched with keys clamped to
    // the slab, so its rows past the request hold whatever the cache holds there:
    // fetch it again with keys clamped to the last key (its scores there are
    // masked to -inf, and finite V rows keep 0 * garbage out of the PV product).
    // The re-fetch lands after the first one (returns are in order).
    if (PAGED) {
      load_tbl(k_begin, nkeys - 1);
      dma_tile(k_begin, nkeys - 1, 0);
    } else if (k_begin + KT > nkeys) {
      dma_tile(k_begin, nkeys - 1, 0);
    }
  }
  // paged: the block numbers of tile 1 travel with tile 0
  if (n_tiles > 1) load_tbl(k_begin + KT, nkeys - 1);
  // padding query rows get a zero Q and no mask
  if (r >= M) {
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) qf[kk] = as_bf16x8(u32x4{0, 0, 0, 0});
    mrow = 0ull;
#pragma unroll
    for (int w = 0; w < 8; ++w) mw[w] = 0u;
  }
  // Q and the mask row are needed now (the empty statement below reads them), so
  // the compiler waits for its loads here; that wait counts every older vector
  // memory operation, tile 0 included, and nothing younger is in flight yet.
  // Tiles 1 and 2 follow, with the request's sizes known (keys clamped to the
  // last key, only tiles of this split), so they need no re-fetch, and stay in
  // flight while tile 0 is computed.
  __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
  asm volatile("" ::"v"(qf[0]), "v"(qf[KSTEPS / 2]), "v"(qf[KSTEPS - 1]), "v"(mrow));
  if constexpr (ROPE) {
    // the queries arrive before their rotary embedding: rotate this lane's half
    // of its row at the node's position P + depth (depth = ancestors in the mask
    // row); the other half of the row is in lane ^ 32
    int anc = 0;
#pragma unroll
    for (int w = 0; w < 8; ++w) anc += __popc(mw[w]);
    const float posf = (float)(P + anc - 1);
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      const u32x4 mine = __builtin_bit_cast(u32x4, qf[kk]);
      u32x4 other;
#pragma unroll
      for (int c = 0; c < 4; ++c) other[c] = (uint32_t)__shfl_xor((int)mine[c], 32, 64);
      const bf16x8 qo = __builtin_bit_cast(bf16x8, other);
      bf16x8 out;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 8 * kk + e;  // pair index (the same for both halves)
        const float fh = rope.f_hi[i], fl = rope.f_lo[i];
        const float p = posf * fh;
        const float err = fmaf(posf, fh, -p) + posf * fl;
        const float rev = (p - rintf(p)) + err;  // the angle in revolutions, |rev| <~ 0.5
        const float sn = __builtin_amdgcn_sinf(rev), cs = __builtin_amdgcn_cosf(rev);
        const float a = (float)qf[kk][e], o = (float)qo[e];
        out[e] = (__bf16)(h == 0 ? fmaf(a, cs, -o * sn) : fmaf(a, cs, o * sn));
      }
      qf[kk] = out;
    }
  }
#pragma unroll
  for (int j = 1; j < NSTAGE - 1; ++j)
    if (n_tiles > j) dma_tile(k_begin + j * KT, nkeys - 1, j);

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[db][v] = 0.0f;
  float m_run = -INFINITY, l_part = 0.0f;

  auto lds_barrier = []() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kLgkmOnlyZero);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // a wavefront whose rows are all padding only helps stage the tiles
  const bool active = row0 + wave * 32 < M;
  const int tg = lane >> 4, tj = lane & 15;

  // LDS byte offsets of this lane's fragments, written so that everything except
  // one XOR with a constant is an instruction immediate.  K: key row 32 kb + l32,
  // chunk (h KSTEPS + kk) ^ kswz(l32) = u ^ kk with u = h KSTEPS ^ kswz(l32), so
  // the offset is 32 kb ROWB + (ka ^ 16 kk).  V (transpose reads): key row
  // 16 ks + 8 hr + r0, column 32 db + c0, chunk 4 db ^ (c0 / 8) ^ vswz(r0), so the
  // offset is (16 ks + 8 hr) ROWB + (va ^ 64 db).
  const uint32_t ka = l32 * ROWB + 16 * ((h * KSTEPS) ^ kswz(l32));
  uint32_t va;
  {
    const int r0 = 4 * (tg >> 1) + (tj >> 2), c0 = 16 * (tg & 1) + 4 * (tj & 3);
    va = r0 * ROWB + 16 * ((c0 >> 3) ^ vswz(r0)) + 2 * (c0 & 7);
  }

  // S^T = K Q^T for two 32-key blocks
  auto qk = [&](int buf, f32x16 (&s)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) s[kb][v] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a =
            *reinterpret_cast<const lds_bf16x8*>(kv_lds + buf * TB + 32 * kb * ROWB + (ka ^ (16u * kk)));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s[kb], 0, 0, 0);
      }
    }
    // schedule: kAhead K fragment reads first, then one MFMA and one read at a time
    if constexpr (kAhead > 0) {
      __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
      for (int i = 0; i < 2 * KSTEPS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i + kAhead < 2 * KSTEPS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
  };
  // tree mask of the tile starting at key kt0 (only tiles that reach past the
  // prefix): the 64-bit window of the lane's mask row in which bit e stands for
  // key kt0 + e (prefix keys set, nodes past the row clear)
  auto word_at = [&](int k) -> uint32_t {  // mask word k (wave-uniform k; 0 past the row)
    uint32_t v = 0u;
#pragma unroll
    for (int w = 0; w < 8; ++w) v = k == w ? mw[w] : v;
    return v;
  };
  auto mask = [&](int kt0, f32x16 (&s)[2]) __attribute__((always_inline)) {
    if (kt0 + KT > P) {
      const int sh = kt0 - P;  // key kt0+e is tree node sh+e
      unsigned long long mt;
      if (sh < 0) {
        mt = sh <= -64 ? ~0ull : ((mrow << -sh) | ((1ull << -sh) - 1ull));
      } else {
        const int q = sh >> 5, r = sh & 31;
        const unsigned long long lo = (unsigned long long)word_at(q) | ((unsigned long long)word_at(q + 1) << 32);
        const unsigned long long hi = word_at(q + 2);
        mt = r ? ((lo >> r) | (hi << (64 - r))) : lo;
      }
      const int lim = nkeys - kt0;  // keys of this tile that exist (1..64)
      const unsigned long long mv = lim >= 64 ? mt : (mt & ((1ull << lim) - 1ull));
      const unsigned long long mh = mv >> (4 * h);
      const uint32_t lo = (uint32_t)mh, hi = (uint32_t)(mh >> 32);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int e = 32 * kb + 8 * (v >> 2) + (v & 3);  // key offset minus 4h
          const uint32_t word = e < 32 ? lo : hi;
          s[kb][v] = ((word >> (e & 31)) & 1u) ? s[kb][v] : -INFINITY;
        }
    }
  };
  // Online softmax without branches: tile max, running max raised only past the
  // slack, exp2, P^T rounded to bf16 and its row sum (which adds exactly the
  // rounded values, two per v_dot2).  Returns the factor the earlier
  // accumulation must be scaled by (1 while the running max stays).
  auto smax = [&](f32x16 (&s)[2], bf16x8 (&pt)[4]) __attribute__((always_inline)) -> float {
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
    {  // the other half of the row sits in lane l ^ 32 (a VALU lane swap, no LDS)
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    const float tmax = mx * sl2;
    const bool need = tmax > m_run + kSlack;
    const float alpha = need ? __builtin_amdgcn_exp2f(m_run - tmax) : 1.0f;
    m_run = need ? tmax : m_run;
    const float mb = m_run == -INFINITY ? 0.0f : m_run;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) s[kb][v] = __builtin_amdgcn_exp2f(fmaf(s[kb][v], sl2, -mb));
    float lsum = l_part * alpha;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kb = ks >> 1, o = 8 * (ks & 1);
      u32x4 w4;
      w4[0] = pack_bf16(s[kb][o + 0], s[kb][o + 1]);
      w4[1] = pack_bf16(s[kb][o + 2], s[kb][o + 3]);
      w4[2] = pack_bf16(s[kb][o + 4], s[kb][o + 5]);
      w4[3] = pack_bf16(s[kb][o + 6], s[kb][o + 7]);
      pt[ks] = as_bf16x8(w4);
#pragma unroll
      for (int e = 0; e < 4; ++e) lsum = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w4[e]), kOnes2, lsum, false);
    }
    l_part = lsum;
    return alpha;
  };
  // O^T += V^T P^T.  The A operand (32 d x 16 keys) comes from the row-major V
  // tile through two transpose reads: in each 16-lane group, lane i receives
  // element i%4 of the 8-byte pieces addressed by lanes i/4, i/4+4, i/4+8,
  // i/4+12, so lane j of the group addresses key row base+j/4, columns
  // 4*(j%4)..+3 of its 16-column slice and gets 4 consecutive keys of one d
  // column.  Keys 16ks+8hr+4h+0..3 (hr = 0, 1) are exactly the runs the S^T
  // accumulator holds for this lane, so P^T needs no shuffling.
  auto pv = [&](int buf, const bf16x8 (&pt)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x4 half[2];
#pragma unroll
        for (int hr = 0; hr < 2; ++hr) {
          half[hr] = ds_read_tr16(kv_lds + (NSTAGE + buf) * TB + (16 * ks + 8 * hr) * ROWB + (va ^ (64u * db)));
        }
        const bf16x8 a = __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pt[ks], acc[db], 0, 0, 0);
      }
    }
    // schedule: the two transpose reads of kAhead MFMAs first, then one MFMA and
    // its two reads at a time
    if constexpr (kAhead > 0) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAhead, 0);
#pragma unroll
      for (int i = 0; i < 4 * DB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i + kAhead < 4 * DB) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    }
  };

  auto compute = [&](int t, int buf) __attribute__((always_inline)) {
    f32x16 s[2];
    bf16x8 pt[4];
    qk(buf, s);
    mask(k_begin + t * KT, s);
    const float alpha = smax(s, pt);
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[db][v] *= alpha;
    }
    pv(buf, pt);
  };
  // step t: wait for this wavefront's part of tile t (the up to NSTAGE - 2 younger
  // tiles may still be in flight, when they exist), barrier (every part landed,
  // and every wavefront is done with tile t-1), request tile t + NSTAGE - 1 (when
  // it exists) into tile t-1's buffer, compute tile t.  Tiles past the request's
  // last tile in this split are never requested, so nothing is left in flight at
  // the end.
  auto step = [&](int t, int buf) __attribute__((always_inline)) {
    const int younger = min(n_tiles - 1 - t, NSTAGE - 2);
    if (NSTAGE == 4 && younger >= 2) __builtin_amdgcn_s_waitcnt(vm_wait_imm(2 * DMA_WAVE));
    else if (NSTAGE == 4 && younger == 1) __builtin_amdgcn_s_waitcnt(vm_wait_imm(DMA_WAVE));
    else __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
    lds_barrier();
    if (t + NSTAGE - 1 < n_tiles) {
      dma_tile(k_begin + (t + NSTAGE - 1) * KT, nkeys - 1, (buf + NSTAGE - 1) % NSTAGE);
      // paged: the block numbers of the tile after it (the wait at the next step
      // covers them, so the compiler's own wait before their use costs nothing)
      if (t + NSTAGE < n_tiles) load_tbl(k_begin + (t + NSTAGE) * KT, nkeys - 1);
    }
    if (active) compute(t, buf);
  };
  for (int t = 0; t < n_tiles; t += NSTAGE) {
#pragma unroll
    for (int j = 0; j < NSTAGE; ++j)
      if (t + j < n_tiles) step(t + j, j);
  }

  // ---- epilogue
  const float l_tot = l_part + __shfl_xor(l_part, 32, 64);
  if (r >= M) return;
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
        w2[0] = pack_bf16(acc[db][4 * v4 + 0] * inv, acc[db][4 * v4 + 1] * inv);
        w2[1] = pack_bf16(acc[db][4 * v4 + 2] * inv, acc[db][4 * v4 + 3] * inv);
        *reinterpret_cast<u32x2*>(op + d0) = w2;
      }
  } else {
    const long long prow = ((long long)bg * n_split + split) * m_pad + r;
    uint16_t* wp = ws_o + prow * D;
    // a split can see no key of a row (tree keys only, none an ancestor): l = 0
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int d0 = 32 * db + 8 * v4 + 4 * h;
        u32x2 w2;
        w2[0] = pack_bf16(acc[db][4 * v4 + 0] * inv, acc[db][4 * v4 + 1] * inv);
        w2[1] = pack_bf16(acc[db][4 * v4 + 2] * inv, acc[db][4 * v4 + 3] * inv);
        *reinterpret_cast<u32x2*>(wp + d0) = w2;
      }
    if (h == 0) {
      ws_ml[2 * prow] = m_run;
      ws_ml[2 * prow + 1] = l_tot;
    }
  }
}

// Merge split partials.  Split s left its normalised output o_s (bf16), its
// running max m_s (log2 domain) and its row sum l_s; the result is
// sum_s w_s o_s / sum_s w_s with w_s = exp2(m_s - max m) l_s.  Splits are read
// BATCH at a time (all loads in flight together; BATCH >= the split count up to
// 16, so a call with few splits issues no redundant loads) and merged online.
template <int D, int BATCH>
__global__ __launch_bounds__(256) void k_attn_combine(const uint16_t* __restrict__ ws_o,
                                                      const float* __restrict__ ws_ml,
                                                      const int* __restrict__ prefix_len,
                                                      const int* __restrict__ tree_size,
                                                      const int* __restrict__ status, long long S_cap, int T_max,
                                                      int Hq, int Hkv, int n_split, int chunk_keys, long long m_pad,
                                                      int rel, uint16_t* __restrict__ O) {
  typedef __bf16 h8 __attribute__((ext_vector_type(8)));
  constexpr int TPR = D / 8;          // threads per row, 8 outputs each
  constexpr int RPB = 256 / TPR;      // rows per block
  const int bg = blockIdx.x;
  const int b = bg / Hkv, g = bg % Hkv;
  const int rep = Hq / Hkv;
  const int r = blockIdx.y * RPB + threadIdx.x / TPR;  // < m_pad (a multiple of RPB)
  const int d0 = 8 * (threadIdx.x % TPR);
  const long long base = (long long)bg * n_split * m_pad + r;
  // the first batch of partials is requested together with the request's sizes
  // (one memory round trip): splits past the ones that saw keys are read (they
  // lie inside the workspace) but never used
  float ms[BATCH], ls[BATCH];
  h8 x[BATCH];
  auto load_batch = [&](int s0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const long long pr = base + (long long)min(s0 + j, n_split - 1) * m_pad;
      ms[j] = ws_ml[2 * pr];
      ls[j] = ws_ml[2 * pr + 1];
      x[j] = *reinterpret_cast<const h8*>(ws_o + pr * D + d0);
    }
  };
  load_batch(0);
  int T = tree_size[b];
  const int P = prefix_len[b];
  if (status[b] != TV_ST_OK || T < 1 || T > T_max) T = 1;
  if (P < 0 || (long long)P + T > S_cap) return;
  const int M = rep * T;
  if (r >= M) return;
  const int nkeys = P + T;
  // splits that saw keys (a prefix): the same partition as the attention kernel's
  const int n_act = rel ? min(n_split, (nkeys + KT - 1) / KT) : (nkeys + chunk_keys - 1) / chunk_keys;
  float mx = -INFINITY, l = 0.0f;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < n_act; s0 += BATCH) {
    if (s0 > 0) load_batch(s0);
    float bm = mx;
#pragma unroll
    for (int j = 0; j < BATCH; ++j)
      if (s0 + j < n_act) bm = fmaxf(bm, ms[j]);
    const float a = mx == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mx - bm);
    l *= a;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= a;
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      if (s0 + j < n_act && ms[j] != -INFINITY) {
        const float w = __builtin_amdgcn_exp2f(ms[j] - bm) * ls[j];
        l += w;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = fmaf(w, (float)x[j][e], o[e]);
      }
    }
    mx = bm;
  }
  const float inv = 1.0f / l;
  const int i = r / rep, head = g * rep + r % rep;
  uint16_t* op = O + (((long long)b * T_max + i) * Hq + head) * D + d0;
  *reinterpret_cast<u32x4*>(op) = u32x4{pack_bf16(o[0] * inv, o[1] * inv), pack_bf16(o[2] * inv, o[3] * inv),
                                        pack_bf16(o[4] * inv, o[5] * inv), pack_bf16(o[6] * inv, o[7] * inv)};
}

// fp32 path: one wavefront per (node, query head, request).
template <int D, bool PAGED, bool ROPE>
__global__ __launch_bounds__(64) void k_attn_fp32(const float* __restrict__ Q, const float* __restrict__ Kc,
                                                  const float* __restrict__ Vc, long long S_cap,
                                                  const int* __restrict__ prefix_len,
                                                  const int* __restrict__ tree_size,
                                                  const uint32_t* __restrict__ tree_mask,
                                                  const int* __restrict__ status, int T_max, int Hq, int Hkv, int W,
                                                  float scale, float* __restrict__ O, Paging pg, Rope rope) {
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
  // row offset of key `key` (linear, or through the block table as in k_attn_bf16)
  auto row = [&](int key) -> long long {
    if constexpr (PAGED) {
      const long long e = pg.table[(long long)b * pg.max_blocks + (key >> pg.lbs)];
      const long long blk = min(max(e, 0ll), pg.n_blocks - 1);
      return (((blk * Hkv + g) << pg.lbs) + (key & ((1 << pg.lbs) - 1))) * D;
    } else {
      return (((long long)b * Hkv + g) * S_cap + key) * D;
    }
  };
  const uint32_t* mp = tree_mask + ((long long)b * T_max + i) * W;
  __shared__ float s_q[D];
  if constexpr (ROPE) {
    // the query before its rotary embedding: pair (j, j + D/2) turns at P + depth
    int anc = 0;
    for (int w = 0; w < W; ++w) anc += __popc(mp[w]);
    const float posf = (float)(P + anc - 1);
    for (int j = lane; j < D / 2; j += 64) {
      const float p = posf * rope.f_hi[j];
      const float rev = (p - rintf(p)) + (fmaf(posf, rope.f_hi[j], -p) + posf * rope.f_lo[j]);
      const float sn = __builtin_amdgcn_sinf(rev), cs = __builtin_amdgcn_cosf(rev);
      const float a = qp[j], o = qp[j + D / 2];
      s_q[j] = fmaf(a, cs, -o * sn);
      s_q[j + D / 2] = fmaf(o, cs, a * sn);
    }
  } else {
    for (int d = lane; d < D; d += 64) s_q[d] = qp[d];
  }
  __syncthreads();
  float m = -INFINITY, l = 0.0f, acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.0f;
  for (int key = lane; key < nkeys; key += 64) {
    if (!(key < P || ((mp[(key - P) >> 5] >> ((key - P) & 31)) & 1u))) continue;
    const long long ro = row(key);
    const float* kr = Kc + ro;
    float sc = 0.0f;
#pragma unroll
    for (int d = 0; d < D; ++d) sc = fmaf(s_q[d], kr[d], sc);
    sc *= scale;
    const float mn = fmaxf(m, sc);
    const float a = expf(m - mn);  // m = -inf -> 0
    const float p = expf(sc - mn);
    const float* vr = Vc + ro;
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

template <int D, int NW, int NS, bool PAGED, bool ROPE>
void launch_bf16(const Plan& p, int B, hipStream_t s, const void* Q, const void* Kc, const void* Vc, long long S_cap,
                 const int* prefix_len, const int* tree_size, const uint32_t* tree_mask, const int* status,
                 int T_max, int Hq, int Hkv, int W, float sl2, void* O, uint16_t* ws_o, float* ws_ml,
                 const Paging& pg, const Rope& rope) {
  hipLaunchKernelGGL((k_attn_bf16<D, NW, NS, PAGED, ROPE>), dim3(p.grid), dim3(NW * 64), 0, s, (const uint16_t*)Q,
                     (const uint16_t*)Kc, (const uint16_t*)Vc, S_cap, prefix_len, tree_size, tree_mask, status, T_max,
                     Hq, Hkv, W, sl2, (uint16_t*)O, ws_o, ws_ml, p.n_split, p.chunk_keys, p.n_rowblk, p.n_units,
                     p.m_pad, B, p.rel, pg, rope);
}

size_t ws_bytes_for(const Plan& p, int B, int Hkv, int d) {
  if (p.n_split <= 1) return 0;
  return (size_t)B * Hkv * p.n_split * p.m_pad * ((size_t)d * sizeof(uint16_t) + 2 * sizeof(float)) + 256;
}

// Both entry points: S_cap is the rows each request can hold (the linear slab, or
// max_blocks << lbs with a block table).
int attention_impl(int dtype, int B, int T_max, int Hq, int Hkv, int d, const void* Q, const void* Kc,
                   const void* Vc, long long S_cap, const int* prefix_len, const int* tree_size,
                   const uint32_t* tree_mask, const int* status, float scale, void* O, void* workspace,
                   size_t ws_bytes, void* stream, const Paging& pg, const Rope* rope = nullptr) {
  if (B <= 0 || T_max <= 0 || Hq <= 0 || Hkv <= 0 || S_cap <= 0) return TV_EINVAL;
  if (Hq % Hkv != 0) return TV_EINVAL;
  if (S_cap > (1LL << 30)) return TV_EUNSUPPORTED;
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
  const bool paged = pg.table != nullptr;
  const Rope rp = rope ? *rope : Rope{};
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dtype == TV_DTYPE_FP32) {
    dim3 grid(T_max, Hq, B);
    if (B > 65535 || Hq > 65535) return TV_EUNSUPPORTED;
#define TV_FP32_LAUNCH(DD, PG, RP)                                                                                 \
  hipLaunchKernelGGL((k_attn_fp32<DD, PG, RP>), grid, dim3(64), 0, s, (const float*)Q, (const float*)Kc,            \
                     (const float*)Vc, S_cap, prefix_len, tree_size, tree_mask, status, T_max, Hq, Hkv, W, scale,    \
                     (float*)O, pg, rp)
    if (d == 64) {
      if (paged) TV_FP32_LAUNCH(64, true, false);
      else if (rope) TV_FP32_LAUNCH(64, false, true);
      else TV_FP32_LAUNCH(64, false, false);
    } else {
      if (paged) TV_FP32_LAUNCH(128, true, false);
      else if (rope) TV_FP32_LAUNCH(128, false, true);
      else TV_FP32_LAUNCH(128, false, false);
    }
#undef TV_FP32_LAUNCH
    TV_CHECK_LAUNCH();
    return TV_OK;
  }
  const Plan p = make_plan(B, T_max, Hq, Hkv, S_cap);
  const size_t need = ws_bytes_for(p, B, Hkv, d);
  if (need && (!workspace || ws_bytes < need)) return TV_EWORKSPACE;
  uint16_t* ws_o = reinterpret_cast<uint16_t*>(workspace);
  float* ws_ml = need ? reinterpret_cast<float*>(ws_o + (size_t)B * Hkv * p.n_split * p.m_pad * d) : nullptr;
  const float sl2 = scale * kLog2e;
#define TV_ATTN_LAUNCH(DD, NWW, NSS, PG, RP)                                                                     \
  launch_bf16<DD, NWW, NSS, PG, RP>(p, B, s, Q, Kc, Vc, S_cap, prefix_len, tree_size, tree_mask, status, T_max, Hq, \
                                    Hkv, W, sl2, O, ws_o, ws_ml, pg, rp)
#define TV_ATTN_NW(DD, PG, RP)           \
  if (p.nw == 4) TV_ATTN_LAUNCH(DD, 4, 2, PG, RP); \
  else TV_ATTN_LAUNCH(DD, 8, 2, PG, RP)
  if (d == 128) {
    if (paged) TV_ATTN_NW(128, true, false);
    else if (rope) TV_ATTN_NW(128, false, true);
    else TV_ATTN_NW(128, false, false);
  } else {
    if (paged) TV_ATTN_NW(64, true, false);
    else if (rope) TV_ATTN_NW(64, false, true);
    else TV_ATTN_NW(64, false, false);
  }
#undef TV_ATTN_NW
#undef TV_ATTN_LAUNCH
  TV_CHECK_LAUNCH();
  if (p.n_split > 1) {
    const int rpb = 256 / (d / 8);
    dim3 grid(B * Hkv, (unsigned)((p.m_pad + rpb - 1) / rpb));
#define TV_COMBINE(DD, BB)                                                                                         \
  hipLaunchKernelGGL((k_attn_combine<DD, BB>), grid, dim3(256), 0, s, ws_o, ws_ml, prefix_len, tree_size, status,   \
                     S_cap, T_max, Hq, Hkv, p.n_split, p.chunk_keys, p.m_pad, p.rel, (uint16_t*)O)
    if (d == 128) {
      if (p.n_split <= 4) TV_COMBINE(128, 4);
      else if (p.n_split <= 8) TV_COMBINE(128, 8);
      else TV_COMBINE(128, 16);
    } else {
      if (p.n_split <= 4) TV_COMBINE(64, 4);
      else if (p.n_split <= 8) TV_COMBINE(64, 8);
      else TV_COMBINE(64, 16);
    }
#undef TV_COMBINE
    TV_CHECK_LAUNCH();
  }
  return TV_OK;
}

}  // namespace
}  // namespace tv

namespace tv {
constexpr size_t kScratchBytes = 64ull << 20;
}

// Scratch of tree_attention_noalloc: the split-KV partials live in this
// file-scope device array instead of a caller workspace.  Each GPU the library
// runs on holds its own copy (64 MiB) until the process ends.  Host code never
// passes the array's name to a kernel: on the host it is a stand-in, not a device
// address.  Its address on each device comes from hipGetSymbolAddress, taken
// once per device with that device current, and is used instead.
static __device__ __align__(256) unsigned char scratch[tv::kScratchBytes];

namespace tv {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// the current device's address of `scratch` (nullptr on failure)
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
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
  return tv::attention_impl(dtype, B, T_max, Hq, Hkv, d, Q, Kc, Vc, S_cap, prefix_len, tree_size, tree_mask, status,
                            scale, O, workspace, ws_bytes, stream, tv::Paging{});
}

extern "C" size_t tree_attention_noalloc_max_bytes(void) { return tv::kScratchBytes; }

extern "C" int tree_attention_noalloc(int dtype, int B, int T_max, int Hq, int Hkv, int d, const void* Q,
                                      const void* Kc, const void* Vc, long long S_cap, const int* prefix_len,
                                      const int* tree_size, const uint32_t* tree_mask, const int* status,
                                      float scale, void* O, void* stream) {
  // the sizes are checked on the host first: a call whose split partials would not
  // fit the scratch array is refused before any device call
  if (dtype == TV_DTYPE_BF16 && B > 0 && T_max > 0 && Hq > 0 && Hkv > 0 && Hq % Hkv == 0 && S_cap > 0 &&
      tree_attention_workspace_bytes(dtype, B, T_max, Hq, Hkv, d, S_cap) > tv::kScratchBytes)
    return TV_EWORKSPACE;
  void* ws = nullptr;
  if (dtype == TV_DTYPE_BF16 && tree_attention_workspace_bytes(dtype, B, T_max, Hq, Hkv, d, S_cap) > 0) {
    ws = tv::scratch_on_current_device();
    if (!ws) return TV_ELAUNCH;
  }
  return tv::attention_impl(dtype, B, T_max, Hq, Hkv, d, Q, Kc, Vc, S_cap, prefix_len, tree_size, tree_mask, status,
                            scale, O, ws, ws ? tv::kScratchBytes : 0, stream, tv::Paging{});
}

extern "C" int tree_attention_rope(int dtype, int B, int T_max, int Hq, int Hkv, int d, const void* Q,
                                   const void* Kc, const void* Vc, long long S_cap, const int* prefix_len,
                                   const int* tree_size, const uint32_t* tree_mask, const int* status,
                                   float rope_theta, float scale, void* O, void* workspace, size_t ws_bytes,
                                   void* stream) {
  if (!(rope_theta > 1.0f) || !(rope_theta < 3.0e38f)) return TV_EINVAL;
  if (S_cap > (1LL << 24)) return TV_EUNSUPPORTED;  // positions stay exact in float32
  if (d != 64 && d != 128) return TV_EUNSUPPORTED;
  tv::Rope rope{};
  const double two_pi = 6.283185307179586476925286766559;
  for (int i = 0; i < d / 2; ++i) {
    const double f = pow((double)rope_theta, -2.0 * i / d) / two_pi;
    rope.f_hi[i] = (float)f;
    rope.f_lo[i] = (float)(f - (double)rope.f_hi[i]);
  }
  return tv::attention_impl(dtype, B, T_max, Hq, Hkv, d, Q, Kc, Vc, S_cap, prefix_len, tree_size, tree_mask, status,
                            scale, O, workspace, ws_bytes, stream, tv::Paging{}, &rope);
}

extern "C" int tree_attention_paged(int dtype, int B, int T_max, int Hq, int Hkv, int d, const void* Q,
                                    const void* K_pool, const void* V_pool, long long num_blocks,
                                    int tokens_per_block, const int* block_table, int max_blocks_per_seq,
                                    const int* prefix_len, const int* tree_size, const uint32_t* tree_mask,
                                    const int* status, float scale, void* O, void* workspace, size_t ws_bytes,
                                    void* stream) {
  const int lbs = tv::log2_block(tokens_per_block);
  if (lbs < 0 || !block_table || max_blocks_per_seq <= 0 || num_blocks <= 0 || Hkv <= 0) return TV_EINVAL;
  if ((long long)B * max_blocks_per_seq > (1LL << 31)) return TV_EINVAL;
  // pool rows (num_blocks * Hkv * tokens_per_block) are addressed with 64-bit offsets
  if (num_blocks > (1LL << 40) / ((long long)Hkv * tokens_per_block)) return TV_EINVAL;
  const long long cap = (long long)max_blocks_per_seq << lbs;
  return tv::attention_impl(dtype, B, T_max, Hq, Hkv, d, Q, K_pool, V_pool, cap, prefix_len, tree_size, tree_mask,
                            status, scale, O, workspace, ws_bytes, stream,
                            tv::Paging{block_table, max_blocks_per_seq, lbs, num_blocks});
}
