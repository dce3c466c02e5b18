// Attention kernels of In-context Sparse Attention on gfx950.
//
// One tile engine serves three callers:
//   * sharp path (paper.rainbus.top summary of arXiv 2605.04569, "Method
//     steps", step (4)): exact softmax attention of the sharp query blocks
//     over the tokens of the kept blocks J, read through block indices (no
//     gather copy);
//   * flat path (same section, step (5), and the 0th-order Taylor paragraph
//     of "Prerequisites"): exact attention over the tokens of E_i, then the
//     pooled keys of J \ E_i, each with additive logit log(n_j) so that block
//     j contributes n_j * exp(q.Kc_j / sqrt(D)) to the denominator and that
//     weight times Vc_j to the numerator; both kinds of key tiles feed one
//     online-softmax accumulator (running max, sum, output);
//   * dense baseline: every token attends every token.
//
// Work decomposition (CDNA4, wave64):
//   * a workgroup owns ROWS query rows; each wave owns 16*QT rows (for
//     32-token flat blocks two waves share each row group, one per 32-key
//     half of every tile, and merge their softmax states at the end);
//   * key tiles of 64 keys are copied into LDS by buffer loads (no register
//     staging); in the pipelined paths the copy of a later tile is in flight
//     while the current one is consumed, in the flat path the other resident
//     workgroups cover the copy's latency;
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (A = K rows from LDS, B = Q
//     fragments kept in registers); lane (g = lane/16, c = lane%16) then holds
//     4 keys of each 16-key sub-tile for query c, so the row max needs only
//     two cross-lane swaps (v_permlane16/32_swap) and the row sum none until
//     the end;
//   * the probabilities, rounded to bf16, are already in the B-operand layout
//     of O^T += V^T P^T; the V^T operand comes from row-major V in LDS through
//     the transposing LDS read ds_read_b64_tr_b16;
//   * O^T accumulates in fp32 with one query per lane, so the online-softmax
//     rescale is a per-lane scalar multiply, skipped unless some row max grew
//     by more than 2^8 (the running max is a reference, not the exact max);
//   * exp is exp2 with log2(e)/sqrt(D) folded into the exponent's fma.
// The sharp and dense paths are software pipelined: while the softmax of
// tile t runs on the vector ALUs, the matrix cores already compute the scores
// of tile t+1; K and V are triple buffered in LDS and copied there straight
// from global memory (buffer_load_dwordx4 ... lds: no register staging, no
// LDS store instructions, no vector address arithmetic) two tiles ahead,
// one workgroup barrier per tile. Tiles
// that need additive logits (padding, partial blocks) are ordered last so
// the steady state runs without them.
// K and V rows are padded to 2D+32 bytes in LDS; with that stride the 16-byte
// K reads and the 8-byte transposing V reads measure free of bank conflicts.
#include "isa_internal.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(16)));
typedef short short4_t __attribute__((__vector_size__(8)));
typedef float float4_t __attribute__((__vector_size__(16)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
struct bf16x2x4_t { bf16x2_t a, b, c, d; };

enum : int { kDense = 0, kSharp = 1, kFlat = 2 };

constexpr int kKeyTile = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;   // log2 units
constexpr float kMinusBig = -1.0e30f;
__device__ constexpr bf16x2_t kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

struct AttnArgs {
  IsaShape s;                // dense: B, H, L, D only
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  uint16_t* O;
  const uint16_t* kcb;       // flat: bf16 block means of K  [B,H,N,D]
  const uint16_t* vcb;       // flat: bf16 block means of V  [B,H,N,D]
  const int32_t* ctx_idx;    // [B,H,k_ctx] kept context blocks (global ids)
  const int32_t* qlist;      // sharp_idx or flat_idx [B,H,n_q]
  const int32_t* exact;      // flat: [B,H,n_flat,k_ns]
  const int32_t* flat_ord;   // flat: [B,H,n_flat] grid order of the rows (nullable: plain order)
  float* lse;                // optional [B,H,L]: log2 of each row's softmax denominator
  int n_q;
  int ntiles_exact;
  int ntiles;
  int ntiles_plain;          // sharp/dense: leading tiles with no additive logit
};

__device__ inline float xor16_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float xor32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float xor16_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float xor32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline short4_t lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4_t*)(p));
}

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// Global block id of position q of the kept list J (source blocks, then the
// kept context blocks); -1 when out of range.
__device__ inline int kept_id(const IsaShape& s, const int32_t* ctx_row, int q) {
  if (q < s.N_src) return q;
  const int j = ctx_row[q - s.N_src];
  return (j >= s.N_src && j < s.N) ? j : -1;
}

// Where the keys of one tile come from (per workgroup, read-only).
struct TileCtx {
  const uint16_t* K;      // token rows of this (batch, head)
  const uint16_t* V;
  const uint16_t* kc;     // flat: bf16 block means of this (batch, head)
  const uint16_t* vc;
  const int* tab;         // LDS: packed (start << 7) | n per listed block
  const int* ptab;        // LDS (flat): (j << 8) | (n << 1) | in_E per kept block
  int ntab, L, N_kv, b, lb, per, ntiles_exact;
};

// One key slot: row pointers that are always safe to read, whether the slot
// holds a real key, and its additive logit in log2 units.
struct SlotSrc {
  const uint16_t* k;
  const uint16_t* v;
  bool valid;
  float bias;
};

template <int D, int MODE>
__device__ inline SlotSrc slot_src(const TileCtx& c, int t, int slot) {
  SlotSrc r;
  if (MODE == kDense) {
    const int tok = t * kKeyTile + slot;
    r.valid = tok < c.L;
    const size_t row = (size_t)(r.valid ? tok : 0) * D;
    r.k = c.K + row;
    r.v = c.V + row;
    r.bias = r.valid ? 0.0f : -INFINITY;
    return r;
  }
  if (MODE == kFlat && t >= c.ntiles_exact) {
    const int p = (t - c.ntiles_exact) * kKeyTile + slot;
    const int e = p < c.N_kv ? c.ptab[p] : 1;
    const int n = (e >> 1) & 127;
    r.valid = !(e & 1) && n > 0;
    const size_t row = (size_t)(r.valid ? (e >> 8) : 0) * D;
    r.k = c.kc + row;
    r.v = c.vc + row;
    r.bias = r.valid ? __log2f((float)n) : -INFINITY;
    return r;
  }
  const int q = t * c.per + (slot >> c.lb), o = slot & (c.b - 1);
  const int e = q < c.ntab ? c.tab[q] : 0;
  r.valid = o < (e & 127);
  const size_t row = (size_t)(r.valid ? (e >> 7) + o : 0) * D;
  r.k = c.K + row;
  r.v = c.V + row;
  r.bias = r.valid ? 0.0f : -INFINITY;
  return r;
}

// Whether tile t carries any non-zero additive logit (uniform over the
// workgroup).
template <int MODE>
__device__ inline bool tile_has_bias(const TileCtx& c, int t) {
  if (MODE == kDense) return (t + 1) * kKeyTile > c.L;
  if (MODE == kFlat && t >= c.ntiles_exact) return true;
  bool any = false;
  for (int u = 0; u < c.per; ++u) {
    const int q = t * c.per + u;
    const int e = q < c.ntab ? c.tab[q] : 0;
    any |= (e & 127) < c.b;
  }
  return any;
}

// ---------------------------------------------------------------- tile math
// S^T tile: s[qt][mt][j] = K[16mt + 4g + j] . Q[16qt + c] for the 16*NMT
// keys of the LDS tile at `kb` (raw dot products).
template <int D, int QT, int NMT = 4>
__device__ __forceinline__ void qk_tile(const char* kb, const bf16x8_t (&qf)[QT][D / 32],
                                        float4_t (&s)[QT][NMT], int g, int c16) {
  constexpr int KSTR = 2 * D + 32;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) s[qt][mt] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(kb + (16 * mt + c16) * KSTR + (32 * kk + 8 * g) * 2);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
        s[qt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[qt][kk], s[qt][mt], 0, 0, 0);
    }
  }
}

// Turns raw scores into log2-unit logits with the per-key offsets.
template <int QT, int NMT = 4>
__device__ __forceinline__ void apply_logit_offsets(float4_t (&s)[QT][NMT], const float* bias,
                                                    float cscale, int g) {
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    const float4_t bv = *reinterpret_cast<const float4_t*>(bias + 16 * mt + 4 * g);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int j = 0; j < 4; ++j) s[qt][mt][j] = __builtin_fmaf(s[qt][mt][j], cscale, bv[j]);
  }
}

// Row maximum over the 16*NMT keys of the tile, times `xs` (log2 units).
template <int QT, int NMT = 4>
__device__ __forceinline__ void row_max(const float4_t (&s)[QT][NMT], float xs, float (&mx)[QT]) {
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    float a;
    if (NMT == 4) {
      a = __builtin_fmaxf(s[qt][0][0], __builtin_fmaxf(s[qt][0][1], s[qt][0][2]));
      a = __builtin_fmaxf(a, __builtin_fmaxf(s[qt][0][3], s[qt][1][0]));
      a = __builtin_fmaxf(a, __builtin_fmaxf(s[qt][1][1], s[qt][1][2]));
      a = __builtin_fmaxf(a, __builtin_fmaxf(s[qt][1][3], s[qt][2][0]));
      a = __builtin_fmaxf(a, __builtin_fmaxf(s[qt][2][1], s[qt][2][2]));
      a = __builtin_fmaxf(a, __builtin_fmaxf(s[qt][2][3], s[qt][3][0]));
      a = __builtin_fmaxf(a, __builtin_fmaxf(s[qt][3][1], s[qt][3][2]));
      a = __builtin_fmaxf(a, s[qt][3][3]);
    } else {
      // pairs (i, i+1) of the 4*NMT held values, one three-way max each
      a = s[qt][0][0];
#pragma unroll
      for (int i = 1; i < 4 * NMT; i += 2) {
        const float x = s[qt][i >> 2][i & 3];
        a = (i + 1 < 4 * NMT) ? __builtin_fmaxf(a, __builtin_fmaxf(x, s[qt][(i + 1) >> 2][(i + 1) & 3]))
                              : __builtin_fmaxf(a, x);
      }
    }
    a = xor16_max(a);
    a = xor32_max(a);
    mx[qt] = a * xs;
  }
}

// Lazy online-softmax rescale: only when some row max exceeds the running
// reference by more than kRescaleSlack (wave-uniform branch).
template <int D, int QT>
__device__ __forceinline__ void rescale(const float (&mx)[QT], float (&m)[QT], float (&lsum)[QT],
                                        float4_t (&o)[QT][D / 16]) {
  bool need = false;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) need |= mx[qt] > m[qt] + kRescaleSlack;
  if (__ballot(need)) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float mn = fmaxf(m[qt], mx[qt]);
      const float alpha = __builtin_amdgcn_exp2f(m[qt] - mn);
      lsum[qt] *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) o[qt][dt] *= alpha;
      m[qt] = mn;
    }
  }
}

// p = exp2(s*xs - m), rounded to bf16 and packed as the B operand of the PV
// product; the per-lane partial row sums accumulate the rounded values.
template <int QT, int NMT = 4>
__device__ __forceinline__ void exp_pack(const float4_t (&s)[QT][NMT], float xs, const float (&m)[QT],
                                         float (&lsum)[QT], bf16x8_t (&pb)[QT][NMT / 2]) {
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float negm = -m[qt];
    float ps = lsum[qt];
#pragma unroll
    for (int kc = 0; kc < NMT / 2; ++kc) {
      bf16x2_t h[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i0 = 8 * kc + 2 * u;   // element index within the 16 held values
        const float x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qt][i0 >> 2][i0 & 3], xs, negm));
        const float x1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qt][(i0 + 1) >> 2][(i0 + 1) & 3], xs, negm));
        h[u] = __builtin_convertvector((float2_t){x0, x1}, bf16x2_t);
        ps = __builtin_amdgcn_fdot2_f32_bf16(h[u], kOnes2, ps, false);
      }
      pb[qt][kc] = __builtin_bit_cast(bf16x8_t, (bf16x2x4_t){h[0], h[1], h[2], h[3]});
    }
    lsum[qt] = ps;
  }
}

// log2-domain log-sum-exp of each owned row (m is the running reference of
// the logits in log2 units, lsum the row's partial sums), kept for the
// backward pass.
template <int QT>
__device__ __forceinline__ void save_lse(float* lse, size_t head, const int (&qtok)[QT],
                                         const bool (&qval)[QT], const float (&m)[QT],
                                         const float (&lsum)[QT], int g) {
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    float lt = xor16_sum(lsum[qt]);
    lt = xor32_sum(lt);
    if (qval[qt] && g == 0) lse[head + qtok[qt]] = m[qt] + __log2f(lt);
  }
}

// O^T += V^T P^T for the 16*NMT keys of the LDS tile at `vb`.
template <int D, int QT, int NMT = 4>
__device__ __forceinline__ void pv_tile(const char* vb, const bf16x8_t (&pb)[QT][NMT / 2],
                                        float4_t (&o)[QT][D / 16], int g, int c16) {
  constexpr int VSTR = 2 * D + 32;
  const int tr_row = 4 * g + (c16 >> 2);
  const int tr_col = 4 * (c16 & 3);
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
#pragma unroll
    for (int kc = 0; kc < NMT / 2; ++kc) {
      const short4_t lo = lds_read_tr(vb + (32 * kc + tr_row) * VSTR + (16 * dt + tr_col) * 2);
      const short4_t hi = lds_read_tr(vb + (32 * kc + 16 + tr_row) * VSTR + (16 * dt + tr_col) * 2);
      const bf16x8_t va = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
        o[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[qt][kc], o[qt][dt], 0, 0, 0);
    }
  }
}

// PIPE: software pipelined (scores of the next tile overlap the softmax of
// the current one; K and V triple-buffered, copied global->LDS directly),
// else one LDS buffer, also filled global->LDS directly, with the copy
// latency hidden by the other resident workgroups.
// KS = 2 (flat path only): the waves split each key tile in two halves of 32
// keys, each half with its own online-softmax state for the same rows, merged
// at the end; twice the waves per workgroup for the same LDS.
// (The key-split flat kernel is held to three workgroups per compute unit
// by its LDS, so it may use the registers of three waves per SIMD.)
template <int D, int MODE, int QT, int NWAVES, bool PIPE, int KS = 1>
__global__ __launch_bounds__(NWAVES * 64) __attribute__((amdgpu_waves_per_eu(PIPE ? 2 : (KS == 2 ? 3 : 4))))
void attn_kernel(AttnArgs a) {
  static_assert(KS == 1 || (KS == 2 && !PIPE && MODE == kFlat && NWAVES % 2 == 0), "key split");
  constexpr int NT = NWAVES * 64;
  constexpr int KSTR = 2 * D + 32;
  constexpr int VSTR = 2 * D + 32;
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int CH = kKeyTile * CPR / NT;    // chunks per thread per tensor
  constexpr int ROWS_W = 16 * QT;
  constexpr int RW = NWAVES / KS;            // waves per key-split half
  constexpr int ROWS = RW * ROWS_W;
  constexpr int KK = D / 32;
  constexpr int DT = D / 16;
  static_assert(CH >= 1 && (kKeyTile * CPR) % NT == 0, "tile split");
  static_assert(NT % CPR == 0, "chunk column must be fixed per thread");

  // Buffer 0 of K and V (the tail and non-pipelined paths use only these);
  // the pipelined path adds two more of each as separate arrays, so that the
  // compiler can tell the asynchronous global->LDS copies into one buffer
  // apart from the reads of another.
  __shared__ __attribute__((aligned(16))) char k_lds[1][kKeyTile * KSTR];
  __shared__ __attribute__((aligned(16))) char v_lds[1][kKeyTile * VSTR];
  __shared__ __attribute__((aligned(16))) char k_ld1[PIPE ? kKeyTile * KSTR : 16];
  __shared__ __attribute__((aligned(16))) char k_ld2[PIPE ? kKeyTile * KSTR : 16];
  __shared__ __attribute__((aligned(16))) char v_ld1[PIPE ? kKeyTile * VSTR : 16];
  __shared__ __attribute__((aligned(16))) char v_ld2[PIPE ? kKeyTile * VSTR : 16];
  __shared__ __attribute__((aligned(16))) float bias_lds[1][kKeyTile];
  // Sharp path: token range of every kept block, packed (start << 7) | n_j,
  // indexed by position in J. Flat path (dynamic LDS): the same for E_i, then
  // (j << 8) | (n_j << 1) | in_E for every position of J.
  __shared__ int jtab[MODE == kSharp ? ISA_MAX_NKV : 1];
  extern __shared__ int dyn_lds[];

  const IsaShape& s = a.s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int rwave = wave % RW, kh = wave / RW;   // row group, key half
  // Workgroups are dispatched round-robin over the 8 XCDs (each with its own
  // L2). For the sharp and dense paths, whose workgroups of one head stream
  // the same K/V, the dispatch index is remapped so that each XCD receives a
  // contiguous run of tiles, i.e. mostly one head at a time. The flat
  // kernel for 32-token blocks (twice the blocks, each gathering its own
  // exact set) takes the same order: it doubles its L2 hit rate when the
  // exact sets are large; the 64-token flat kernel keeps the plain order
  // unless the flat blocks come with a grid order (flat_ord: blocks whose
  // exact sets overlap next to each other), which each XCD's run follows.
  int tile_x = blockIdx.x, bh = blockIdx.y;
  const bool ordered = MODE == kFlat && a.flat_ord != nullptr;
  if (MODE != kFlat || KS == 2 || ordered) {
    const int total = gridDim.x * gridDim.y;
    if ((total & 7) == 0) {
      const int id = blockIdx.x + gridDim.x * blockIdx.y;
      const int logical = (id & 7) * (total >> 3) + (id >> 3);
      tile_x = logical % gridDim.x;
      bh = logical / gridDim.x;
    }
  }
  if (ordered) tile_x = __builtin_amdgcn_readfirstlane(a.flat_ord[(size_t)bh * s.n_flat + tile_x]);
  const size_t head = (size_t)bh * s.L;     // first token row of this (batch, head)
  const int32_t* ctx_row = a.ctx_idx + (size_t)bh * s.k_ctx;
  const int b = s.b;
  const int lb = b == 64 ? 6 : 5;

  // ---- query rows owned by this lane
  int qtok[QT];
  bool qval[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int lr = rwave * ROWS_W + 16 * qt + c16;
    qval[qt] = false;
    qtok[qt] = 0;
    if (MODE == kDense) {
      const int tok = tile_x * ROWS + lr;
      qval[qt] = tok < s.L;
      qtok[qt] = tok;
    } else {
      const int e = (MODE == kSharp) ? tile_x * (ROWS >> lb) + (lr >> lb) : tile_x;
      const int o = (MODE == kSharp) ? (lr & (b - 1)) : lr;
      if (e < a.n_q) {
        const int j = a.qlist[(size_t)bh * a.n_q + e];
        if (j >= 0 && j < s.N) {
          int st, n;
          isa_block_range(s, j, st, n);
          qval[qt] = o < n;
          qtok[qt] = st + o;
        }
      }
    }
  }

  bf16x8_t qf[QT][KK];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (qval[qt]) w = *reinterpret_cast<const uint4*>(a.Q + (head + qtok[qt]) * D + 32 * kk + 8 * g);
      qf[qt][kk] = __builtin_bit_cast(bf16x8_t, w);
    }
  }

  int* etab = dyn_lds;                            // flat: [k_ns]
  int* ptab = dyn_lds + (MODE == kFlat ? s.k_ns : 0);   // flat: [N_kv]
  if (MODE == kSharp) {
    // Kept blocks in J order, except that the (at most two) partial blocks
    // move to the end: the last source block and, if kept, the last context
    // block, whose positions in J are N_src-1 and N_kv-1.
    const int p1 = (s.L_src % b) ? s.N_src - 1 : -1;
    const int p2 = (s.L_ctx % b && s.k_ctx > 0 && ctx_row[s.k_ctx - 1] == s.N - 1) ? s.N_kv - 1 : -1;
    const int npart = (p1 >= 0) + (p2 >= 0);
    for (int q = tid; q < s.N_kv; q += NT) {
      const int j = kept_id(s, ctx_row, q);
      int st = 0, n = 0;
      if (j >= 0) isa_block_range(s, j, st, n);
      int dest;
      if (q == p1) dest = s.N_kv - npart;
      else if (q == p2) dest = s.N_kv - 1;
      else dest = q - ((p1 >= 0 && q > p1) ? 1 : 0);
      jtab[dest] = (st << 7) | n;
    }
    __syncthreads();
  } else if (MODE == kFlat) {
    const int32_t* exact_row = a.exact + ((size_t)bh * s.n_flat + tile_x) * s.k_ns;
    for (int q = tid; q < s.k_ns; q += NT) {
      const int j = exact_row[q];
      int st = 0, n = 0;
      if (j >= 0 && j < s.N) isa_block_range(s, j, st, n);
      etab[q] = (st << 7) | n;
    }
    for (int p = tid; p < s.N_kv; p += NT) {
      const int j = kept_id(s, ctx_row, p);
      int st = 0, n = 0;
      if (j >= 0) isa_block_range(s, j, st, n);
      ptab[p] = j >= 0 ? ((j << 8) | (n << 1)) : 1;
    }
    __syncthreads();
    for (int q = tid; q < s.k_ns; q += NT) {
      const int j = exact_row[q];
      int p = -1;
      if (j >= 0 && j < s.N_src) {
        p = j;
      } else if (j >= s.N_src && j < s.N) {
        int lo = 0, hi = s.k_ctx;     // lower bound of j in the ascending kept list
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (ctx_row[mid] < j) lo = mid + 1; else hi = mid;
        }
        if (lo < s.k_ctx && ctx_row[lo] == j) p = s.N_src + lo;
      }
      if (p >= 0) ptab[p] |= 1;
    }
    __syncthreads();
  }

  // ---- key tile source
  const int per = kKeyTile >> lb;   // blocks per key tile (exact tiles)
  TileCtx tc;
  tc.K = a.K + head * D;
  tc.V = a.V + head * D;
  tc.kc = (MODE == kFlat) ? a.kcb + (size_t)bh * s.N * D : nullptr;
  tc.vc = (MODE == kFlat) ? a.vcb + (size_t)bh * s.N * D : nullptr;
  tc.tab = (MODE == kSharp) ? jtab : etab;
  tc.ptab = ptab;
  tc.ntab = (MODE == kSharp) ? s.N_kv : s.k_ns;
  tc.L = s.L;
  tc.N_kv = s.N_kv;
  tc.b = b;
  tc.lb = lb;
  tc.per = per;
  tc.ntiles_exact = a.ntiles_exact;

  uint4 kr[CH], vr[CH];
  float br[CH];
  uint32_t vmask[CH];     // all ones for a real key, zero for padding
  const int c8 = tid % CPR;

#define ISA_LOAD_TILE(T)                                                        \
  _Pragma("unroll") for (int i = 0; i < CH; ++i) {                              \
    const SlotSrc ss = slot_src<D, MODE>(tc, (T), (tid + i * NT) / CPR);        \
    vmask[i] = ss.valid ? 0xffffffffu : 0u;                                     \
    br[i] = ss.bias;                                                            \
    kr[i] = *reinterpret_cast<const uint4*>(ss.k + c8 * 8);                     \
    vr[i] = *reinterpret_cast<const uint4*>(ss.v + c8 * 8);                     \
  }
#define ISA_STORE_TILE(KB, VB)                                                  \
  _Pragma("unroll") for (int i = 0; i < CH; ++i) {                              \
    const int slot = (tid + i * NT) / CPR;                                      \
    const uint32_t m = vmask[i];                                                \
    *reinterpret_cast<uint4*>(&k_lds[(KB)][slot * KSTR + c8 * 16]) =            \
        make_uint4(kr[i].x & m, kr[i].y & m, kr[i].z & m, kr[i].w & m);         \
    *reinterpret_cast<uint4*>(&v_lds[(VB)][slot * VSTR + c8 * 16]) =            \
        make_uint4(vr[i].x & m, vr[i].y & m, vr[i].z & m, vr[i].w & m);         \
    if (c8 == 0) bias_lds[(VB)][slot] = br[i];                                  \
  }

  const float cscale = kLog2e / sqrtf((float)D);
  float m[QT], lsum[QT];
  float4_t oacc[QT][DT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m[qt] = kMinusBig;
    lsum[qt] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[qt][dt] = float4_t{0.f, 0.f, 0.f, 0.f};
  }
  const int ntiles = a.ntiles;
  bf16x8_t pb[QT][2];

  if (!PIPE) {
    // One LDS buffer; latency is hidden by the other workgroups resident on
    // the compute unit (small register and LDS footprint). With the key
    // split each wave takes NMT 16-key sub-tiles of every tile.
    constexpr int NMT = 4 / KS;
    const char* kb = k_lds[0] + kh * 16 * NMT * KSTR;
    const char* vb = v_lds[0] + kh * 16 * NMT * VSTR;
    const float* bb = bias_lds[0] + kh * 16 * NMT;
    // Each tile goes global -> LDS directly with buffer loads (no register
    // staging): wave w copies the 1 KiB pieces w, w + NWAVES, ... of the
    // padded K and V tiles, lane l of a piece bytes 16 l .. 16 l + 15 of it,
    // i.e. row x / KSTR, byte column x % KSTR (padding columns copy the row's
    // first chunk, never read). A slot that holds no key (past a block's n
    // tokens, a pooled position inside E_i or outside J) gets an offset past
    // the end of every resource, so the copy writes zeros.
    constexpr int KTB = kKeyTile * KSTR;
    constexpr int NPC = KTB / 1024;
    constexpr int NPW = (NPC + NWAVES - 1) / NWAVES;
    static_assert(KTB % 1024 == 0, "tile must be whole 1 KiB pieces");
    constexpr uint32_t kNoRow = 0x80000000u;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    int pslot[NPW];
    uint32_t pcol[NPW];
#pragma unroll
    for (int pp = 0; pp < NPW; ++pp) {
      const int x = (pp * NWAVES + wave_u) * 1024 + 16 * lane;
      pslot[pp] = x / KSTR;
      const int col = x - pslot[pp] * KSTR;
      pcol[pp] = (uint32_t)(col < 2 * D ? col : 0);
    }
    const RowsRsrc k_rs = rows_rsrc(tc.K, (int)((size_t)s.L * D * 2));
    const RowsRsrc v_rs = rows_rsrc(tc.V, (int)((size_t)s.L * D * 2));
    const RowsRsrc kc_rs = rows_rsrc(tc.kc, (int)((size_t)s.N * D * 2));
    const RowsRsrc vc_rs = rows_rsrc(tc.vc, (int)((size_t)s.N * D * 2));
    for (int t = 0; t < ntiles; ++t) {
      const bool hb = tile_has_bias<MODE>(tc, t);
      if (t > 0) __syncthreads();   // previous tile fully consumed
      const bool pooled = t >= tc.ntiles_exact;
#pragma unroll
      for (int pp = 0; pp < NPW; ++pp) {
        const int piece = pp * NWAVES + wave_u;
        if (piece < NPC) {
          const int slot = pslot[pp];
          uint32_t off;
          if (!pooled) {
            const int q = t * tc.per + (slot >> tc.lb), o = slot & (tc.b - 1);
            const int e = q < tc.ntab ? tc.tab[q] : 0;
            off = o < (e & 127) ? (uint32_t)(((e >> 7) + o) * D * 2) + pcol[pp] : kNoRow;
          } else {
            const int p = (t - tc.ntiles_exact) * kKeyTile + slot;
            const int e = p < tc.N_kv ? tc.ptab[p] : 1;
            const bool valid = !(e & 1) && ((e >> 1) & 127) > 0;
            off = valid ? (uint32_t)((e >> 8) * D * 2) + pcol[pp] : kNoRow;
          }
          copy16_to_lds(pooled ? kc_rs : k_rs, k_lds[0] + piece * 1024, off, 0);
          copy16_to_lds(pooled ? vc_rs : v_rs, v_lds[0] + piece * 1024, off, 0);
        }
      }
      if (tid < kKeyTile) bias_lds[0][tid] = slot_src<D, MODE>(tc, t, tid).bias;
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's copies landed
      __syncthreads();
      float4_t sc[QT][NMT];
      bf16x8_t pk[QT][NMT / 2];
      qk_tile<D, QT, NMT>(kb, qf, sc, g, c16);
      if (hb) apply_logit_offsets<QT, NMT>(sc, bb, cscale, g);
      float mx[QT];
      row_max<QT, NMT>(sc, hb ? 1.0f : cscale, mx);
      rescale<D, QT>(mx, m, lsum, oacc);
      exp_pack<QT, NMT>(sc, hb ? 1.0f : cscale, m, lsum, pk);
      // the row statistics are final after the last tile's probabilities:
      // saving them here keeps m from living through the last PV product
      if (KS == 1 && t == ntiles - 1 && a.lse != nullptr)
        save_lse<QT>(a.lse, head, qtok, qval, m, lsum, g);
      pv_tile<D, QT, NMT>(vb, pk, oacc, g, c16);
    }
  } else {
    // Steady state: the leading tiles, which carry no additive logits. K
    // and V go global -> LDS directly (buffer loads into LDS, no register
    // staging), three buffers each; tile t+2 is copied while tile t is
    // processed and waited for before the barrier that ends the step.
    const int P = a.ntiles_plain;
    if (P > 0) {
      constexpr int KTB = kKeyTile * KSTR;            // bytes of one staged tile
      constexpr int NPC = KTB / 1024;                  // 1 KiB pieces per tile
      static_assert(KTB % 1024 == 0, "tile must be whole 1 KiB pieces");
      // Wave w copies pieces w, w + NWAVES, ... of each buffer; lane l of a
      // piece holds its bytes 16 l .. 16 l + 15, i.e. chunk (x % KSTR) / 16 of
      // staged row x / KSTR (padding chunks copy row data that is never read).
      // A piece never straddles a kept block (block starts fall on 1 KiB
      // boundaries for b = 32, 64), so its block start is wave-uniform; the
      // lane's element offset within the block is fixed for every tile.
      const int wave_u = __builtin_amdgcn_readfirstlane(wave);
      // Pieces 0 .. NFULL*NWAVES - 1 of K and of V go to every wave in turn;
      // the NREM pieces left over of each tensor go one per wave to the last
      // 2 NREM waves (K, then V), so that the two waves sharing a SIMD
      // (w and w + 4) issue the same number of copies between them.
      constexpr int NFULL = NPC / NWAVES;
      constexpr int NREM = NPC - NFULL * NWAVES;
      static_assert(!PIPE || (2 * NREM <= NWAVES && NWAVES == 8), "leftover pieces, one per wave");
      uint32_t dma_off[NFULL + 1];   // byte offset of the lane's chunk from its block start
      int dma_blk[NFULL + 1];        // which of the tile's (at most two) blocks the piece is in
      const bool extra = wave_u >= NWAVES - 2 * NREM;
      const bool extra_v = wave_u >= NWAVES - NREM;
      const int xpiece = NFULL * NWAVES + (extra_v ? wave_u - (NWAVES - NREM) : wave_u - (NWAVES - 2 * NREM));
#pragma unroll
      for (int pp = 0; pp <= NFULL; ++pp) {
        const int piece = pp < NFULL ? pp * NWAVES + wave_u : (extra ? xpiece : 0);
        const int x = piece * 1024 + 16 * lane;
        const int row = x / KSTR, col = x - row * KSTR;
        const int ce = col < 2 * D ? col / 2 : 0;
        dma_off[pp] = (uint32_t)(((MODE == kDense ? row : (row & (b - 1))) * D + ce) * 2);
        dma_blk[pp] = MODE == kDense ? 0 : (piece * 1024 / KSTR) >> lb;
      }
      // The copies are buffer loads into LDS: a buffer resource over this
      // head's rows (out-of-range reads return zero), the lane's fixed 32-bit
      // offset and the wave-uniform byte offset of the block, so no address
      // arithmetic runs on the vector units. Both block entries of a tile
      // are read before either is used (the second repeats the first for
      // b = 64).
      const int head_bytes = (int)((size_t)s.L * D * 2);
      const RowsRsrc k_rs = rows_rsrc(tc.K, head_bytes);
      const RowsRsrc v_rs = rows_rsrc(tc.V, head_bytes);
#define ISA_DMA_TILE(T, KD, VD)                                                  \
      {                                                                          \
        uint32_t base0 = (uint32_t)(T) * kKeyTile, base1 = base0;                \
        if (MODE != kDense) {                                                    \
          const int e0 = tc.tab[(T) * tc.per];                                   \
          const int e1 = tc.tab[(T) * tc.per + tc.per - 1];                      \
          base0 = (uint32_t)(__builtin_amdgcn_readfirstlane(e0) >> 7);           \
          base1 = (uint32_t)(__builtin_amdgcn_readfirstlane(e1) >> 7);           \
        }                                                                        \
        _Pragma("unroll") for (int pp = 0; pp < NFULL; ++pp) {                   \
          const int piece = pp * NWAVES + wave_u;                                \
          const int bo = (int)((dma_blk[pp] ? base1 : base0) * (uint32_t)(2 * D)); \
          copy16_to_lds(k_rs, (KD) + piece * 1024, dma_off[pp], bo);            \
          copy16_to_lds(v_rs, (VD) + piece * 1024, dma_off[pp], bo);            \
        }                                                                        \
        if (NREM > 0 && extra) {                                                 \
          const int bo = (int)((dma_blk[NFULL] ? base1 : base0) * (uint32_t)(2 * D)); \
          if (extra_v) copy16_to_lds(v_rs, (VD) + xpiece * 1024, dma_off[NFULL], bo); \
          else copy16_to_lds(k_rs, (KD) + xpiece * 1024, dma_off[NFULL], bo);   \
        }                                                                        \
      }
      ISA_DMA_TILE(0, k_lds[0], v_lds[0])
      if (P > 1) { ISA_DMA_TILE(1, k_ld1, v_ld1) }
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's copies landed
      __syncthreads();
      float4_t scur[QT][4], snext[QT][4];
      qk_tile<D, QT>(k_lds[0], qf, scur, g, c16);
      float mx[QT];
      row_max<QT>(scur, cscale, mx);
      // One step: scores of tile t+1 from KC, probabilities of tile t, O += V P
      // with VC; tile t+2 copied into (KD, VD).
#define ISA_STEP(t, KC, VC, KD, VD)                                              \
      {                                                                          \
        __syncthreads();                                                         \
        const bool more2 = (t) + 2 < P;                                          \
        if (more2) { ISA_DMA_TILE((t) + 2, KD, VD) }                             \
        rescale<D, QT>(mx, m, lsum, oacc);                                       \
        qk_tile<D, QT>(KC, qf, snext, g, c16);                                   \
        exp_pack<QT>(scur, cscale, m, lsum, pb);                                 \
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);                       \
        _Pragma("unroll") for (int i = 0; i < 14; ++i) {                         \
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                     \
          __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);                     \
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                     \
        }                                                                        \
        _Pragma("unroll") for (int i = 0; i < 2; ++i) {                          \
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                     \
          __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);                     \
        }                                                                        \
        pv_tile<D, QT>(VC, pb, oacc, g, c16);                                    \
        row_max<QT>(snext, cscale, mx);                                          \
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);                       \
        _Pragma("unroll") for (int i = 0; i < 14; ++i) {                         \
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);                     \
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 1);                     \
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);                     \
        }                                                                        \
        _Pragma("unroll") for (int i = 0; i < 2; ++i) {                          \
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);                     \
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 1);                     \
        }                                                                        \
        if (more2) __builtin_amdgcn_s_waitcnt(0x0F70);                           \
        _Pragma("unroll") for (int qt = 0; qt < QT; ++qt)                        \
          _Pragma("unroll") for (int mt = 0; mt < 4; ++mt) scur[qt][mt] = snext[qt][mt]; \
      }
      for (int t = 0; t < P; t += 3) {
        ISA_STEP(t, k_ld1, v_lds[0], k_ld2, v_ld2)
        if (t + 1 >= P) break;
        ISA_STEP(t + 1, k_ld2, v_ld1, k_lds[0], v_lds[0])
        if (t + 2 >= P) break;
        ISA_STEP(t + 2, k_lds[0], v_ld2, k_ld1, v_ld1)
      }
#undef ISA_STEP
#undef ISA_DMA_TILE
      __syncthreads();
    }
    // Tail: the few tiles with padding or partial blocks, one at a time.
    for (int t = P; t < ntiles; ++t) {
      ISA_LOAD_TILE(t)
      ISA_STORE_TILE(0, 0)
      __syncthreads();
      float4_t sc[QT][4];
      qk_tile<D, QT>(k_lds[0], qf, sc, g, c16);
      apply_logit_offsets<QT>(sc, bias_lds[0], cscale, g);
      float mx[QT];
      row_max<QT>(sc, 1.0f, mx);
      rescale<D, QT>(mx, m, lsum, oacc);
      exp_pack<QT>(sc, 1.0f, m, lsum, pb);
      pv_tile<D, QT>(v_lds[0], pb, oacc, g, c16);
      __syncthreads();
    }
  }
#undef ISA_LOAD_TILE
#undef ISA_STORE_TILE

  float ltot[QT];   // softmax denominator of each owned row
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) ltot[qt] = xor32_sum(xor16_sum(lsum[qt]));
  if (KS == 2) {
    // merge the two key halves: the second half's waves hand (m, sum, O^T)
    // over through the K/V buffers, no longer read, and leave
    __syncthreads();
    float4_t* xo = reinterpret_cast<float4_t*>(&k_lds[0][0]);
    float2_t* xm = reinterpret_cast<float2_t*>(&v_lds[0][0]);
    if (kh == 1) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) xo[((rwave * QT + qt) * DT + dt) * 64 + lane] = oacc[qt][dt];
        xm[(rwave * QT + qt) * 64 + lane] = float2_t{m[qt], ltot[qt]};
      }
    }
    __syncthreads();
    if (kh == 1) return;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float2_t o2 = xm[(rwave * QT + qt) * 64 + lane];
      const float mm = fmaxf(m[qt], o2.x);
      const float a1 = __builtin_amdgcn_exp2f(m[qt] - mm), a2 = __builtin_amdgcn_exp2f(o2.x - mm);
      ltot[qt] = ltot[qt] * a1 + o2.y * a2;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        oacc[qt][dt] = oacc[qt][dt] * a1 + xo[((rwave * QT + qt) * DT + dt) * 64 + lane] * a2;
      m[qt] = mm;
    }
  }

  // ---- normalise and write the owned rows
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    if (!qval[qt]) continue;
    const float inv = 1.0f / ltot[qt];
    uint16_t* orow = a.O + (head + qtok[qt]) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      uint2 w;
      w.x = pack_bf16x2(oacc[qt][dt][0] * inv, oacc[qt][dt][1] * inv);
      w.y = pack_bf16x2(oacc[qt][dt][2] * inv, oacc[qt][dt][3] * inv);
      *reinterpret_cast<uint2*>(orow + 16 * dt + 4 * g) = w;
    }
  }
  if ((PIPE || KS == 2) && a.lse != nullptr) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
      if (qval[qt] && g == 0) a.lse[head + qtok[qt]] = m[qt] + __log2f(ltot[qt]);
  }
}

// The flat kernels take their block tables in dynamic LDS: their limit is
// raised once per instantiation and device (host-side only).
template <int D, int MODE, int QT, int NWAVES, bool PIPE, int KS = 1>
hipError_t prepare() {
  if (MODE != kFlat) return hipSuccess;
  static unsigned long long done = 0;
  return isa_ensure_dyn_lds(reinterpret_cast<const void*>(&attn_kernel<D, MODE, QT, NWAVES, PIPE, KS>),
                            (int)(2 * ISA_MAX_NKV * sizeof(int)), &done);
}

template <int D, int MODE, int QT, int NWAVES, bool PIPE, int KS = 1>
hipError_t launch(const AttnArgs& a, dim3 grid, hipStream_t st) {
  size_t dyn = 0;
  if (MODE == kFlat) {
    dyn = (size_t)(a.s.k_ns + a.s.N_kv) * sizeof(int);
    const hipError_t attr = prepare<D, MODE, QT, NWAVES, PIPE, KS>();
    if (attr != hipSuccess) return attr;
  }
  attn_kernel<D, MODE, QT, NWAVES, PIPE, KS><<<grid, NWAVES * 64, dyn, st>>>(a);
  return hipGetLastError();
}

AttnArgs base_args(const IsaShape& s, const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                   uint16_t* O) {
  AttnArgs a{};
  a.s = s;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  return a;
}

}  // namespace

hipError_t isa_attn_prepare_device() {
  hipError_t e = prepare<128, kFlat, 1, 4, false>();
  if (e == hipSuccess) e = prepare<64, kFlat, 1, 4, false>();
  if (e == hipSuccess) e = prepare<128, kFlat, 1, 4, false, 2>();
  if (e == hipSuccess) e = prepare<64, kFlat, 1, 4, false, 2>();
  return e;
}

hipError_t isa_launch_sharp_attn(const IsaShape& s, const uint16_t* Q, const uint16_t* K,
                                 const uint16_t* V, const int32_t* ctx_idx,
                                 const int32_t* sharp_idx, uint16_t* O, float* lse,
                                 hipStream_t st) {
  if (s.n_sharp == 0) return hipSuccess;
  AttnArgs a = base_args(s, Q, K, V, O);
  a.lse = lse;
  a.ctx_idx = ctx_idx;
  a.qlist = sharp_idx;
  a.n_q = s.n_sharp;
  a.ntiles = (s.N_kv * s.b + kKeyTile - 1) / kKeyTile;
  {
    // tiles made only of full kept blocks (partial blocks are ordered last)
    int npart = (s.L_src % s.b) ? 1 : 0;
    if (s.L_ctx % s.b) npart += 1;   // conservative: the last context block may be kept
    a.ntiles_plain = (s.N_kv - npart) * s.b / kKeyTile;
  }
  const int rows = 8 * 32;
  const int blocks_per_wg = rows / s.b;
  dim3 grid((s.n_sharp + blocks_per_wg - 1) / blocks_per_wg, s.B * s.H);
  return s.D == 128 ? launch<128, kSharp, 2, 8, true>(a, grid, st)
                    : launch<64, kSharp, 2, 8, true>(a, grid, st);
}


hipError_t isa_launch_flat_attn(const IsaShape& s, const uint16_t* Q, const uint16_t* K,
                                const uint16_t* V, const uint16_t* kc_bf16,
                                const uint16_t* vc_bf16, const int32_t* ctx_idx,
                                const int32_t* flat_idx, const int32_t* flat_exact_idx,
                                const int32_t* flat_ord, uint16_t* O, float* lse, hipStream_t st) {
  if (s.n_flat == 0) return hipSuccess;
  AttnArgs a = base_args(s, Q, K, V, O);
  a.flat_ord = flat_ord;
  a.lse = lse;
  a.kcb = kc_bf16;
  a.vcb = vc_bf16;
  a.ctx_idx = ctx_idx;
  a.qlist = flat_idx;
  a.exact = flat_exact_idx;
  a.n_q = s.n_flat;
  a.ntiles_exact = (s.k_ns * s.b + kKeyTile - 1) / kKeyTile;
  const int pooled = s.k_ns < s.N_kv ? (s.N_kv + kKeyTile - 1) / kKeyTile : 0;
  a.ntiles = a.ntiles_exact + pooled;
  dim3 grid(s.n_flat, s.B * s.H);
  // one flat block per workgroup, 16 query rows per wave; a 32-token block
  // takes two waves per key half
  if (s.b == 64)
    return s.D == 128 ? launch<128, kFlat, 1, 4, false>(a, grid, st)
                      : launch<64, kFlat, 1, 4, false>(a, grid, st);
  return s.D == 128 ? launch<128, kFlat, 1, 4, false, 2>(a, grid, st)
                    : launch<64, kFlat, 1, 4, false, 2>(a, grid, st);
}

// Grid order of the flat blocks: by the first (smallest) block id of each
// exact set E_i, ties by row (a stable rank, one workgroup per head, the
// keys in LDS). Flat blocks whose exact sets begin at the same block share
// many of their blocks when attention is local, so the workgroups that one
// XCD runs together gather overlapping blocks and find them in its L2; with
// no such structure the order is as good as any other.
namespace {

constexpr int kOrderThreads = 1024;

__global__ __launch_bounds__(kOrderThreads) void flat_order_kernel(IsaShape s, const int32_t* exact,
                                                                    int32_t* ord) {
  __shared__ int key[2 * ISA_MAX_SEG_BLOCKS];
  const int bh = blockIdx.x;
  const int32_t* ex = exact + (size_t)bh * s.n_flat * s.k_ns;
  for (int r = threadIdx.x; r < s.n_flat; r += kOrderThreads) key[r] = ex[(size_t)r * s.k_ns];
  __syncthreads();
  int32_t* o = ord + (size_t)bh * s.n_flat;
  for (int r = threadIdx.x; r < s.n_flat; r += kOrderThreads) {
    const int k = key[r];
    int rank = 0;
    for (int q = 0; q < s.n_flat; ++q) {
      const int m = key[q];
      rank += (m < k || (m == k && q < r)) ? 1 : 0;
    }
    o[rank] = r;
  }
}

}  // namespace

hipError_t isa_launch_flat_order(const IsaShape& s, const int32_t* flat_exact_idx, int32_t* flat_ord,
                                 hipStream_t st) {
  if (s.n_flat == 0 || s.k_ns == 0) return hipSuccess;
  flat_order_kernel<<<s.B * s.H, kOrderThreads, 0, st>>>(s, flat_exact_idx, flat_ord);
  return hipGetLastError();
}

hipError_t isa_launch_dense_attn(int B, int H, int L, int D, const uint16_t* Q,
                                 const uint16_t* K, const uint16_t* V, uint16_t* O,
                                 hipStream_t st) {
  IsaShape s{};
  s.B = B;
  s.H = H;
  s.L = L;
  s.L_src = L;
  s.D = D;
  s.b = kKeyTile;
  AttnArgs a = base_args(s, Q, K, V, O);
  a.ntiles = (L + kKeyTile - 1) / kKeyTile;
  a.ntiles_plain = L / kKeyTile;
  dim3 grid((L + 255) / 256, B * H);
  return D == 128 ? launch<128, kDense, 2, 8, true>(a, grid, st)
                  : launch<64, kDense, 2, 8, true>(a, grid, st);
}
