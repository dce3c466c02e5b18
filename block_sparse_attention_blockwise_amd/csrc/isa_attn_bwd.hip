// Backward pass of In-context Sparse Attention on gfx950 (the operator is
// trained end to end: paper.rainbus.top summary of arXiv 2605.04569, "Core
// method" and "Novelty" (c)).
//
// The selections of the forward pass are piecewise constant, so the
// gradients flow through the attention terms with J, the sharp/flat split
// and every E_i held fixed. For a query row t with key rows u (exact tokens,
// and for a flat block also the pooled keys Kc_j with logit offset ln n_j):
//   P = softmax over u,   Delta_t = dO_t . O_t,   dS_tu = P_tu (dO_t . v_u - Delta_t),
//   dq_t = sum_u dS_tu k_u / sqrt(D),   dk_u += dS_tu q_t / sqrt(D),   dv_u += P_tu dO_t.
// The pooled keys pass their gradients to the tokens of their block through
// the mean of step (1): each token of block j receives dKc_j / n_j and
// dVc_j / n_j.
//
// Kernels (all deterministic: every sum has a fixed order, no float atomics):
//   * bwd_prep_kernel: per head, a bitmap of E_i over the positions of J and,
//     for every kept block, the ascending list of flat blocks whose E_i holds
//     it (filled in order from the bitmap, linear in the number of blocks);
//   * delta_kernel: Delta_t for every row;
//   * dq_kernel (query-major, as the forward): per query block, over the key
//     tiles the forward used; S^T = K Q^T and dP^T = V dO^T on the matrix
//     cores, P recomputed from the saved log-sum-exp, dQ^T += K^T dS^T;
//   * dkv_pc_kernel (key-major): per 128 keys of J (whole kept blocks), the
//     keys held in registers, over every query block that reads them exactly
//     (all sharp blocks, then each kept block's flat blocks with the other
//     keys masked); producer waves form S = Q K^T, P and dV^T += dO^T P,
//     consumer waves (one block behind, P passed through LDS) dP = dO V^T,
//     dS and dK^T += Q^T dS; the pooled gradients dKc_j / n_j, dVc_j / n_j
//     are added before the rows are written; zero_pruned_kernel zeroes the
//     rows of pruned blocks;
//   * dkv_pooled_kernel (key-major over the pooled keys): per 64 positions of
//     J, over every flat block; writes dKc, dVc (fp32).
// The sharp dq_kernel and dkv_pc_kernel stage their streamed operands (key
// tiles, query blocks) with buffer loads straight into LDS buffers
// that are separate arrays, one step ahead; rows past a block's valid tokens
// copy real rows and are masked by a -inf logit offset or a +inf log-sum-exp.
// With decoupled RoPE the gradients of the rotated Q and K are turned back by
// the transposed rotation in the epilogues.
#include <initializer_list>

#include "isa_internal.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(16)));
typedef short short4_t __attribute__((__vector_size__(8)));
typedef float float4_t __attribute__((__vector_size__(16)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
struct bf16x2x4_t { bf16x2_t a, b, c, d; };

constexpr int kKeyTile = 64;
constexpr float kLog2e = 1.4426950408889634f;

struct BwdArgs {
  IsaShape s;
  const uint16_t* Q;          // the attention inputs (rotated when RoPE is on)
  const uint16_t* K;
  const uint16_t* V;
  const uint16_t* dO;
  const float* lse;           // [B,H,L] log2-domain log-sum-exp from the forward
  const float* delta;         // [B,H,L]
  const uint16_t* kcb;        // [B,H,N,D] bf16 block means (the forward's Taylor operands)
  const uint16_t* vcb;
  const int32_t* ctx_idx;     // [B,H,k_ctx]
  const int32_t* qlist;       // dq: sharp_idx or flat_idx
  const int32_t* sharp_idx;   // [B,H,n_sharp]
  const int32_t* flat_idx;    // [B,H,n_flat]
  const int32_t* exact;       // [B,H,n_flat,k_ns]
  const int32_t* flat_ord;    // [B,H,n_flat] grid order of the flat dQ kernel (nullable: plain order)
  const uint64_t* ebits;      // [B,H,n_flat,W] bit p of row r: position p of J is in E_r
  const int32_t* inv_off;     // [B,H,N_kv+1]
  const int32_t* inv_list;    // [B,H,n_flat*k_ns] flat block ids reading each position exactly
  const int32_t* chunk_ord;   // [B,H,N_kv] 128-key chunks of J, longest stream first (n_flat > 0)
  const float* dkc;           // [B,H,N,D] pooled-key gradients (nullable)
  const float* dvc;
  float* dkc_out;
  float* dvc_out;
  const float2* rope;         // cos/sin table (nullable: no RoPE)
  // residual gamma * O_coarse (gamma != 0 only)
  const double* srows;        // [B,H,N,N_kv] coarse rows S[i, J] of the forward
  const double* qc;           // [B,H,N,D] fp64 block means
  const double* kc;
  float* dqc;                 // [B,H,N,D] gradient of Qc (scaled), added to the rows' dQ
  float* doc;                 // [B,H,N,D] gamma * sum of dO over each block
  float* ocs;                 // [B,H,N,D] O_coarse as the forward added it (without gamma)
  float* dsc;                 // [B,H,N,N_kv] gradient of the coarse logits
  float* pc;                  // [B,H,N,N_kv] coarse softmax
  uint16_t* dQ;
  uint16_t* dK;
  uint16_t* dV;
  int n_q;
  int ntiles_exact;
  int ntiles;
  int W;                      // 64-bit words per bitmap row
};

__device__ inline short4_t lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4_t*)(p));
}

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// Position of global block j in the kept list J, or -1.
__device__ inline int kept_pos(const IsaShape& s, const int32_t* ctx_row, int j) {
  if (j >= 0 && j < s.N_src) return j;
  if (j < s.N_src || j >= s.N) return -1;
  int lo = 0, hi = s.k_ctx;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (ctx_row[mid] < j) lo = mid + 1; else hi = mid;
  }
  return (lo < s.k_ctx && ctx_row[lo] == j) ? s.N_src + lo : -1;
}

// Global block id at position q of J, or -1.
__device__ inline int kept_id(const IsaShape& s, const int32_t* ctx_row, int q) {
  if (q < s.N_src) return q;
  if (q >= s.N_kv) return -1;
  const int j = ctx_row[q - s.N_src];
  return (j >= s.N_src && j < s.N) ? j : -1;
}

// ---------------------------------------------------------------- tile math
// s[nf][mt] = A rows (16 mt + 4g + e of the LDS tile) . B fragment nf
// (column c16); A is read from LDS rows of stride 2D+32 bytes.
template <int D, int MT, int NF>
__device__ __forceinline__ void mm_rows(const char* lds, const bf16x8_t (&f)[NF][D / 32],
                                        float4_t (&s)[NF][MT], int g, int c16) {
  constexpr int STR = 2 * D + 32;
#pragma unroll
  for (int nf = 0; nf < NF; ++nf)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) s[nf][mt] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(lds + (16 * mt + c16) * STR + (32 * kk + 8 * g) * 2);
#pragma unroll
      for (int nf = 0; nf < NF; ++nf)
        s[nf][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, f[nf][kk], s[nf][mt], 0, 0, 0);
    }
  }
}

// mm_rows whose sums start from a per-row value c0[row] (LDS) instead of 0.
template <int D, int MT, int NF>
__device__ __forceinline__ void mm_rows_from(const char* lds, const bf16x8_t (&f)[NF][D / 32],
                                             float4_t (&s)[NF][MT], const float* c0, int g, int c16) {
  constexpr int STR = 2 * D + 32;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const float4_t c = *reinterpret_cast<const float4_t*>(c0 + 16 * mt + 4 * g);
#pragma unroll
    for (int nf = 0; nf < NF; ++nf) s[nf][mt] = c;
  }
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(lds + (16 * mt + c16) * STR + (32 * kk + 8 * g) * 2);
#pragma unroll
      for (int nf = 0; nf < NF; ++nf)
        s[nf][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, f[nf][kk], s[nf][mt], 0, 0, 0);
    }
  }
}

// acc[nf][dt] += (LDS rows)^T . pk[nf]: the LDS tile (16*MT rows) is read
// transposed, its rows being the contraction index in the order pack_bf16
// produces.
template <int D, int MT, int NF>
__device__ __forceinline__ void mm_tr(const char* lds, const bf16x8_t (&pk)[NF][MT / 2],
                                      float4_t (&acc)[NF][D / 16], int g, int c16) {
  constexpr int STR = 2 * D + 32;
  const int tr_row = 4 * g + (c16 >> 2);
  const int tr_col = 4 * (c16 & 3);
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
#pragma unroll
    for (int kc = 0; kc < MT / 2; ++kc) {
      const short4_t lo = lds_read_tr(lds + (32 * kc + tr_row) * STR + (16 * dt + tr_col) * 2);
      const short4_t hi = lds_read_tr(lds + (32 * kc + 16 + tr_row) * STR + (16 * dt + tr_col) * 2);
      const bf16x8_t va = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int nf = 0; nf < NF; ++nf)
        acc[nf][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pk[nf][kc], acc[nf][dt], 0, 0, 0);
    }
  }
}

// Scheduling pattern for one mm_rows (RD = 1 LDS read per step) or mm_tr
// (RD = 2) call: the reads run PF steps ahead of the NF products per step.
template <int NS, int NF, int RD, int PF, int ID>
__device__ __forceinline__ void ahead() {
  __builtin_amdgcn_sched_group_barrier(0x100, RD * PF, ID);
#pragma unroll
  for (int i = 0; i < NS - PF; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, NF, ID);
    __builtin_amdgcn_sched_group_barrier(0x100, RD, ID);
  }
#pragma unroll
  for (int i = 0; i < PF; ++i) __builtin_amdgcn_sched_group_barrier(0x008, NF, ID);
}

// LDS read distance of the dK/dV products (measured: 2 ahead beats 0, 3, 4)
constexpr int kDkvAhead = 2;

// Rounds an mm_rows result to bf16 in the operand layout mm_tr expects.
template <int MT, int NF>
__device__ __forceinline__ void pack_bf16(const float4_t (&x)[NF][MT], bf16x8_t (&pk)[NF][MT / 2]) {
#pragma unroll
  for (int nf = 0; nf < NF; ++nf) {
#pragma unroll
    for (int kc = 0; kc < MT / 2; ++kc) {
      bf16x2_t h[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i0 = 8 * kc + 2 * u;
        h[u] = __builtin_convertvector((float2_t){x[nf][i0 >> 2][i0 & 3], x[nf][(i0 + 1) >> 2][(i0 + 1) & 3]},
                                       bf16x2_t);
      }
      pk[nf][kc] = __builtin_bit_cast(bf16x8_t, (bf16x2x4_t){h[0], h[1], h[2], h[3]});
    }
  }
}

// Transposed RoPE rotation of one gradient pair (gx, gy) at position `pos`,
// pair index `i` (the inverse of the forward rotation by angle pos*f_i).
__device__ inline void rope_back(const float2* tab, int half, int pos, int i, float& gx, float& gy) {
  const float2 cs = tab[(size_t)pos * half + i];
  const float x = gx * cs.x + gy * cs.y;
  const float y = gy * cs.x - gx * cs.y;
  gx = x;
  gy = y;
}

// Writes 4 consecutive gradient values (d0..d0+3 of one token row) as bf16,
// after the optional RoPE transpose (pairs (d0, d0+1) and (d0+2, d0+3)).
__device__ inline void store4(uint16_t* row, int d0, float4_t v, const float2* rope, int half, int pos) {
  float x0 = v[0], x1 = v[1], x2 = v[2], x3 = v[3];
  if (rope != nullptr) {
    rope_back(rope, half, pos, d0 >> 1, x0, x1);
    rope_back(rope, half, pos, (d0 >> 1) + 1, x2, x3);
  }
  uint2 w;
  w.x = pack_bf16x2(x0, x1);
  w.y = pack_bf16x2(x2, x3);
  *reinterpret_cast<uint2*>(row + d0) = w;
}

// ---------------------------------------------------------------- prep
// One workgroup per head: the E bitmap (one row of ceil(N_kv/64) words per
// flat block), the count of flat blocks per kept position, their offsets,
// the order of the dK/dV kernel's 128-key chunks, and then each position's
// list of flat blocks, filled in ascending order by one thread walking the
// bitmap column (linear in n_flat, no sort, so the order is fixed however
// many flat blocks share a position).
constexpr int kPrepThreads = 1024;

__global__ __launch_bounds__(kPrepThreads) void bwd_prep_kernel(BwdArgs a) {
  const IsaShape& s = a.s;
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int32_t* ctx_row = a.ctx_idx + (size_t)bh * s.k_ctx;
  const int32_t* ex = a.exact + (size_t)bh * s.n_flat * s.k_ns;
  const int32_t* frow = a.flat_idx + (size_t)bh * s.n_flat;
  uint64_t* bits = const_cast<uint64_t*>(a.ebits) + (size_t)bh * s.n_flat * a.W;
  int32_t* off = const_cast<int32_t*>(a.inv_off) + (size_t)bh * (s.N_kv + 1);
  int32_t* lst = const_cast<int32_t*>(a.inv_list) + (size_t)bh * s.n_flat * s.k_ns;
  __shared__ int cnt[ISA_MAX_NKV + 1];
  __shared__ int part[kPrepThreads];
  __shared__ int clen[ISA_MAX_NKV / 2];
  for (int p = tid; p <= s.N_kv; p += kPrepThreads) cnt[p] = 0;
  __syncthreads();
  for (int r = tid; r < s.n_flat; r += kPrepThreads) {
    uint64_t* brow = bits + (size_t)r * a.W;
    for (int w = 0; w < a.W; ++w) brow[w] = 0;
    int cw = -1;
    uint64_t word = 0;
    for (int q = 0; q < s.k_ns; ++q) {
      const int p = kept_pos(s, ctx_row, ex[(size_t)r * s.k_ns + q]);
      if (p < 0) continue;
      atomicAdd(&cnt[p], 1);   // integer count: the result does not depend on the order
      if ((p >> 6) != cw) {
        if (cw >= 0) brow[cw] = word;
        cw = p >> 6;
        word = 0;
      }
      word |= 1ull << (p & 63);
    }
    if (cw >= 0) brow[cw] = word;
  }
  __syncthreads();
  // exclusive scan of cnt[0..N_kv) in contiguous chunks
  const int per = (s.N_kv + kPrepThreads - 1) / kPrepThreads;
  const int p0 = tid * per, p1 = min(p0 + per, s.N_kv);
  int sum = 0;
  for (int p = p0; p < p1; ++p) sum += cnt[p];
  part[tid] = sum;
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int t = 0; t < kPrepThreads; ++t) {
      const int v = part[t];
      part[t] = acc;
      acc += v;
    }
  }
  __syncthreads();
  int acc = part[tid];
  for (int p = p0; p < p1; ++p) {
    off[p] = acc;
    acc += cnt[p];
  }
  if (tid == kPrepThreads - 1) off[s.N_kv] = part[tid] + sum;
  __syncthreads();
  // Chunk order of the dK/dV grid: the chunks whose keys the most flat
  // blocks read exactly (the longest streams) first, ties by position. The
  // workgroups dispatched together then run streams of about the same length,
  // so they stay in step through the part all of them read in the same order
  // (the sharp blocks), and each of its blocks is fetched into L2 once for
  // all of them rather than again for each straggler.
  {
    const int kpb = 128 / s.b;
    const int C = (s.N_kv + kpb - 1) / kpb;
    for (int c = tid; c < C; c += kPrepThreads) {
      int n = 0;
      for (int u = 0; u < kpb; ++u) {
        const int p = c * kpb + u;
        if (p < s.N_kv) n += cnt[p];
      }
      clen[c] = n;
    }
    __syncthreads();
    int32_t* ord = const_cast<int32_t*>(a.chunk_ord) + (size_t)bh * s.N_kv;
    for (int c = tid; c < C; c += kPrepThreads) {
      const int n = clen[c];
      int r = 0;
      for (int d = 0; d < C; ++d) {
        const int m = clen[d];
        r += (m > n || (m == n && d < c)) ? 1 : 0;
      }
      ord[r] = c;
    }
  }
  // each position's flat blocks in ascending order: walk the bitmap column
  for (int p = tid; p < s.N_kv; p += kPrepThreads) {
    int k = off[p];
    const uint64_t bit = 1ull << (p & 63);
    const uint64_t* col = bits + (p >> 6);
    int r = 0;
    for (; r + 8 <= s.n_flat; r += 8) {
      uint64_t w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) w[u] = col[(size_t)(r + u) * a.W];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (w[u] & bit) lst[k++] = frow[r + u];
    }
    for (; r < s.n_flat; ++r)
      if (col[(size_t)r * a.W] & bit) lst[k++] = frow[r];
  }
}

// ---------------------------------------------------------------- Delta
// Delta_t = dO_t . o_t with o_t the attention output: with the residual on,
// the forward added gamma * O_coarse of the row's block to it, which is taken
// off again here.
__device__ inline int token_block(const IsaShape& s, int t) {
  return t < s.L_src ? t / s.b : s.N_src + (t - s.L_src) / s.b;
}

template <int D>
__global__ __launch_bounds__(256) void delta_kernel(BwdArgs a, const uint16_t* __restrict__ O, size_t rows) {
  constexpr int TPR = D / 8;
  const size_t row = ((size_t)blockIdx.x * 256 + threadIdx.x) / TPR;
  const int c = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    const uint4 x = *reinterpret_cast<const uint4*>(a.dO + row * D + c * 8);
    const uint4 y = *reinterpret_cast<const uint4*>(O + row * D + c * 8);
    const uint32_t xu[4] = {x.x, x.y, x.z, x.w}, yu[4] = {y.x, y.y, y.z, y.w};
    float oc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (a.ocs != nullptr) {
      const size_t bh = row / a.s.L;
      const int i = token_block(a.s, (int)(row % a.s.L));
      const float* src = a.ocs + ((bh * a.s.N + i) * D + c * 8);
#pragma unroll
      for (int k = 0; k < 8; ++k) oc[k] = a.s.gamma * src[k];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc += __uint_as_float(xu[i] << 16) * (__uint_as_float(yu[i] << 16) - oc[2 * i]);
      acc += __uint_as_float(xu[i] & 0xffff0000u) * (__uint_as_float(yu[i] & 0xffff0000u) - oc[2 * i + 1]);
    }
  }
#pragma unroll
  for (int o = 1; o < TPR; o <<= 1) acc += __shfl_xor(acc, o, 64);
  if (row < rows && c == 0) const_cast<float*>(a.delta)[row] = acc;
}

// ---------------------------------------------------------------- residual
// Backward of gamma * O_coarse (O_coarse_i = softmax over J of S[i, J]
// applied to Vc[J], broadcast to the tokens of block i). Per query block i:
// dOc_i = gamma * sum of dO over the block's rows (res_dosum_kernel), the
// coarse softmax P_i (fp64, from the forward's coarse rows), O_coarse_i as
// the forward computed it, Delta_i = dOc_i . O_coarse_i, the logit gradient
// dS_i = P_i * (dOc_i . Vc_p - Delta_i) (the dot in fp32 as in the token-level
// backward, P and the difference in fp64) and dQc_i = sum_p dS_ip Kc_p / sqrt(D)
// (fp32).
// A workgroup takes kResRows consecutive query blocks of a head; J streams
// through LDS in tiles of kResTile pooled keys (Vc rows, and Kc rows for
// the second pass), shared by the workgroup's rows.
constexpr int kResThreads = 256;
constexpr int kResRows = 16;
constexpr int kResTile = 64;

__device__ inline float bf16f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// dOc_i = gamma * the sum of dO over the token rows of block i, one
// workgroup per block: 16-byte loads, partial sums per token group, then a
// fixed-order sum of the groups.
template <int D>
__global__ __launch_bounds__(kResThreads) void res_dosum_kernel(BwdArgs a) {
  constexpr int CPR = D / 8, G = kResThreads / CPR;
  const IsaShape& s = a.s;
  const int i = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int k = tid % CPR, tg = tid / CPR;
  __shared__ float part[G][D];
  int st, n;
  isa_block_range(s, i, st, n);
  const uint16_t* src = a.dO + ((size_t)bh * s.L + st) * D + 8 * k;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int x = tg; x < n; x += G) {
    const uint4 w = *reinterpret_cast<const uint4*>(src + (size_t)x * D);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] += __uint_as_float(u[q] << 16);
      acc[2 * q + 1] += __uint_as_float(u[q] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[tg][8 * k + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    float t = 0.f;
    for (int g = 0; g < G; ++g) t += part[g][tid];
    a.doc[((size_t)bh * s.N + i) * D + tid] = s.gamma * t;
  }
}

template <int D>
__global__ __launch_bounds__(kResThreads) void res_row_kernel(BwdArgs a) {
  constexpr int VST = D + 2;                        // bf16 row stride: 4-byte stores, conflict-free column reads
  constexpr int RPT = kResRows * D / kResThreads;   // rows per thread in the column-parallel phases
  constexpr int RQ = kResRows / (kResThreads / kResTile);   // rows per thread in the key-parallel phase
  const IsaShape& s = a.s;
  const int i0 = blockIdx.x * kResRows, bh = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int nr = min(kResRows, s.N - i0);
  __shared__ double rmax[kResRows], rz[kResRows], rdl[kResRows];
  __shared__ float wf[kResRows][kResTile];
  __shared__ __attribute__((aligned(16))) uint16_t vt[kResTile * VST];
  __shared__ float kt[kResTile][D];
  __shared__ float dov[kResRows][D], ocv[kResRows][D];
  __shared__ int jt[kResTile];
  const int32_t* ctx_row = a.ctx_idx + (size_t)bh * s.k_ctx;
  const double* rows = a.srows + ((size_t)bh * s.N + i0) * s.N_kv;
  const size_t nbase = ((size_t)bh * s.N) * D;

  // row max and normaliser of the coarse softmax, one wave per row
  for (int r = wave; r < nr; r += kResThreads / 64) {
    const double* row = rows + (size_t)r * s.N_kv;
    double mx = -INFINITY;
    for (int p = lane; p < s.N_kv; p += 64) mx = fmax(mx, row[p]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o, 64));
    double z = 0.0;
    for (int p = lane; p < s.N_kv; p += 64) z += exp(row[p] - mx);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o, 64);
    if (lane == 0) {
      rmax[r] = mx;
      rz[r] = z;
    }
  }
  // dOc (res_dosum_kernel); thread: column d of RPT rows
  const int d = tid % D, rg = tid / D;
  float acc[RPT];
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    const int r = rg * RPT + u;
    dov[r][d] = r < nr ? a.doc[nbase + (size_t)(i0 + r) * D + d] : 0.f;
    acc[u] = 0.f;
  }

  // stages the Vc (and Kc) rows of J positions p0 .. p0+63: all of a
  // thread's 16-byte loads are issued before any LDS store
  auto stage_keys = [&](int p0, bool with_k) {
    constexpr int VC = kResTile * D / 8 / kResThreads;   // 16-byte Vc chunks per thread
    constexpr int KC = kResTile * D / 2 / kResThreads;   // 16-byte Kc chunks (two fp64) per thread
    if (tid < kResTile) jt[tid] = p0 + tid < s.N_kv ? kept_id(s, ctx_row, p0 + tid) : -1;
    __syncthreads();
    uint4 vr[VC];
#pragma unroll
    for (int x = 0; x < VC; ++x) {
      const int c = tid + x * kResThreads, pp = c / (D / 8), k8 = c % (D / 8), j = jt[pp];
      vr[x] = j >= 0 ? *reinterpret_cast<const uint4*>(a.vcb + nbase + (size_t)j * D + 8 * k8)
                     : make_uint4(0, 0, 0, 0);
    }
    double2 kr[KC];
    if (with_k) {
#pragma unroll
      for (int x = 0; x < KC; ++x) {
        const int c = tid + x * kResThreads, pp = c / (D / 2), k2 = c % (D / 2), j = jt[pp];
        kr[x] = j >= 0 ? *reinterpret_cast<const double2*>(a.kc + nbase + (size_t)j * D + 2 * k2)
                       : make_double2(0.0, 0.0);
      }
    }
#pragma unroll
    for (int x = 0; x < VC; ++x) {
      const int c = tid + x * kResThreads, pp = c / (D / 8), k8 = c % (D / 8);
      uint32_t* dst = reinterpret_cast<uint32_t*>(&vt[pp * VST + 8 * k8]);
      dst[0] = vr[x].x;
      dst[1] = vr[x].y;
      dst[2] = vr[x].z;
      dst[3] = vr[x].w;
    }
    if (with_k) {
#pragma unroll
      for (int x = 0; x < KC; ++x) {
        const int c = tid + x * kResThreads, pp = c / (D / 2), k2 = c % (D / 2);
        kt[pp][2 * k2] = (float)kr[x].x;
        kt[pp][2 * k2 + 1] = (float)kr[x].y;
      }
    }
  };

  // pass 1: O_coarse = sum_p exp(S - max) Vc_p / z, as the forward formed it
  for (int p0 = 0; p0 < s.N_kv; p0 += kResTile) {
    __syncthreads();
    stage_keys(p0, false);
    for (int c = tid; c < kResRows * kResTile; c += kResThreads) {
      const int r = c / kResTile, pp = c % kResTile;
      const bool ok = r < nr && p0 + pp < s.N_kv && jt[pp] >= 0;
      wf[r][pp] = ok ? (float)exp(rows[(size_t)r * s.N_kv + p0 + pp] - rmax[r]) : 0.f;
    }
    __syncthreads();
    for (int pp = 0; pp < kResTile; ++pp) {
      const float v = bf16f(vt[pp * VST + d]);
#pragma unroll
      for (int u = 0; u < RPT; ++u) acc[u] += wf[rg * RPT + u][pp] * v;
    }
  }
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    const int r = rg * RPT + u;
    ocv[r][d] = r < nr ? (float)((double)acc[u] / rz[r]) : 0.f;
  }
  __syncthreads();
  if (tid < kResRows) {
    double dl = 0.0;
    for (int k = 0; k < D; ++k) dl += (double)dov[tid][k] * (double)ocv[tid][k];
    rdl[tid] = dl;
  }

  // pass 2: dS over the kept blocks (to pc and dsc), dQc = sum_p dS Kc_p
  float* pc_rows = a.pc + ((size_t)bh * s.N + i0) * s.N_kv;
  float* ds_rows = a.dsc + ((size_t)bh * s.N + i0) * s.N_kv;
  const int pp = tid % kResTile, rq = tid / kResTile;   // key-parallel: key pp, rows rq*RQ ..
  float q[RPT];
#pragma unroll
  for (int u = 0; u < RPT; ++u) q[u] = 0.f;
  for (int p0 = 0; p0 < s.N_kv; p0 += kResTile) {
    __syncthreads();
    stage_keys(p0, true);
    __syncthreads();
    const int p = p0 + pp;
    float dot[RQ];
#pragma unroll
    for (int u = 0; u < RQ; ++u) dot[u] = 0.f;
#pragma unroll 8
    for (int k = 0; k < D; ++k) {
      const float v = bf16f(vt[pp * VST + k]);
#pragma unroll
      for (int u = 0; u < RQ; ++u) dot[u] += dov[rq * RQ + u][k] * v;
    }
#pragma unroll
    for (int u = 0; u < RQ; ++u) {
      const int r = rq * RQ + u;
      double ds = 0.0;
      if (r < nr && p < s.N_kv) {
        const double P = exp(rows[(size_t)r * s.N_kv + p] - rmax[r]) / rz[r];
        ds = P * ((double)dot[u] - rdl[r]);
        pc_rows[(size_t)r * s.N_kv + p] = (float)P;
        ds_rows[(size_t)r * s.N_kv + p] = (float)ds;
      }
      wf[r][pp] = (float)ds;
    }
    __syncthreads();
#pragma unroll 8
    for (int x = 0; x < kResTile; ++x) {
      const float kv = kt[x][d];
#pragma unroll
      for (int u = 0; u < RPT; ++u) q[u] += wf[rg * RPT + u][x] * kv;
    }
  }
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    const int r = rg * RPT + u;
    if (r >= nr) continue;
    const size_t o = nbase + (size_t)(i0 + r) * D + d;
    a.dqc[o] = q[u] / sqrtf((float)D);
    a.ocs[o] = ocv[r][d];
  }
}

// dKc_p += sum_i dS_ip Qc_i / sqrt(D) and dVc_p += sum_i P_ip dOc_i for 64
// kept blocks per workgroup (a product of the coarse-row matrices with Qc
// and dOc), summed in a fixed order over i; adds to the pooled-key gradients
// when those were written (accumulate), else stores.
template <int D>
__global__ __launch_bounds__(256) void res_col_kernel(BwdArgs a, int accumulate) {
  constexpr int PT = 64, IC = 32;
  constexpr int DPT = D / 4;   // d values per thread
  const IsaShape& s = a.s;
  const int bh = blockIdx.y, p0 = blockIdx.x * PT, tid = threadIdx.x;
  const int pl = tid / 4, d0 = (tid % 4) * DPT;
  __shared__ float ds_t[IC][PT], p_t[IC][PT];
  __shared__ __attribute__((aligned(16))) float qc_t[IC][D];
  __shared__ __attribute__((aligned(16))) float do_t[IC][D];
  float dk[DPT], dv[DPT];
#pragma unroll
  for (int x = 0; x < DPT; ++x) dk[x] = dv[x] = 0.f;
  const size_t rbase = (size_t)bh * s.N;
  // per chunk of IC rows, every load of a thread is issued before its LDS
  // stores (dS and P rows in 4-byte words: N_kv need not be a multiple of 4)
  constexpr int NS = IC * PT / 256, NQ = IC * D / 2 / 256, ND = IC * D / 4 / 256;
  for (int i0 = 0; i0 < s.N; i0 += IC) {
    float dsr[NS], pr[NS];
    double2 qr[NQ];
    float4 dr[ND];
#pragma unroll
    for (int x = 0; x < NS; ++x) {
      const int c = tid + x * 256, ii = c / PT, pp = c % PT;
      const bool ok = i0 + ii < s.N && p0 + pp < s.N_kv;
      const size_t o = (rbase + i0 + ii) * s.N_kv + p0 + pp;
      dsr[x] = ok ? a.dsc[o] : 0.f;
      pr[x] = ok ? a.pc[o] : 0.f;
    }
#pragma unroll
    for (int x = 0; x < NQ; ++x) {
      const int c = tid + x * 256, ii = c / (D / 2), k2 = c % (D / 2);
      qr[x] = i0 + ii < s.N ? *reinterpret_cast<const double2*>(a.qc + (rbase + i0 + ii) * D + 2 * k2)
                            : make_double2(0.0, 0.0);
    }
#pragma unroll
    for (int x = 0; x < ND; ++x) {
      const int c = tid + x * 256, ii = c / (D / 4), k4 = c % (D / 4);
      dr[x] = i0 + ii < s.N ? *reinterpret_cast<const float4*>(a.doc + (rbase + i0 + ii) * D + 4 * k4)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < NS; ++x) {
      const int c = tid + x * 256;
      ds_t[c / PT][c % PT] = dsr[x];
      p_t[c / PT][c % PT] = pr[x];
    }
#pragma unroll
    for (int x = 0; x < NQ; ++x) {
      const int c = tid + x * 256, ii = c / (D / 2), k2 = c % (D / 2);
      qc_t[ii][2 * k2] = (float)qr[x].x;
      qc_t[ii][2 * k2 + 1] = (float)qr[x].y;
    }
#pragma unroll
    for (int x = 0; x < ND; ++x) {
      const int c = tid + x * 256, ii = c / (D / 4), k4 = c % (D / 4);
      *reinterpret_cast<float4*>(&do_t[ii][4 * k4]) = dr[x];
    }
    __syncthreads();
#pragma unroll 4
    for (int ii = 0; ii < IC; ++ii) {
      const float x = ds_t[ii][pl], y = p_t[ii][pl];
#pragma unroll
      for (int k = 0; k < DPT; ++k) {
        dk[k] += x * qc_t[ii][d0 + k];
        dv[k] += y * do_t[ii][d0 + k];
      }
    }
  }
  const int p = p0 + pl;
  if (p >= s.N_kv) return;
  const int j = kept_id(s, a.ctx_idx + (size_t)bh * s.k_ctx, p);
  if (j < 0) return;
  const float rs = 1.0f / sqrtf((float)D);
  float* ok = a.dkc_out + (rbase + j) * D + d0;
  float* ov = a.dvc_out + (rbase + j) * D + d0;
#pragma unroll
  for (int k = 0; k < DPT; ++k) {
    ok[k] = (accumulate ? ok[k] : 0.f) + dk[k] * rs;
    ov[k] = (accumulate ? ov[k] : 0.f) + dv[k];
  }
}

// ---------------------------------------------------------------- dQ
// Query-major, as the forward: each wave owns 16*QT query rows. Sharp
// blocks all read the tokens of J, so a workgroup takes NWAVES*16*QT rows
// (several blocks) and the key tiles stream through two LDS buffers (PIPE);
// a flat block has its own key set (the tokens of E_i, then the pooled keys
// of J), so it gets a workgroup of its own (NWAVES*16*QT/KS = b).
enum : int { kSharp = 1, kFlat = 2 };

// KS = 2 (flat path, 32-token blocks): the waves split each key tile in two
// 32-key halves for the same rows; the halves' dQ sums are added at the end.
template <int D, int MODE, int QT, int NWAVES, bool PIPE, int KS = 1>
__global__ __launch_bounds__(NWAVES * 64) __attribute__((amdgpu_waves_per_eu(PIPE ? 2 : 3)))
void dq_kernel(BwdArgs a) {
  static_assert(KS == 1 || (KS == 2 && !PIPE && MODE == kFlat && NWAVES % 2 == 0), "key split");
  constexpr int NT = NWAVES * 64;
  constexpr int STR = 2 * D + 32;
  constexpr int CPR = D / 8;
  constexpr int CH = kKeyTile * CPR / NT;
  constexpr int KK = D / 32;
  constexpr int DT = D / 16;
  constexpr int ROWS_W = 16 * QT;
  constexpr int RW = NWAVES / KS;     // waves per key half
  constexpr int ROWS = RW * ROWS_W;
  constexpr int MTW = 4 / KS;         // 16-key sub-tiles per wave and tile
  static_assert(CH >= 1 && NT % CPR == 0, "tile split");
  // Buffer 0 of K, V and the logit offsets; the pipelined form adds buffer 1
  // as separate arrays, so that the compiler can tell the asynchronous
  // global->LDS copies into one buffer apart from the reads of the other.
  __shared__ __attribute__((aligned(16))) char k_lds[1][kKeyTile * STR];
  __shared__ __attribute__((aligned(16))) char v_lds[1][kKeyTile * STR];
  __shared__ __attribute__((aligned(16))) float bias_lds[1][kKeyTile];
  __shared__ __attribute__((aligned(16))) char k_ld1[PIPE ? kKeyTile * STR : 16];
  __shared__ __attribute__((aligned(16))) char v_ld1[PIPE ? kKeyTile * STR : 16];
  __shared__ __attribute__((aligned(16))) float bias_ld1[PIPE ? kKeyTile : 4];
  extern __shared__ int tabs[];   // sharp: [N_kv]; flat: [k_ns] then [N_kv]

  const IsaShape& s = a.s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int rwave = wave % RW, kh = wave / RW;   // row group, key half
  int qx = blockIdx.x, bh = blockIdx.y;
  // flat blocks in the forward's grid order (exact sets that overlap next
  // to each other), each XCD taking a contiguous run of it
  if (MODE == kFlat && a.flat_ord != nullptr) {
    const int total = gridDim.x * gridDim.y;
    if ((total & 7) == 0) {
      const int id = blockIdx.x + gridDim.x * blockIdx.y;
      const int logical = (id & 7) * (total >> 3) + (id >> 3);
      qx = logical % gridDim.x;
      bh = logical / gridDim.x;
    }
    qx = __builtin_amdgcn_readfirstlane(a.flat_ord[(size_t)bh * s.n_flat + qx]);
  }
  const size_t head = (size_t)bh * s.L;
  const int32_t* ctx_row = a.ctx_idx + (size_t)bh * s.k_ctx;
  const int b = s.b, lb = b == 64 ? 6 : 5;

  // this lane's query rows
  int qtok[QT];
  bool qval[QT];
  float lse2[QT], dl[QT];
  bf16x8_t qf[QT][KK], df[QT][KK];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int lr = rwave * ROWS_W + 16 * qt + c16;
    const int e = MODE == kSharp ? qx * (ROWS >> lb) + (lr >> lb) : qx;
    const int o = MODE == kSharp ? (lr & (b - 1)) : lr;
    qval[qt] = false;
    qtok[qt] = 0;
    if (e < a.n_q) {
      int st, n;
      isa_block_range_checked(s, a.qlist[(size_t)bh * a.n_q + e], st, n);
      qval[qt] = o < n;
      qtok[qt] = st + (qval[qt] ? o : 0);
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      uint4 wq = make_uint4(0, 0, 0, 0), wd = make_uint4(0, 0, 0, 0);
      if (qval[qt]) {
        wq = *reinterpret_cast<const uint4*>(a.Q + (head + qtok[qt]) * D + 32 * kk + 8 * g);
        wd = *reinterpret_cast<const uint4*>(a.dO + (head + qtok[qt]) * D + 32 * kk + 8 * g);
      }
      qf[qt][kk] = __builtin_bit_cast(bf16x8_t, wq);
      df[qt][kk] = __builtin_bit_cast(bf16x8_t, wd);
    }
    lse2[qt] = qval[qt] ? a.lse[head + qtok[qt]] : INFINITY;
    dl[qt] = qval[qt] ? a.delta[head + qtok[qt]] : 0.0f;
  }

  // key tables: (start << 7) | n per listed block; pooled: (j << 8) | (n << 1) | in_E
  int* jtab = tabs;
  int* ptab = tabs + (MODE == kFlat ? s.k_ns : 0);
  int ntab;
  if (MODE == kSharp) {
    ntab = s.N_kv;
    for (int q = tid; q < s.N_kv; q += NT) {
      const int j = kept_id(s, ctx_row, q);
      int st = 0, n = 0;
      if (j >= 0) isa_block_range(s, j, st, n);
      jtab[q] = (st << 7) | n;
    }
  } else {
    ntab = s.k_ns;
    const int32_t* ex = a.exact + ((size_t)bh * s.n_flat + qx) * s.k_ns;
    for (int q = tid; q < s.k_ns; q += NT) {
      const int j = ex[q];
      int st = 0, n = 0;
      if (j >= 0 && j < s.N) isa_block_range(s, j, st, n);
      jtab[q] = (st << 7) | n;
    }
    for (int p = tid; p < s.N_kv; p += NT) {
      const int j = kept_id(s, ctx_row, p);
      int st = 0, n = 0;
      if (j >= 0) isa_block_range(s, j, st, n);
      ptab[p] = j >= 0 ? ((j << 8) | (n << 1)) : 1;
    }
    __syncthreads();
    for (int q = tid; q < s.k_ns; q += NT) {
      const int p = kept_pos(s, ctx_row, ex[q]);
      if (p >= 0) ptab[p] |= 1;
    }
  }
  __syncthreads();

  const int per = kKeyTile >> lb;
  const uint16_t* Kh = a.K + head * D;
  const uint16_t* Vh = a.V + head * D;
  const uint16_t* kch = MODE == kFlat ? a.kcb + (size_t)bh * s.N * D : nullptr;
  const uint16_t* vch = MODE == kFlat ? a.vcb + (size_t)bh * s.N * D : nullptr;
  const float cscale = kLog2e / sqrtf((float)D);
  float4_t dq[QT][DT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) dq[qt][dt] = float4_t{0.f, 0.f, 0.f, 0.f};

  auto consume = [&](const char* kbuf, const char* vbuf, const float* bbuf) {
    const char* kb = kbuf + kh * 16 * MTW * STR;   // this wave's keys
    const char* vb = vbuf + kh * 16 * MTW * STR;
    const float* bb = bbuf + kh * 16 * MTW;
    float4_t sc[QT][MTW], dp[QT][MTW];
    mm_rows<D, MTW, QT>(kb, qf, sc, g, c16);
    // the probabilities need only S: the vector ALUs form them while the
    // matrix cores compute dP (group barriers interleave one MFMA with six
    // VALU ops)
    mm_rows<D, MTW, QT>(vb, df, dp, g, c16);
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt) {
      const float4_t bv = *reinterpret_cast<const float4_t*>(bb + 16 * mt + 4 * g);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sc[qt][mt][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[qt][mt][e], cscale, bv[e]) - lse2[qt]);
    }
#pragma unroll
    for (int i = 0; i < MTW * QT * 4 / 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
    }
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[qt][mt][e] = sc[qt][mt][e] * (dp[qt][mt][e] - dl[qt]);
    bf16x8_t pk[QT][MTW / 2];
    pack_bf16<MTW, QT>(sc, pk);
    mm_tr<D, MTW, QT>(kb, pk, dq, g, c16);
  };

  if constexpr (PIPE) {
    // K and V go global -> LDS directly (buffer loads into LDS), one tile
    // ahead. Wave w copies the 1 KiB pieces w, w + NWAVES, ... of each padded
    // tile; lane l of a piece holds its bytes 16 l .. 16 l + 15, i.e. chunk
    // (x % STR) / 16 of key slot x / STR (padding chunks copy data that is
    // never read). A piece lies within one listed block (block starts fall
    // on 1 KiB boundaries for b = 32, 64); a slot past the block's n tokens
    // copies the block's first row and gets logit offset -inf, so it adds
    // exactly zero. Each wave waits for its own copies before the barrier
    // that ends the step.
    static_assert(MODE == kSharp, "pipelined dQ is the sharp path");
    constexpr int KTB = kKeyTile * STR;
    constexpr int NPC = KTB / 1024;
    constexpr int NPW = (NPC + NWAVES - 1) / NWAVES;
    static_assert(KTB % 1024 == 0, "tile must be whole 1 KiB pieces");
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    int poff[NPW], pslot[NPW];
#pragma unroll
    for (int pp = 0; pp < NPW; ++pp) {
      const int x = (pp * NWAVES + wave_u) * 1024 + 16 * lane;
      const int row = x / STR, col = x - row * STR;
      pslot[pp] = row;
      poff[pp] = col < 2 * D ? col / 2 : 0;
    }
    const int head_bytes = (int)((size_t)s.L * D * 2);
    const RowsRsrc k_rs = rows_rsrc(Kh, head_bytes);
    const RowsRsrc v_rs = rows_rsrc(Vh, head_bytes);
    auto dma = [&](int t, char* kd, char* vd, float* bd) {
#pragma unroll
      for (int pp = 0; pp < NPW; ++pp) {
        const int piece = pp * NWAVES + wave_u;
        if (piece < NPC) {
          const int q = t * per + (((piece * 1024) / STR) >> lb);
          const int e = __builtin_amdgcn_readfirstlane(q < ntab ? jtab[q] : 0);
          const int o = pslot[pp] & (b - 1);
          const uint32_t lane_off = (uint32_t)(((o < (e & 127) ? o : 0) * D + poff[pp]) * 2);
          copy16_to_lds(k_rs, kd + piece * 1024, lane_off, (e >> 7) * D * 2);
          copy16_to_lds(v_rs, vd + piece * 1024, lane_off, (e >> 7) * D * 2);
        }
      }
      if (tid < kKeyTile) {
        const int q = t * per + (tid >> lb), o = tid & (b - 1);
        const int e = q < ntab ? jtab[q] : 0;
        bd[tid] = o < (e & 127) ? 0.0f : -INFINITY;
      }
    };
    dma(0, k_lds[0], v_lds[0], bias_lds[0]);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's copies landed
    __syncthreads();
    for (int t = 0; t < a.ntiles; t += 2) {
      {
        const bool more = t + 1 < a.ntiles;
        if (more) dma(t + 1, k_ld1, v_ld1, bias_ld1);
        consume(k_lds[0], v_lds[0], bias_lds[0]);
        if (more) __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        if (!more) break;
      }
      {
        const bool more = t + 2 < a.ntiles;
        if (more) dma(t + 2, k_lds[0], v_lds[0], bias_lds[0]);
        consume(k_ld1, v_ld1, bias_ld1);
        if (more) __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
      }
    }
  } else {
    // One LDS buffer, filled global -> LDS directly by buffer loads (the other
    // resident workgroups cover the copy latency): wave w copies the 1 KiB
    // pieces w, w + NWAVES, ... of the padded K and V tiles, lane l bytes
    // 16 l .. 16 l + 15 of a piece (row x / STR, byte column x % STR; padding
    // columns copy the row's first chunk, never read). A slot that holds no
    // key gets an offset past the end of every resource, so the copy writes
    // zeros, and logit offset -inf.
    constexpr int KTB = kKeyTile * STR;
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
      pslot[pp] = x / STR;
      const int col = x - pslot[pp] * STR;
      pcol[pp] = (uint32_t)(col < 2 * D ? col : 0);
    }
    const int head_bytes = (int)((size_t)s.L * D * 2), pooled_bytes = (int)((size_t)s.N * D * 2);
    const RowsRsrc k_rs = rows_rsrc(Kh, head_bytes), v_rs = rows_rsrc(Vh, head_bytes);
    const RowsRsrc kc_rs = rows_rsrc(kch, pooled_bytes), vc_rs = rows_rsrc(vch, pooled_bytes);
    for (int t = 0; t < a.ntiles; ++t) {
      if (t > 0) __syncthreads();   // previous tile fully consumed
      const bool pooled = MODE == kFlat && t >= a.ntiles_exact;
#pragma unroll
      for (int pp = 0; pp < NPW; ++pp) {
        const int piece = pp * NWAVES + wave_u;
        if (piece < NPC) {
          const int slot = pslot[pp];
          uint32_t off;
          if (pooled) {
            const int p = (t - a.ntiles_exact) * kKeyTile + slot;
            const int e = p < s.N_kv ? ptab[p] : 1;
            const bool valid = !(e & 1) && ((e >> 1) & 127) > 0;
            off = valid ? (uint32_t)((e >> 8) * D * 2) + pcol[pp] : kNoRow;
          } else {
            const int q = t * per + (slot >> lb), o = slot & (b - 1);
            const int e = q < ntab ? jtab[q] : 0;
            off = o < (e & 127) ? (uint32_t)(((e >> 7) + o) * D * 2) + pcol[pp] : kNoRow;
          }
          copy16_to_lds(pooled ? kc_rs : k_rs, k_lds[0] + piece * 1024, off, 0);
          copy16_to_lds(pooled ? vc_rs : v_rs, v_lds[0] + piece * 1024, off, 0);
        }
      }
      if (tid < kKeyTile) {
        float bias;
        if (pooled) {
          const int p = (t - a.ntiles_exact) * kKeyTile + tid;
          const int e = p < s.N_kv ? ptab[p] : 1;
          const int n = (e >> 1) & 127;
          bias = (!(e & 1) && n > 0) ? __log2f((float)n) : -INFINITY;
        } else {
          const int q = t * per + (tid >> lb), o = tid & (b - 1);
          const int e = q < ntab ? jtab[q] : 0;
          bias = o < (e & 127) ? 0.0f : -INFINITY;
        }
        bias_lds[0][tid] = bias;
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's copies landed
      __syncthreads();
      consume(k_lds[0], v_lds[0], bias_lds[0]);
    }
  }
  if constexpr (KS == 2) {
    // the second key half's waves hand their dQ sums over through the K
    // buffer (no longer read) and leave; the first half adds them
    float4_t* xq = reinterpret_cast<float4_t*>(&k_lds[0][0]);
    static_assert(RW * QT * DT * 64 * sizeof(float4_t) <= sizeof(k_lds[0]), "merge buffer");
    __syncthreads();
    if (kh == 1) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) xq[((rwave * QT + qt) * DT + dt) * 64 + lane] = dq[qt][dt];
    }
    __syncthreads();
    if (kh == 1) return;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) dq[qt][dt] += xq[((rwave * QT + qt) * DT + dt) * 64 + lane];
  }

  const float rs = 1.0f / sqrtf((float)D);
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    if (!qval[qt]) continue;
    const int pos = qtok[qt] < s.L_src ? qtok[qt] : qtok[qt] - s.L_src;
    uint16_t* row = a.dQ + (head + qtok[qt]) * D;
    // the residual reaches Q through the block mean
    const float* gq = nullptr;
    float inv_n = 0.f;
    if (a.dqc != nullptr) {
      const int jb = token_block(s, qtok[qt]);
      int st, n;
      isa_block_range(s, jb, st, n);
      gq = a.dqc + ((size_t)bh * s.N + jb) * D;
      inv_n = 1.0f / (float)n;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      float4_t x = dq[qt][dt] * rs;
      if (gq) x += *reinterpret_cast<const float4_t*>(gq + 16 * dt + 4 * g) * inv_n;
      store4(row, 16 * dt + 4 * g, x, a.rope, D / 2, pos);
    }
  }
}

// ---------------------------------------------------------------- dK, dV
// The pooled-key kernel streams query blocks (b token rows of Q and dO, with
// the rows' log-sum-exp and Delta) through two LDS buffers: the next block is
// fetched into registers while the current one is used. Rows past a block's
// n valid tokens are zero with log-sum-exp +inf, so they get probability 0.
// (The exact-key kernel below copies its query blocks straight into LDS.)
template <int D, int NT, int BR>
struct QueryStage {
  static constexpr int STR = 2 * D + 32;
  static constexpr int CPR = D / 8;
  static constexpr int NCH = BR * CPR;               // 16-byte chunks per tensor
  static constexpr int CHQ = (NCH + NT - 1) / NT;
  static_assert(NCH % NT == 0 || NCH < NT, "query tile split");
  uint4 q[CHQ], d[CHQ];
  float lv, dv;

  __device__ __forceinline__ void fetch(const BwdArgs& a, size_t head, int jq, int tid) {
    int st, n;
    isa_block_range_checked(a.s, jq, st, n);
#pragma unroll
    for (int i = 0; i < CHQ; ++i) {
      const int ch = tid + i * NT, r = ch / CPR, c = ch % CPR;
      q[i] = make_uint4(0, 0, 0, 0);
      d[i] = make_uint4(0, 0, 0, 0);
      if (ch < NCH && r < n) {
        q[i] = *reinterpret_cast<const uint4*>(a.Q + (head + st + r) * D + c * 8);
        d[i] = *reinterpret_cast<const uint4*>(a.dO + (head + st + r) * D + c * 8);
      }
    }
    lv = INFINITY;
    dv = 0.0f;
    if (tid < BR && tid < n) {
      lv = a.lse[head + st + tid];
      dv = a.delta[head + st + tid];
    }
  }

  __device__ __forceinline__ void put(char* q_lds, char* d_lds, float* l_lds, float* dl_lds, int tid) const {
#pragma unroll
    for (int i = 0; i < CHQ; ++i) {
      const int ch = tid + i * NT, r = ch / CPR, c = ch % CPR;
      if (ch < NCH) {
        *reinterpret_cast<uint4*>(q_lds + r * STR + c * 16) = q[i];
        *reinterpret_cast<uint4*>(d_lds + r * STR + c * 16) = d[i];
      }
    }
    if (tid < BR) {
      l_lds[tid] = lv;
      dl_lds[tid] = -dv;   // stored negated: the dP sums start from it
    }
  }
};

// One query block against this wave's 16*NF keys (kf, vf in registers,
// per-fragment additive logit kbias in log2 units): accumulates dK^T (raw,
// before the 1/sqrt(D) scale) and dV^T.
template <int D, int MT, int NF>
__device__ __forceinline__ void kv_block(const char* q_lds, const char* d_lds, const float* l_lds,
                                         const float* dl_lds, const bf16x8_t (&kf)[NF][D / 32],
                                         const bf16x8_t (&vf)[NF][D / 32], const float (&kbias)[NF],
                                         float cscale, float4_t (&dk)[NF][D / 16],
                                         float4_t (&dv)[NF][D / 16], int g, int c16) {
  float4_t sc[NF][MT], dp[NF][MT];
  mm_rows<D, MT, NF>(q_lds, kf, sc, g, c16);
  mm_rows<D, MT, NF>(d_lds, vf, dp, g, c16);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const float4_t lv = *reinterpret_cast<const float4_t*>(l_lds + 16 * mt + 4 * g);
    const float4_t dl = *reinterpret_cast<const float4_t*>(dl_lds + 16 * mt + 4 * g);
#pragma unroll
    for (int nf = 0; nf < NF; ++nf) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[nf][mt][e], cscale, kbias[nf]) - lv[e]);
        sc[nf][mt][e] = p;
        dp[nf][mt][e] = p * (dp[nf][mt][e] + dl[e]);
      }
    }
  }
  bf16x8_t pp[NF][MT / 2], pd[NF][MT / 2];
  pack_bf16<MT, NF>(sc, pp);
  pack_bf16<MT, NF>(dp, pd);
  mm_tr<D, MT, NF>(d_lds, pp, dv, g, c16);
  mm_tr<D, MT, NF>(q_lds, pd, dk, g, c16);
}

// Exact keys, producer/consumer form: one workgroup per 128 keys of J (whole
// kept blocks), 8 waves in 4 pairs, each pair owning 32 keys. The producer
// wave of a pair computes S = Q K^T and P for the current query block and
// passes P (bf16) to its consumer through LDS; it keeps its own packed copy
// and accumulates dV^T += dO^T P for that block at the start of the next
// step, so that its exponentials run while the consumer's products do. The
// consumer works one query block behind: dP = dO V^T, dS = P (dP - Delta)
// and dK^T += Q^T dS. Each operand read from LDS feeds two matrix-core
// products (32 keys per wave) while both roles stay within 256 registers, so
// two waves share each SIMD. Query blocks stream through three LDS buffers
// (the producer's, the consumer's and the one being filled), copied there
// with buffer loads into LDS while the other two are in use.
template <int D, int BR>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void dkv_pc_kernel(BwdArgs a) {
  constexpr int NT = 512;
  constexpr int MT = BR / 16;
  constexpr int NF = 2;                    // 32 keys per wave
  constexpr int KEYS = 128;
  constexpr int KPB = KEYS / BR;
  constexpr int STR = 2 * D + 32;
  constexpr int KK = D / 32;
  constexpr int DT = D / 16;
  constexpr int PX = NF * MT * 2;          // packed bf16 pairs of P per lane
  // The three query-block buffers of Q and of dO are separate arrays, so
  // that the compiler can tell the asynchronous global->LDS copies into one
  // buffer apart from the reads of the others.
  __shared__ __attribute__((aligned(16))) char q_l0[BR * STR];
  __shared__ __attribute__((aligned(16))) char q_l1[BR * STR];
  __shared__ __attribute__((aligned(16))) char q_l2[BR * STR];
  __shared__ __attribute__((aligned(16))) char d_l0[BR * STR];
  __shared__ __attribute__((aligned(16))) char d_l1[BR * STR];
  __shared__ __attribute__((aligned(16))) char d_l2[BR * STR];
  __shared__ __attribute__((aligned(16))) float l_lds[3][BR];
  __shared__ __attribute__((aligned(16))) float dl_lds[3][BR];
  __shared__ uint32_t pex[2][4][PX][64];

  const IsaShape& s = a.s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const bool producer = wave < 4;
  const int pair = wave & 3;
  // Every workgroup of a head streams the same query blocks; dispatch goes
  // round-robin over the 8 XCDs (each with its own L2), so the index is
  // remapped to give each XCD a contiguous run of key chunks, i.e. mostly
  // one head at a time (chunks vary fastest in the grid).
  int cx = blockIdx.x, bh = blockIdx.y;
  {
    const int total = gridDim.x * gridDim.y;
    if ((total & 7) == 0) {
      const int id = blockIdx.x + gridDim.x * blockIdx.y;
      const int logical = (id & 7) * (total >> 3) + (id >> 3);
      cx = logical % gridDim.x;
      bh = logical / gridDim.x;
    }
  }
  // chunks in the order the prep kernel set (longest streams first)
  if (s.n_flat > 0) cx = __builtin_amdgcn_readfirstlane(a.chunk_ord[(size_t)bh * s.N_kv + cx]);
  const int pb = cx * KPB;
  const size_t head = (size_t)bh * s.L;
  const int32_t* ctx_row = a.ctx_idx + (size_t)bh * s.k_ctx;

  int kb[NF], kj[NF], ktok[NF], kn[NF];
  bool kval[NF];
  // producer: K rows of its keys; consumer: V rows of the same keys
  bf16x8_t fr[NF][KK];
  const uint16_t* src = producer ? a.K : a.V;
#pragma unroll
  for (int nf = 0; nf < NF; ++nf) {
    const int kidx = pair * 32 + 16 * nf + c16;
    kb[nf] = kidx / BR;
    const int o = kidx % BR;
    kj[nf] = kept_id(s, ctx_row, pb + kb[nf]);
    int st = 0, n = 0;
    if (kj[nf] >= 0) isa_block_range(s, kj[nf], st, n);
    kn[nf] = n;
    kval[nf] = o < n;
    ktok[nf] = st + (kval[nf] ? o : 0);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (kval[nf]) w = *reinterpret_cast<const uint4*>(src + (head + ktok[nf]) * D + 32 * kk + 8 * g);
      fr[nf][kk] = __builtin_bit_cast(bf16x8_t, w);
    }
  }

  // query schedule: the sharp blocks, then each kept block's flat list
  const int32_t* srow = a.sharp_idx + (size_t)bh * s.n_sharp;
  const int32_t* off = a.inv_off + (size_t)bh * (s.N_kv + 1);
  const int32_t* lst = a.inv_list + (size_t)bh * s.n_flat * s.k_ns;
  int fb[KPB + 1];
  fb[0] = s.n_sharp;
#pragma unroll
  for (int u = 0; u < KPB; ++u) {
    const int p = pb + u;
    const int c = (s.n_flat > 0 && p < s.N_kv) ? off[p + 1] - off[p] : 0;
    fb[u + 1] = fb[u] + __builtin_amdgcn_readfirstlane(c);   // the same in every lane
  }
  const int total = fb[KPB];
  // start of each kept block's flat list (the same in every lane)
  int lbase[KPB];
#pragma unroll
  for (int u = 0; u < KPB; ++u)
    lbase[u] = (s.n_flat > 0 && pb + u < s.N_kv) ? __builtin_amdgcn_readfirstlane(off[pb + u]) : 0;
  // which of this workgroup's kept blocks a stream entry belongs to (-1: a
  // sharp block, read by all of them)
  auto act_of = [&](int i) -> int {
    if (i < s.n_sharp) return -1;
    int u = 0;
#pragma unroll
    for (int v = 0; v < KPB; ++v)
      if (i >= fb[v + 1]) u = v + 1;
    return u;
  };
  // block id of stream entry j (per lane; 0 past the end)
  auto entry_at = [&](int j) -> int {
    if (j >= total) return 0;
    if (j < s.n_sharp) return srow[j];
    const int u = act_of(j);
    return lst[lbase[u] + (j - fb[u])];
  };
  // The stream's block ids sit in two 64-entry windows across the lanes
  // (entries W .. W+63 and W+64 .. W+127), read with v_readlane: no memory
  // access on the step's critical path. The next window is loaded 64 steps
  // before it is needed.
  int W = 0;
  int win = entry_at(lane), wnext = entry_at(64 + lane);
  auto id_at = [&](int i) -> int {
    const int r = __builtin_amdgcn_readfirstlane(i - W);
    return r < 64 ? __builtin_amdgcn_readlane(win, r) : __builtin_amdgcn_readlane(wnext, r - 64);
  };
  auto slide = [&](int i) {   // keep entries i+1 .. i+2 inside the windows
    if (i + 1 >= W + 64) {
      W += 64;
      win = wnext;
      wnext = entry_at(W + 64 + lane);
    }
  };

  const float cscale = kLog2e / sqrtf((float)D);
  float4_t acc[NF][DT];   // producer: dV^T; consumer: dK^T (raw)
#pragma unroll
  for (int nf = 0; nf < NF; ++nf)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[nf][dt] = float4_t{0.f, 0.f, 0.f, 0.f};

  if (total > 0) {
    // Query blocks go global -> LDS directly (buffer loads into LDS) one
    // block ahead. Wave w copies the 1 KiB pieces w, w + 8, ... of the padded
    // Q block and pieces 7 - w, 15 - w, ... of the dO block; lane l of a piece
    // holds its bytes 16 l .. 16 l + 15, i.e. chunk (x % STR) / 16 of row
    // x / STR (padding chunks copy data that is never read). Rows past the
    // block's n tokens copy its first row and get log-sum-exp +inf, so their
    // probabilities, and every product they feed, are exactly zero. Each
    // wave waits for its own copies before the barrier that ends the step.
    constexpr int QTB = BR * STR;
    constexpr int NPC = QTB / 1024;
    constexpr int NPW = (NPC + 7) / 8;
    static_assert(QTB % 1024 == 0 && NT == 512, "query block must be whole 1 KiB pieces");
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    int qrow[NPW], qoff[NPW], drow[NPW], doff[NPW];
#pragma unroll
    for (int pp = 0; pp < NPW; ++pp) {
      {
        const int x = (pp * 8 + wave_u) * 1024 + 16 * lane;
        qrow[pp] = x / STR;
        const int col = x - qrow[pp] * STR;
        qoff[pp] = col < 2 * D ? col / 2 : 0;
      }
      {
        const int x = (pp * 8 + 7 - wave_u) * 1024 + 16 * lane;
        drow[pp] = x / STR;
        const int col = x - drow[pp] * STR;
        doff[pp] = col < 2 * D ? col / 2 : 0;
      }
    }
    float lv = INFINITY, dv = 0.0f;
    const int head_bytes = (int)((size_t)s.L * D * 2);
    const RowsRsrc q_rs = rows_rsrc(a.Q + head * D, head_bytes);
    const RowsRsrc d_rs = rows_rsrc(a.dO + head * D, head_bytes);
    auto fetch = [&](int jq, char* qd, char* dd) {
      int st, n;
      isa_block_range_checked(s, jq, st, n);
#pragma unroll
      for (int pp = 0; pp < NPW; ++pp) {
        const int pq = pp * 8 + wave_u, pd = pp * 8 + 7 - wave_u;
        if (pq < NPC)
          copy16_to_lds(q_rs, qd + pq * 1024, (uint32_t)(((qrow[pp] < n ? qrow[pp] : 0) * D + qoff[pp]) * 2),
                        st * D * 2);
        if (pd < NPC)
          copy16_to_lds(d_rs, dd + pd * 1024, (uint32_t)(((drow[pp] < n ? drow[pp] : 0) * D + doff[pp]) * 2),
                        st * D * 2);
      }
      lv = INFINITY;
      dv = 0.0f;
      if (tid < BR && tid < n) {
        lv = a.lse[head + st + tid];
        dv = a.delta[head + st + tid];
      }
    };
    auto put_stats = [&](int buf) {
      if (tid < BR) {
        l_lds[buf][tid] = lv;
        dl_lds[buf][tid] = -dv;   // stored negated: the dP sums start from it
      }
    };
    bf16x8_t pcar[NF][MT / 2];
    int act_cur = act_of(0);
    fetch(id_at(0), q_l0, d_l0);
    put_stats(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's copies landed
    __syncthreads();
    // One step i: producer on buffer cur (i % 3), consumer on prev
    // ((i + 2) % 3), next block copied into next ((i + 1) % 3).
    auto step = [&](int i, int cur, int prev, int next, const char* QC, const char* DC, const char* QP,
                    const char* DP, char* QN, char* DN) __attribute__((always_inline)) {
      int par = i & 1;
      asm volatile("" : "+s"(cur), "+s"(prev), "+s"(next), "+s"(par));
      slide(i);
      const bool more = i + 1 < total;
      const int act_next = more ? act_of(i + 1) : -1;
      if (more) fetch(id_at(i + 1), QN, DN);
      if (producer) {
        if (i > 0) {
          mm_tr<D, MT, NF>(DP, pcar, acc, g, c16);
          ahead<DT * (MT / 2), NF, 2, kDkvAhead, 2>();
        }
        if (i < total) {
          float kbias[NF];
#pragma unroll
          for (int nf = 0; nf < NF; ++nf)
            kbias[nf] = (kval[nf] && (act_cur < 0 || act_cur == kb[nf])) ? 0.0f : -INFINITY;
          float4_t sc[NF][MT];
          mm_rows<D, MT, NF>(QC, fr, sc, g, c16);
          ahead<KK * MT, NF, 1, kDkvAhead, 1>();
          bool open = act_cur < 0;   // no key of this wave masked (sharp blocks, full kept blocks)
#pragma unroll
          for (int nf = 0; nf < NF; ++nf) open = open && kval[nf];
          if (__all(open)) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              const float4_t lv = *reinterpret_cast<const float4_t*>(l_lds[cur] + 16 * mt + 4 * g);
#pragma unroll
              for (int nf = 0; nf < NF; ++nf)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  sc[nf][mt][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[nf][mt][e], cscale, -lv[e]));
            }
          } else {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              const float4_t lv = *reinterpret_cast<const float4_t*>(l_lds[cur] + 16 * mt + 4 * g);
#pragma unroll
              for (int nf = 0; nf < NF; ++nf)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  sc[nf][mt][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[nf][mt][e], cscale, kbias[nf]) - lv[e]);
            }
          }
          bf16x8_t (&pp)[NF][MT / 2] = pcar;
          pack_bf16<MT, NF>(sc, pp);
          // the consumer's copy of P: the operand words themselves. Word u of
          // pp[nf][kc] holds the bf16 pair (2h, 2h+1), h = u % 2, of fragment
          // mt = 2kc + u / 2: the word the consumer reads at 2 (nf MT + mt) + h.
          uint32_t* px = &pex[par][pair][0][lane];
#pragma unroll
          for (int nf = 0; nf < NF; ++nf)
#pragma unroll
            for (int kc = 0; kc < MT / 2; ++kc) {
              const uint4 w = __builtin_bit_cast(uint4, pp[nf][kc]);
              px[(2 * nf * MT + 4 * kc) * 64] = w.x;
              px[(2 * nf * MT + 4 * kc + 1) * 64] = w.y;
              px[(2 * nf * MT + 4 * kc + 2) * 64] = w.z;
              px[(2 * nf * MT + 4 * kc + 3) * 64] = w.w;
            }
        }
      } else if (i > 0) {
        // dP - Delta: the sums start from -Delta of each row
        float4_t dp[NF][MT];
        mm_rows_from<D, MT, NF>(DP, fr, dp, dl_lds[prev], g, c16);
        ahead<KK * MT, NF, 1, kDkvAhead, 3>();
        const uint32_t* px = &pex[par ^ 1][pair][0][lane];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
          for (int nf = 0; nf < NF; ++nf) {
            const uint32_t u0 = px[(2 * (nf * MT + mt)) * 64], u1 = px[(2 * (nf * MT + mt) + 1) * 64];
            const float p[4] = {__uint_as_float(u0 << 16), __uint_as_float(u0 & 0xffff0000u),
                                __uint_as_float(u1 << 16), __uint_as_float(u1 & 0xffff0000u)};
#pragma unroll
            for (int e = 0; e < 4; ++e) dp[nf][mt][e] = p[e] * dp[nf][mt][e];
          }
        }
        bf16x8_t pd[NF][MT / 2];
        pack_bf16<MT, NF>(dp, pd);
        mm_tr<D, MT, NF>(QP, pd, acc, g, c16);
        ahead<DT * (MT / 2), NF, 2, kDkvAhead, 4>();
      }
      if (more) {
        put_stats(next);
        __builtin_amdgcn_s_waitcnt(0x0F70);
      }
      __syncthreads();
      act_cur = act_next;
    };
    for (int i = 0; i <= total; i += 3) {
      step(i, 0, 2, 1, q_l0, d_l0, q_l2, d_l2, q_l1, d_l1);
      if (i + 1 > total) break;
      step(i + 1, 1, 0, 2, q_l1, d_l1, q_l0, d_l0, q_l2, d_l2);
      if (i + 2 > total) break;
      step(i + 2, 2, 1, 0, q_l2, d_l2, q_l1, d_l1, q_l0, d_l0);
    }
  }

  const float rs = 1.0f / sqrtf((float)D);
#pragma unroll
  for (int nf = 0; nf < NF; ++nf) {
    if (!kval[nf]) continue;
    const int j = kj[nf];
    const float inv_n = 1.0f / (float)kn[nf];
    const int pos = ktok[nf] - (j < s.N_src ? 0 : s.L_src);
    // pooled-key gradients reach every token of the block through the mean
    const float* gp = producer ? a.dvc : a.dkc;
    if (gp) gp += ((size_t)bh * s.N + j) * D;
    uint16_t* row = (producer ? a.dV : a.dK) + (head + ktok[nf]) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d0 = 16 * dt + 4 * g;
      float4_t x = producer ? acc[nf][dt] : acc[nf][dt] * rs;
      if (gp) x += *reinterpret_cast<const float4_t*>(gp + d0) * inv_n;
      store4(row, d0, x, producer ? nullptr : a.rope, D / 2, pos);
    }
  }
}

// Zero gradients for the tokens of pruned context blocks (not in J).
template <int D>
__global__ __launch_bounds__(256) void zero_pruned_kernel(BwdArgs a) {
  const IsaShape& s = a.s;
  const int bh = blockIdx.x, j = s.N_src + blockIdx.y;
  const int32_t* ctx_row = a.ctx_idx + (size_t)bh * s.k_ctx;
  if (kept_pos(s, ctx_row, j) >= 0) return;
  int st, n;
  isa_block_range(s, j, st, n);
  constexpr int CPR = D / 8;
  const size_t head = (size_t)bh * s.L;
  for (int ch = threadIdx.x; ch < n * CPR; ch += 256) {
    const size_t off = (head + st + ch / CPR) * D + (ch % CPR) * 8;
    *reinterpret_cast<uint4*>(a.dK + off) = make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(a.dV + off) = make_uint4(0, 0, 0, 0);
  }
}

// Pooled keys: one workgroup per 64 positions of J (4 waves of 16), over
// every flat block; writes dKc (scaled) and dVc in fp32 by global block id.
template <int D, int MT>
__global__ __launch_bounds__(256) void dkv_pooled_kernel(BwdArgs a) {
  constexpr int NT = 256;
  constexpr int BR = MT * 16;
  constexpr int STR = 2 * D + 32;
  constexpr int KK = D / 32;
  constexpr int DT = D / 16;
  __shared__ __attribute__((aligned(16))) char q_lds[2][BR * STR];
  __shared__ __attribute__((aligned(16))) char d_lds[2][BR * STR];
  __shared__ __attribute__((aligned(16))) float l_lds[2][BR];
  __shared__ __attribute__((aligned(16))) float dl_lds[2][BR];

  const IsaShape& s = a.s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int bh = blockIdx.x, p0 = blockIdx.y * kKeyTile;
  const size_t head = (size_t)bh * s.L;
  const int32_t* ctx_row = a.ctx_idx + (size_t)bh * s.k_ctx;
  const int kp = p0 + wave * 16 + c16;
  const int jg = kp < s.N_kv ? kept_id(s, ctx_row, kp) : -1;
  int kst = 0, kn = 0;
  if (jg >= 0) isa_block_range(s, jg, kst, kn);
  const bool kval = jg >= 0 && kn > 0;
  bf16x8_t kf[1][KK], vf[1][KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    uint4 wk = make_uint4(0, 0, 0, 0), wv = make_uint4(0, 0, 0, 0);
    if (kval) {
      wk = *reinterpret_cast<const uint4*>(a.kcb + ((size_t)bh * s.N + jg) * D + 32 * kk + 8 * g);
      wv = *reinterpret_cast<const uint4*>(a.vcb + ((size_t)bh * s.N + jg) * D + 32 * kk + 8 * g);
    }
    kf[0][kk] = __builtin_bit_cast(bf16x8_t, wk);
    vf[0][kk] = __builtin_bit_cast(bf16x8_t, wv);
  }
  const float kb0 = kval ? __log2f((float)kn) : -INFINITY;
  const float cscale = kLog2e / sqrtf((float)D);
  const int32_t* frow = a.flat_idx + (size_t)bh * s.n_flat;
  const uint64_t* bits = a.ebits + (size_t)bh * s.n_flat * a.W + (p0 >> 6);
  float4_t dk[1][DT], dv[1][DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dk[0][dt] = dv[0][dt] = float4_t{0.f, 0.f, 0.f, 0.f};
  QueryStage<D, NT, BR> stage;
  stage.fetch(a, head, frow[0], tid);
  stage.put(q_lds[0], d_lds[0], l_lds[0], dl_lds[0], tid);
  __syncthreads();
  for (int r = 0; r < s.n_flat; ++r) {
    const int buf = r & 1;
    const bool more = r + 1 < s.n_flat;
    if (more) stage.fetch(a, head, frow[r + 1], tid);
    const uint64_t w = bits[(size_t)r * a.W];
    const float kbias[1] = {((w >> (kp - p0)) & 1ull) ? -INFINITY : kb0};
    kv_block<D, MT, 1>(q_lds[buf], d_lds[buf], l_lds[buf], dl_lds[buf], kf, vf, kbias, cscale, dk, dv,
                       g, c16);
    if (more) stage.put(q_lds[buf ^ 1], d_lds[buf ^ 1], l_lds[buf ^ 1], dl_lds[buf ^ 1], tid);
    __syncthreads();
  }
  if (!kval) return;
  const float rs = 1.0f / sqrtf((float)D);
  float* ok = a.dkc_out + ((size_t)bh * s.N + jg) * D;
  float* ov = a.dvc_out + ((size_t)bh * s.N + jg) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const int d0 = 16 * dt + 4 * g;
    *reinterpret_cast<float4_t*>(ok + d0) = dk[0][dt] * rs;
    *reinterpret_cast<float4_t*>(ov + d0) = dv[0][dt];
  }
}

// The dQ kernels take their block tables in dynamic LDS: their limit is
// raised once per instantiation and device (host-side only).
template <int D, int MODE, int QT, int NWAVES, bool PIPE, int KS = 1>
hipError_t prepare_dq() {
  static unsigned long long done = 0;
  return isa_ensure_dyn_lds(reinterpret_cast<const void*>(&dq_kernel<D, MODE, QT, NWAVES, PIPE, KS>),
                            2 * ISA_MAX_NKV * (int)sizeof(int), &done);
}

template <int D>
hipError_t launch_all(const IsaShape& s, BwdArgs a, const uint16_t* O, hipStream_t st) {
  const int BH = s.B * s.H;
  hipError_t e = hipSuccess;
  if (s.n_flat > 0) {
    bwd_prep_kernel<<<BH, kPrepThreads, 0, st>>>(a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const bool residual = s.gamma != 0.0f;
  if (!residual) a.dqc = a.doc = a.ocs = nullptr;
  if (residual) {
    res_dosum_kernel<D><<<dim3(s.N, BH), kResThreads, 0, st>>>(a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    res_row_kernel<D><<<dim3((s.N + kResRows - 1) / kResRows, BH), kResThreads, 0, st>>>(a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const size_t rows = (size_t)BH * s.L;
    const size_t threads = rows * (D / 8);
    delta_kernel<D><<<(unsigned)((threads + 255) / 256), 256, 0, st>>>(a, O, rows);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const bool pooled = s.n_flat > 0 && s.k_ns < s.N_kv;
  if (pooled) {
    dim3 grid(BH, (s.N_kv + kKeyTile - 1) / kKeyTile);
    if (s.b == 64) dkv_pooled_kernel<D, 4><<<grid, 256, 0, st>>>(a);
    else dkv_pooled_kernel<D, 2><<<grid, 256, 0, st>>>(a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (residual) {
    res_col_kernel<D><<<dim3((s.N_kv + 63) / 64, BH), 256, 0, st>>>(a, pooled ? 1 : 0);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    BwdArgs k = a;
    if (!pooled && !residual) k.dkc = k.dvc = nullptr;
    const int kpb = 128 / s.b;   // 128 keys per workgroup
    dim3 grid((s.N_kv + kpb - 1) / kpb, BH);
    if (s.b == 64) dkv_pc_kernel<D, 64><<<grid, 512, 0, st>>>(k);
    else dkv_pc_kernel<D, 32><<<grid, 512, 0, st>>>(k);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (s.N_ctx > s.k_ctx) {
      zero_pruned_kernel<D><<<dim3(BH, s.N_ctx), 256, 0, st>>>(k);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (s.n_sharp > 0) {
    BwdArgs q = a;
    q.qlist = a.sharp_idx;
    q.n_q = s.n_sharp;
    q.ntiles_exact = q.ntiles = (s.N_kv * s.b + kKeyTile - 1) / kKeyTile;
    constexpr int ROWS = 8 * 32;   // 8 waves of 32 rows
    dim3 grid((s.n_sharp + ROWS / s.b - 1) / (ROWS / s.b), BH);
    const size_t dyn = (size_t)s.N_kv * sizeof(int);
    const hipError_t attr = prepare_dq<D, kSharp, 2, 8, true>();
    if (attr != hipSuccess) return attr;
    dq_kernel<D, kSharp, 2, 8, true><<<grid, 512, dyn, st>>>(q);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (s.n_flat > 0) {
    BwdArgs q = a;
    q.qlist = a.flat_idx;
    q.n_q = s.n_flat;
    q.ntiles_exact = (s.k_ns * s.b + kKeyTile - 1) / kKeyTile;
    q.ntiles = q.ntiles_exact + (s.k_ns < s.N_kv ? (s.N_kv + kKeyTile - 1) / kKeyTile : 0);
    dim3 grid(s.n_flat, BH);
    const size_t dyn = (size_t)(s.k_ns + s.N_kv) * sizeof(int);
    if (s.b == 64) {
      const hipError_t attr = prepare_dq<D, kFlat, 1, 4, false>();
      if (attr != hipSuccess) return attr;
      dq_kernel<D, kFlat, 1, 4, false><<<grid, 256, dyn, st>>>(q);
    } else {
      const hipError_t attr = prepare_dq<D, kFlat, 1, 4, false, 2>();
      if (attr != hipSuccess) return attr;
      dq_kernel<D, kFlat, 1, 4, false, 2><<<grid, 256, dyn, st>>>(q);
    }
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

hipError_t isa_bwd_prepare_device() {
  hipError_t e = hipSuccess;
  for (hipError_t x : {prepare_dq<128, kSharp, 2, 8, true>(), prepare_dq<64, kSharp, 2, 8, true>(),
                       prepare_dq<128, kFlat, 1, 4, false>(), prepare_dq<64, kFlat, 1, 4, false>(),
                       prepare_dq<128, kFlat, 1, 4, false, 2>(), prepare_dq<64, kFlat, 1, 4, false, 2>()})
    if (e == hipSuccess) e = x;
  return e;
}

hipError_t isa_launch_backward(const IsaShape& s, const IsaBwdBuffers& w, hipStream_t st) {
  BwdArgs a{};
  a.s = s;
  a.Q = w.Q;
  a.K = w.K;
  a.V = w.V;
  a.dO = w.dO;
  a.lse = w.lse;
  a.delta = w.delta;
  a.kcb = w.kcb;
  a.vcb = w.vcb;
  a.ctx_idx = w.ctx_idx;
  a.sharp_idx = w.sharp_idx;
  a.flat_idx = w.flat_idx;
  a.exact = w.exact;
  a.flat_ord = w.flat_ord;
  a.ebits = w.ebits;
  a.inv_off = w.inv_off;
  a.inv_list = w.inv_list;
  a.chunk_ord = w.chunk_ord;
  a.dkc = a.dkc_out = w.dkc;
  a.dvc = a.dvc_out = w.dvc;
  a.rope = w.rope;
  a.srows = w.srows;
  a.qc = w.qc;
  a.kc = w.kc;
  a.dqc = w.dqc;
  a.doc = w.doc;
  a.ocs = w.ocs;
  a.dsc = w.dsc;
  a.pc = w.pc;
  a.dQ = w.dQ;
  a.dK = w.dK;
  a.dV = w.dV;
  a.W = (s.N_kv + 63) / 64;
  return s.D == 128 ? launch_all<128>(s, a, w.O, st) : launch_all<64>(s, a, w.O, st);
}
