// Selection path of In-context Sparse Attention, all scores in fp64.
//
// Steps, as given in the paper.rainbus.top summary of arXiv 2605.04569,
// section "Method steps":
//   step (2): context importance = coarse scores of the source query blocks
//             summed per context key block; keep the top alpha_s fraction;
//   step (1)+(3): coarse rows S[i, J] = Qc_i . Kc_j / sqrt(D) over the kept
//             blocks J; sharpness M_i = variance of the softmax of S[i, :]
//             restricted to the source key blocks; the least sharp alpha_f
//             fraction of query blocks is "flat";
//   step (5): per flat block, the exact set E_i = top alpha_ns fraction of J
//             by coarse score.
// Every top-k prefers the lower index among equal scores, and every output
// list is ascending. Selection uses an exact radix bisection on the ordered
// bit pattern of the fp64 scores (no floating-point comparison tolerance),
// then resolves ties at the threshold by index order with a block-wide scan.
#include "isa_internal.h"

namespace {

// Maps an fp64 value to an unsigned key with the same order (no NaN input).
__device__ inline unsigned long long order_key(double x) {
  unsigned long long u = (unsigned long long)__double_as_longlong(x);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

__device__ inline int wave_sum_int(int x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__device__ inline double wave_sum_f64(double x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__device__ inline double wave_max_f64(double x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x = fmax(x, __shfl_xor(x, off, 64));
  return x;
}

// Sum of one int per thread over the workgroup; every thread gets the sum.
// `scratch` holds NT/64 ints of LDS.
template <int NT>
__device__ inline int block_sum_int(int x, int* scratch) {
  x = wave_sum_int(x);
  const int wave = threadIdx.x / 64;
  if ((threadIdx.x & 63) == 0) scratch[wave] = x;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) t += scratch[w];
  __syncthreads();
  return t;
}

// Exclusive prefix sum over threads in thread order; `scratch` NT/64 ints.
template <int NT>
__device__ inline int block_exclusive_scan(int x, int* scratch) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x / 64;
  int inc = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(inc, off, 64);
    if (lane >= off) inc += y;
  }
  if (lane == 63) scratch[wave] = inc;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += scratch[w];
  __syncthreads();
  return before + inc - x;
}

// Marks the k largest keys among the valid items (lower index wins ties).
// Thread t holds items t*IPT .. t*IPT+IPT-1 (index order == thread order).
template <int NT, int IPT>
__device__ void block_topk(const unsigned long long (&key)[IPT], const bool (&valid)[IPT], int k,
                           bool (&sel)[IPT], int* scratch) {
  if (k <= 0) {
#pragma unroll
    for (int u = 0; u < IPT; ++u) sel[u] = false;
    return;
  }
  // Largest threshold T with #{key >= T} >= k: the k-th largest key. Once
  // exactly k keys are at or above a trial threshold they are the top k (the
  // k-th key and everything equal to it lie above it), so the search stops.
  unsigned long long T = 0;
  for (int bit = 63; bit >= 0; --bit) {
    const unsigned long long trial = T | (1ull << bit);
    int c = 0;
#pragma unroll
    for (int u = 0; u < IPT; ++u) c += (valid[u] && key[u] >= trial) ? 1 : 0;
    const int tot = block_sum_int<NT>(c, scratch);
    if (tot >= k) {
      T = trial;
      if (tot == k) break;
    }
  }
  int gt = 0, ties = 0;
#pragma unroll
  for (int u = 0; u < IPT; ++u) {
    gt += (valid[u] && key[u] > T) ? 1 : 0;
    ties += (valid[u] && key[u] == T) ? 1 : 0;
  }
  const int need = k - block_sum_int<NT>(gt, scratch);
  int tie_rank = block_exclusive_scan<NT>(ties, scratch);
#pragma unroll
  for (int u = 0; u < IPT; ++u) {
    const bool tie = valid[u] && key[u] == T;
    sel[u] = (valid[u] && key[u] > T) || (tie && tie_rank < need);
    if (tie) ++tie_rank;
  }
}

// Writes the items with flag == want, in index order, to out[pos] = map(i).
template <int NT, int IPT, typename Map>
__device__ void block_compact(const bool (&flag)[IPT], const bool (&valid)[IPT], bool want,
                              int32_t* out, Map map, int* scratch) {
  int cnt = 0;
#pragma unroll
  for (int u = 0; u < IPT; ++u) cnt += (valid[u] && flag[u] == want) ? 1 : 0;
  int pos = block_exclusive_scan<NT>(cnt, scratch);
#pragma unroll
  for (int u = 0; u < IPT; ++u) {
    if (valid[u] && flag[u] == want) out[pos++] = map(threadIdx.x * IPT + u);
  }
}

__device__ inline int kept_block_id(const IsaShape& s, const int32_t* ctx_row, int p) {
  return p < s.N_src ? p : ctx_row[p - s.N_src];
}

// ---------------------------------------------------------------- step (2)
constexpr int kCtxThreads = 1024;
constexpr int kCtxIPT = ISA_MAX_SEG_BLOCKS / kCtxThreads;

__global__ __launch_bounds__(kCtxThreads) void ctx_topk_kernel(IsaShape s, const double* __restrict__ qc,
                                                               const double* __restrict__ kc,
                                                               int32_t* __restrict__ ctx_idx,
                                                               double* __restrict__ ctx_score) {
  const int bh = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int NW = kCtxThreads / 64;
  __shared__ double part[kCtxThreads * 2];
  __shared__ double qbar[128];
  __shared__ double score[ISA_MAX_SEG_BLOCKS];
  __shared__ int scratch[kCtxThreads / 64];
  const int D = s.D;
  // qbar = sum of the source rows of Qc: 16-byte loads, one partial per
  // group of rows, the groups then summed in a fixed order
  {
    const int cpr = D / 2, groups = kCtxThreads / cpr;
    const int c = tid % cpr, gq = tid / cpr;
    const double* src = qc + (size_t)bh * s.N * D + 2 * c;
    double a0 = 0.0, a1 = 0.0;
#pragma unroll 8
    for (int i = gq; i < s.N_src; i += groups) {
      const double2 v = *reinterpret_cast<const double2*>(src + (size_t)i * D);
      a0 += v.x;
      a1 += v.y;
    }
    part[gq * D + 2 * c] = a0;
    part[gq * D + 2 * c + 1] = a1;
    __syncthreads();
    if (tid < D) {
      double acc = 0.0;
      for (int g = 0; g < groups; ++g) acc += part[g * D + tid];
      qbar[tid] = acc;
    }
    __syncthreads();
  }
  // r_j = qbar . Kc_j / sqrt(D): D/2 lanes per context block (two fp64 each)
  // and a butterfly sum across them
  const double sq = sqrt((double)D);
  {
    const int sub = D / 2, bpw = 64 / sub;
    const int sl = lane % sub, sb = lane / sub;
    const double q0 = qbar[2 * sl], q1 = qbar[2 * sl + 1];
    const double* kbase = kc + ((size_t)bh * s.N + s.N_src) * D + 2 * sl;
#pragma unroll 4
    for (int j0 = wave * bpw; j0 < s.N_ctx; j0 += NW * bpw) {
      const int j = j0 + sb;
      double acc = 0.0;
      if (j < s.N_ctx) {
        const double2 k = *reinterpret_cast<const double2*>(kbase + (size_t)j * D);
        acc = fma(q1, k.y, q0 * k.x);
      }
      for (int off = 1; off < sub; off <<= 1) acc += __shfl_xor(acc, off, 64);
      if (sl == 0 && j < s.N_ctx) score[j] = acc / sq;
    }
  }
  __syncthreads();
  unsigned long long key[kCtxIPT];
  bool valid[kCtxIPT], sel[kCtxIPT];
#pragma unroll
  for (int u = 0; u < kCtxIPT; ++u) {
    const int j = tid * kCtxIPT + u;
    valid[u] = j < s.N_ctx;
    key[u] = 0;
    if (valid[u]) {
      const double r = score[j];
      if (ctx_score) ctx_score[(size_t)bh * s.N_ctx + j] = r;
      key[u] = order_key(r);
    }
  }
  if (s.k_ctx == 0) return;
  block_topk<kCtxThreads, kCtxIPT>(key, valid, s.k_ctx, sel, scratch);
  const int n_src = s.N_src;
  block_compact<kCtxThreads, kCtxIPT>(sel, valid, true, ctx_idx + (size_t)bh * s.k_ctx,
                                      [n_src](int j) { return n_src + j; }, scratch);
}

// ------------------------------------------------- step (1) coarse rows
// S[i, p] = Qc_i . Kc_{J[p]} / sqrt(D) in fp64 for a 64 x 64 tile per
// workgroup; each thread accumulates a 4 x 4 block from LDS-staged slices.
constexpr int kCoarseRows = 64, kCoarseCols = 64, kCoarseDc = 16;

__global__ __launch_bounds__(256) void coarse_rows_kernel(IsaShape s, const double* __restrict__ qc,
                                                          const double* __restrict__ kc,
                                                          const int32_t* __restrict__ ctx_idx,
                                                          double* __restrict__ srows) {
  const int i0 = blockIdx.x * kCoarseRows, p0 = blockIdx.y * kCoarseCols, bh = blockIdx.z;
  const int D = s.D;
  __shared__ double qs[kCoarseDc][kCoarseRows + 1];
  __shared__ double ks[kCoarseDc][kCoarseCols + 1];
  __shared__ int gid[kCoarseCols];
  const int32_t* ctx_row = ctx_idx + (size_t)bh * s.k_ctx;
  if (threadIdx.x < kCoarseCols) {
    const int p = p0 + threadIdx.x;
    int g = p < s.N_kv ? kept_block_id(s, ctx_row, p) : -1;
    gid[threadIdx.x] = (g >= 0 && g < s.N) ? g : -1;   // ids outside [0, N) read as zero rows
  }
  const int tr = threadIdx.x >> 4, tc = threadIdx.x & 15;   // rows 4tr.., cols tc + 16c
  double acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = 0.0;
  __syncthreads();
  const int lr = threadIdx.x >> 2, ld = (threadIdx.x & 3) * 4;   // loader: row, 4 dims
  // the next slice is loaded into registers while the current one is used
  const int li = i0 + lr, lg = gid[lr];
  const double* qrow = qc + ((size_t)bh * s.N + (li < s.N ? li : 0)) * D + ld;
  const double* krow = kc + ((size_t)bh * s.N + (lg >= 0 ? lg : 0)) * D + ld;
  double2 qn[2], kn[2];
  auto load = [&](int d0) {
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      qn[x] = li < s.N ? *reinterpret_cast<const double2*>(qrow + d0 + 2 * x) : make_double2(0.0, 0.0);
      kn[x] = lg >= 0 ? *reinterpret_cast<const double2*>(krow + d0 + 2 * x) : make_double2(0.0, 0.0);
    }
  };
  load(0);
  for (int d0 = 0; d0 < D; d0 += kCoarseDc) {
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      qs[ld + 2 * x][lr] = qn[x].x;
      qs[ld + 2 * x + 1][lr] = qn[x].y;
      ks[ld + 2 * x][lr] = kn[x].x;
      ks[ld + 2 * x + 1][lr] = kn[x].y;
    }
    __syncthreads();
    if (d0 + kCoarseDc < D) load(d0 + kCoarseDc);
#pragma unroll
    for (int dd = 0; dd < kCoarseDc; ++dd) {
      double a[4], bv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] = qs[dd][4 * tr + r];
#pragma unroll
      for (int c = 0; c < 4; ++c) bv[c] = ks[dd][tc + 16 * c];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = fma(a[r], bv[c], acc[r][c]);
    }
    __syncthreads();
  }
  const double sq = sqrt((double)D);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = i0 + 4 * tr + r;
    if (i >= s.N) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int p = p0 + tc + 16 * c;
      if (p < s.N_kv) srows[((size_t)bh * s.N + i) * s.N_kv + p] = acc[r][c] / sq;
    }
  }
}

// ------------------------------------------------------ step (3) sharpness
__global__ __launch_bounds__(256) void sharpness_kernel(IsaShape s, const double* __restrict__ srows,
                                                        double* __restrict__ sharp) {
  const int wave = threadIdx.x / 64, lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + wave, bh = blockIdx.y;
  if (i >= s.N) return;   // whole wave; no workgroup barrier below
  const double* row = srows + ((size_t)bh * s.N + i) * s.N_kv;   // source columns first
  const int n = s.N_src;
  double mx = -INFINITY;
  for (int j = lane; j < n; j += 64) mx = fmax(mx, row[j]);
  mx = wave_max_f64(mx);
  double z = 0.0;
  for (int j = lane; j < n; j += 64) z += exp(row[j] - mx);
  z = wave_sum_f64(z);
  const double inv_n = 1.0 / (double)n;
  double acc = 0.0;
  for (int j = lane; j < n; j += 64) {
    const double pr = exp(row[j] - mx) / z - inv_n;
    acc += pr * pr;
  }
  acc = wave_sum_f64(acc);
  if (lane == 0) sharp[(size_t)bh * s.N + i] = acc / (double)n;
}

// ----------------------------------------------------------- step (3) split
constexpr int kSplitThreads = 1024;
constexpr int kSplitIPT = 2 * ISA_MAX_SEG_BLOCKS / kSplitThreads;

__global__ __launch_bounds__(kSplitThreads) void split_kernel(IsaShape s, const double* __restrict__ sharp,
                                                              int32_t* __restrict__ sharp_idx,
                                                              int32_t* __restrict__ flat_idx) {
  const int bh = blockIdx.x;
  __shared__ int scratch[kSplitThreads / 64];
  unsigned long long key[kSplitIPT];
  bool valid[kSplitIPT], sel[kSplitIPT];
#pragma unroll
  for (int u = 0; u < kSplitIPT; ++u) {
    const int i = threadIdx.x * kSplitIPT + u;
    valid[u] = i < s.N;
    key[u] = valid[u] ? order_key(sharp[(size_t)bh * s.N + i]) : 0;
  }
  block_topk<kSplitThreads, kSplitIPT>(key, valid, s.n_sharp, sel, scratch);
  auto ident = [](int i) { return i; };
  if (s.n_sharp > 0)
    block_compact<kSplitThreads, kSplitIPT>(sel, valid, true, sharp_idx + (size_t)bh * s.n_sharp,
                                            ident, scratch);
  if (s.n_flat > 0)
    block_compact<kSplitThreads, kSplitIPT>(sel, valid, false, flat_idx + (size_t)bh * s.n_flat,
                                            ident, scratch);
}

// --------------------------------------------- step (5) exact set per block
// One wave selects the k largest of the n keys it holds (lower index wins
// ties). Lane l holds items p = l + 64u, so index order is u-major,
// lane-minor. Counting uses ballots (scalar popcounts), no workgroup barrier.
template <int IPL>
__device__ inline void wave_topk(const unsigned long long (&key)[IPL], int n, int k,
                                 bool (&sel)[IPL]) {
  const int lane = threadIdx.x & 63;
  const unsigned long long below = (1ull << lane) - 1ull;
  unsigned long long T = 0;
  for (int bit = 63; bit >= 0; --bit) {
    const unsigned long long trial = T | (1ull << bit);
    int c = 0;
#pragma unroll
    for (int u = 0; u < IPL; ++u) c += __popcll(__ballot(lane + 64 * u < n && key[u] >= trial));
    if (c >= k) {
      T = trial;
      if (c == k) break;   // exactly k at or above T: the top k (see block_topk)
    }
  }
  int gt = 0;
#pragma unroll
  for (int u = 0; u < IPL; ++u) gt += __popcll(__ballot(lane + 64 * u < n && key[u] > T));
  const int need = k - gt;
  int before = 0;
#pragma unroll
  for (int u = 0; u < IPL; ++u) {
    const bool valid = lane + 64 * u < n;
    const bool tie = valid && key[u] == T;
    const unsigned long long m = __ballot(tie);
    const int rank = before + __popcll(m & below);
    sel[u] = (valid && key[u] > T) || (tie && rank < need);
    before += __popcll(m);
  }
}

constexpr int kFlatTopkWaves = 4;

template <int IPL>
__global__ __launch_bounds__(64 * kFlatTopkWaves) void flat_topk_kernel(IsaShape s, const double* __restrict__ srows,
                                                                        const int32_t* __restrict__ ctx_idx,
                                                                        const int32_t* __restrict__ flat_idx,
                                                                        int32_t* __restrict__ exact) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * kFlatTopkWaves + (threadIdx.x >> 6), bh = blockIdx.y;
  if (r >= s.n_flat) return;   // whole wave; no workgroup barrier below
  const int i = flat_idx[(size_t)bh * s.n_flat + r];
  const double* row = srows + ((size_t)bh * s.N + i) * s.N_kv;
  unsigned long long key[IPL];
  bool sel[IPL];
#pragma unroll
  for (int u = 0; u < IPL; ++u) {
    const int p = lane + 64 * u;
    key[u] = p < s.N_kv ? order_key(row[p]) : 0ull;
  }
  wave_topk<IPL>(key, s.N_kv, s.k_ns, sel);
  const int32_t* ctx_row = ctx_idx + (size_t)bh * s.k_ctx;
  int32_t* out = exact + ((size_t)bh * s.n_flat + r) * s.k_ns;
  const unsigned long long below = (1ull << lane) - 1ull;
  int base = 0;
#pragma unroll
  for (int u = 0; u < IPL; ++u) {
    const unsigned long long m = __ballot(sel[u]);
    if (sel[u]) out[base + __popcll(m & below)] = kept_block_id(s, ctx_row, lane + 64 * u);
    base += __popcll(m);
  }
}

// ------------------------------------------------ step (6) coarse residual
// O_coarse = softmax(S[:, J]) Vc[J] over the query blocks of a head is an
// (N x N_kv) by (N_kv x D) product whose right operand every block shares.
// One workgroup takes kResRows consecutive query blocks: it forms each row's
// max and normaliser z_i in fp64 (one wave per row), then streams J in tiles
// of kResTile pooled keys (the Vc rows staged in LDS, the weights
// exp(S - max) formed once per tile) and accumulates in fp32; finally
// gamma * O_coarse_i / z_i is added to every token row of block i (bf16
// read-modify-write in 16-byte vectors).
constexpr int kResThreads = 256;
constexpr int kResRows = 16;
constexpr int kResTile = 64;

__device__ inline float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ inline uint16_t f32_to_bf16_rne_sel(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <int D>
__global__ __launch_bounds__(kResThreads) void coarse_residual_kernel(IsaShape s, const double* __restrict__ srows,
                                                                      const uint16_t* __restrict__ vcb,
                                                                      const int32_t* __restrict__ ctx_idx,
                                                                      uint16_t* __restrict__ O) {
  constexpr int CPR = D / 8;                        // 16-byte chunks per row
  constexpr int RPT = kResRows * D / kResThreads;   // rows accumulated per thread
  const int i0 = blockIdx.x * kResRows, bh = blockIdx.y;
  const int nr = min(kResRows, s.N - i0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ double rmax[kResRows], rz[kResRows];
  __shared__ float w[kResRows][kResTile];
  __shared__ __attribute__((aligned(16))) uint16_t vt[kResTile][D];
  __shared__ float oc[kResRows][D];
  const double* rows = srows + ((size_t)bh * s.N + i0) * s.N_kv;
  const int32_t* ctx_row = ctx_idx + (size_t)bh * s.k_ctx;
  const uint16_t* vh = vcb + (size_t)bh * s.N * D;

  for (int r = wave; r < nr; r += kResThreads / 64) {
    const double* row = rows + (size_t)r * s.N_kv;
    double mx = -INFINITY;
    for (int p = lane; p < s.N_kv; p += 64) mx = fmax(mx, row[p]);
    mx = wave_max_f64(mx);
    double z = 0.0;
    for (int p = lane; p < s.N_kv; p += 64) z += exp(row[p] - mx);
    z = wave_sum_f64(z);
    if (lane == 0) {
      rmax[r] = mx;
      rz[r] = z;
    }
  }
  const int d = tid % D, rg = tid / D;   // column d of rows rg*RPT .. rg*RPT+RPT-1
  float acc[RPT];
#pragma unroll
  for (int u = 0; u < RPT; ++u) acc[u] = 0.0f;
  __syncthreads();
  for (int p0 = 0; p0 < s.N_kv; p0 += kResTile) {
    // all of a thread's 16-byte loads are issued before its LDS stores
    constexpr int VC = kResTile * CPR / kResThreads;
    uint4 vr[VC];
#pragma unroll
    for (int x = 0; x < VC; ++x) {
      const int c = tid + x * kResThreads, pp = c / CPR, k = c % CPR, p = p0 + pp;
      vr[x] = make_uint4(0, 0, 0, 0);
      if (p < s.N_kv) {
        const int j = kept_block_id(s, ctx_row, p);
        if (j >= 0 && j < s.N) vr[x] = *reinterpret_cast<const uint4*>(vh + (size_t)j * D + 8 * k);
      }
    }
#pragma unroll
    for (int x = 0; x < VC; ++x) {
      const int c = tid + x * kResThreads;
      *reinterpret_cast<uint4*>(&vt[c / CPR][8 * (c % CPR)]) = vr[x];
    }
    for (int c = tid; c < kResRows * kResTile; c += kResThreads) {
      const int r = c / kResTile, pp = c % kResTile, p = p0 + pp;
      w[r][pp] = (r < nr && p < s.N_kv) ? (float)exp(rows[(size_t)r * s.N_kv + p] - rmax[r]) : 0.0f;
    }
    __syncthreads();
#pragma unroll 8
    for (int pp = 0; pp < kResTile; ++pp) {
      const float v = bf16_to_f32(vt[pp][d]);
#pragma unroll
      for (int u = 0; u < RPT; ++u) acc[u] += w[rg * RPT + u][pp] * v;
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    const int r = rg * RPT + u;
    oc[r][d] = r < nr ? s.gamma * (float)((double)acc[u] / rz[r]) : 0.0f;
  }
  __syncthreads();
  for (int r = 0; r < nr; ++r) {
    int start, n;
    isa_block_range(s, i0 + r, start, n);
    uint16_t* base = O + ((size_t)bh * s.L + start) * D;
    for (int c = tid; c < n * CPR; c += kResThreads) {
      const int k = c % CPR;
      const uint4 x = *reinterpret_cast<const uint4*>(base + (size_t)c * 8);
      uint32_t wd[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float lo = bf16_to_f32((uint16_t)(wd[q] & 0xffffu)) + oc[r][8 * k + 2 * q];
        const float hi = bf16_to_f32((uint16_t)(wd[q] >> 16)) + oc[r][8 * k + 2 * q + 1];
        wd[q] = (uint32_t)f32_to_bf16_rne_sel(lo) | ((uint32_t)f32_to_bf16_rne_sel(hi) << 16);
      }
      *reinterpret_cast<uint4*>(base + (size_t)c * 8) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    }
  }
}

}  // namespace

hipError_t isa_launch_coarse_residual(const IsaShape& s, const double* srows,
                                      const uint16_t* vc_bf16, const int32_t* ctx_idx,
                                      uint16_t* O, hipStream_t st) {
  if (s.gamma == 0.0f) return hipSuccess;
  dim3 grid((s.N + kResRows - 1) / kResRows, s.B * s.H);
  if (s.D == 128)
    coarse_residual_kernel<128><<<grid, kResThreads, 0, st>>>(s, srows, vc_bf16, ctx_idx, O);
  else
    coarse_residual_kernel<64><<<grid, kResThreads, 0, st>>>(s, srows, vc_bf16, ctx_idx, O);
  return hipGetLastError();
}

hipError_t isa_launch_ctx_topk(const IsaShape& s, const double* qc, const double* kc,
                               int32_t* ctx_idx, double* ctx_score, hipStream_t st) {
  if (s.N_ctx == 0) return hipSuccess;
  ctx_topk_kernel<<<s.B * s.H, kCtxThreads, 0, st>>>(s, qc, kc, ctx_idx, ctx_score);
  return hipGetLastError();
}

hipError_t isa_launch_coarse_rows(const IsaShape& s, const double* qc, const double* kc,
                                  const int32_t* ctx_idx, double* srows, hipStream_t st) {
  dim3 grid((s.N + kCoarseRows - 1) / kCoarseRows, (s.N_kv + kCoarseCols - 1) / kCoarseCols,
            s.B * s.H);
  coarse_rows_kernel<<<grid, 256, 0, st>>>(s, qc, kc, ctx_idx, srows);
  return hipGetLastError();
}

hipError_t isa_launch_sharpness(const IsaShape& s, const double* srows, double* sharp,
                                hipStream_t st) {
  dim3 grid((s.N + 3) / 4, s.B * s.H);
  sharpness_kernel<<<grid, 256, 0, st>>>(s, srows, sharp);
  return hipGetLastError();
}

hipError_t isa_launch_split(const IsaShape& s, const double* sharp, int32_t* sharp_idx,
                            int32_t* flat_idx, hipStream_t st) {
  split_kernel<<<s.B * s.H, kSplitThreads, 0, st>>>(s, sharp, sharp_idx, flat_idx);
  return hipGetLastError();
}

hipError_t isa_launch_flat_topk(const IsaShape& s, const double* srows, const int32_t* ctx_idx,
                                const int32_t* flat_idx, int32_t* flat_exact_idx,
                                hipStream_t st) {
  if (s.n_flat == 0 || s.k_ns == 0) return hipSuccess;
  dim3 grid((s.n_flat + kFlatTopkWaves - 1) / kFlatTopkWaves, s.B * s.H);
  const int ipl = (s.N_kv + 63) / 64;
  const int nt = 64 * kFlatTopkWaves;
  if (ipl <= 4)
    flat_topk_kernel<4><<<grid, nt, 0, st>>>(s, srows, ctx_idx, flat_idx, flat_exact_idx);
  else if (ipl <= 8)
    flat_topk_kernel<8><<<grid, nt, 0, st>>>(s, srows, ctx_idx, flat_idx, flat_exact_idx);
  else if (ipl <= 16)
    flat_topk_kernel<16><<<grid, nt, 0, st>>>(s, srows, ctx_idx, flat_idx, flat_exact_idx);
  else if (ipl <= 32)
    flat_topk_kernel<32><<<grid, nt, 0, st>>>(s, srows, ctx_idx, flat_idx, flat_exact_idx);
  else
    flat_topk_kernel<64><<<grid, nt, 0, st>>>(s, srows, ctx_idx, flat_idx, flat_exact_idx);
  return hipGetLastError();
}
