// Selection path of In-context Sparse Attention, all scores in fp64.
//
// Steps, as given in the paper.rainbus.top summary of arXiv 2605.04569,
// section "Method steps":
//   step (2): context importance = coarse scores of the source query blocks
//             summed per context key block; keep the top alpha_s fraction;
//   step (1)+(3): coarse scores S[i, j] = Qc_i . Kc_j / sqrt(D); sharpness
//             M_i = variance of the softmax of S[i, :] restricted to the
//             source key blocks; the least sharp alpha_f fraction of query
//             blocks is "flat";
//   step (5): per flat block, the exact set E_i = top alpha_ns fraction of J
//             by coarse score.
// The coarse scores are formed where they are used, on the fp64 matrix cores
// (v_mfma_f64_16x16x4f64), and never stored: the sharpness kernel folds each
// 16 x 16 tile into per-row online softmax statistics, the exact-set kernel
// keeps only its own flat blocks' rows (in LDS) for their top-k. Only the
// gamma residual (step (6)) materialises the rows S[i, J] it needs.
// Every top-k prefers the lower index among equal scores, and every output
// list is ascending. Selection uses an exact radix bisection on the ordered
// bit pattern of the fp64 scores (no floating-point comparison tolerance),
// then resolves ties at the threshold by index order with a block-wide scan.
#include <initializer_list>

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

// Workgroups are dispatched round-robin over the 8 XCDs, each with its own
// L2. Work item `id` of `total` (in dispatch order) is renamed so that each
// XCD receives a contiguous run of items, i.e. mostly one (batch, head),
// whose pooled keys then stay in that XCD's L2.
__device__ inline int xcd_order(int id, int total) {
  if ((total & 7) != 0) return id;
  return (id & 7) * (total >> 3) + (id >> 3);
}

// ------------------------------------------- coarse scores on matrix cores
// v_mfma_f64_16x16x4f64: lane l supplies A[m][k] and B[k][n] with m = n =
// l % 16, k = l / 16, and receives C[l / 16 + 4 i][l % 16], i = 0..3. Step
// kk = 2x + e of a D-long dot product pairs dimension 8x + 2k + e of the A
// row and of the B column: the four lanes of one row read 64 contiguous
// bytes per 16-byte load, so a load instruction touches 16 rows' segments
// rather than 64 scattered pieces.
typedef double double4_t __attribute__((ext_vector_type(4)));

// Lane l's D/4 dimensions of one row (pairs 8x + 2k, 8x + 2k + 1). Callers
// point past-the-end lanes at a readable row (row 0 of the head) and discard
// the products those lanes feed, so no value needs zeroing.
template <int D>
__device__ inline void load_frag(const double* __restrict__ row, int k, double (&f)[D / 4]) {
#pragma unroll
  for (int x = 0; x < D / 8; ++x) {
    const double2 v = *reinterpret_cast<const double2*>(row + 8 * x + 2 * k);
    f[2 * x] = v.x;
    f[2 * x + 1] = v.y;
  }
}

// Raw dot products of the 16 A rows with the 16 B rows held by the wave:
// two independent accumulation chains (even and odd steps kk), so each
// product's accumulator was written two products earlier, added at the end.
template <int D>
__device__ inline double4_t coarse_mma(const double (&a)[D / 4], const double (&b)[D / 4]) {
  double4_t c0 = {0.0, 0.0, 0.0, 0.0}, c1 = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int kk = 0; kk < D / 4; kk += 2) {
    c0 = __builtin_amdgcn_mfma_f64_16x16x4f64(a[kk], b[kk], c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f64_16x16x4f64(a[kk + 1], b[kk + 1], c1, 0, 0, 0);
  }
  return c0 + c1;
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

// ------------------------------------ coarse rows of the gamma residual
// S[i, p] = Qc_i . Kc_{J[p]} / sqrt(D) in fp64 for every query block and
// kept block (the residual's pooled attention and its backward read whole
// rows); a 64 x 64 tile per workgroup, each thread accumulating a 4 x 4
// block from LDS-staged slices.
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
// M_i = (1/n) sum_j (p_ij - 1/n)^2 with p_i = softmax(S[i, 0..n)), n = N_src,
// equal to (sum_j p_ij^2 - 1/n) / n. Each wave takes 16 query blocks and
// walks the source key blocks 16 at a time; every lane keeps, for each of its
// four rows, the online statistics of its columns: the running maximum m,
// z = sum exp(S - m) and w = sum exp(2 (S - m)), so sum p^2 = w / z^2. The
// 16 lanes of a row then merge their statistics in a fixed butterfly order
// (each merge is symmetric, so every lane ends with the same bits).
constexpr int kSharpWaves = 4;

__device__ inline void stats_add(double v, double& m, double& z, double& w) {
  const double d = v - m;                 // +inf while m = -inf
  const double e = exp(-fabs(d));         // exp(m - v) when v is the new maximum
  const bool up = d > 0.0;
  z = up ? z * e + 1.0 : z + e;
  w = up ? w * (e * e) + 1.0 : w + e * e;
  m = up ? v : m;
}

__device__ inline void stats_merge(double& m, double& z, double& w, double m2, double z2, double w2) {
  const double mm = fmax(m, m2);
  if (mm == -INFINITY) return;            // neither side has seen a column
  const double e1 = exp(m - mm), e2 = exp(m2 - mm);
  z = z * e1 + z2 * e2;
  w = w * (e1 * e1) + w2 * (e2 * e2);
  m = mm;
}

// The source key blocks are streamed through LDS 16 rows (one tile of
// columns) at a time, loaded once per workgroup with contiguous 16-byte
// loads and shared by its waves; two buffers let the next tile's loads run
// while the current tile's products do. A staged row is D + 2 doubles, so the
// 16 lanes of one k read 16 different bank groups.
template <int D>
__global__ __launch_bounds__(64 * kSharpWaves) void sharpness_kernel(IsaShape s, const double* __restrict__ qc,
                                                                     const double* __restrict__ kc,
                                                                     double* __restrict__ sharp) {
  constexpr int NT = 64 * kSharpWaves;
  constexpr int ST2 = (D + 2) / 2;            // double2 per staged row
  constexpr int CPT = 16 * (D / 2) / NT;      // double2 each thread stages per tile
  static_assert(CPT * NT == 16 * (D / 2), "tile must split evenly over the threads");
  __shared__ double2 tile[2][16 * ST2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int id = xcd_order(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x * gridDim.y);
  const int bh = id / gridDim.x;
  const int r0 = ((id % gridDim.x) * kSharpWaves + wave) * 16;   // may be >= N: computes, never writes
  const int m16 = lane & 15, k = lane >> 4;
  const double* qh = qc + (size_t)bh * s.N * D;
  const double* kh = kc + (size_t)bh * s.N * D;   // source key blocks are rows 0..N_src-1
  double a[D / 4];   // rows past N read row 0; their statistics are never written
  load_frag<D>(qh + (size_t)(r0 + m16 < s.N ? r0 + m16 : 0) * D, k, a);
  const double rsq = 1.0 / sqrt((double)D);   // S = dot / sqrt(D) as a product (one rounding)
  double mx[4], z[4], w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    mx[i] = -INFINITY;
    z[i] = 0.0;
    w[i] = 0.0;
  }
  // thread tid stages double2 c2 of tile row `row`, for q = tid + NT u
  const int ntile = (s.N_src + 15) / 16;
  double2 g[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) {   // columns past N_src stage row 0; their products are skipped
    const int q = tid + NT * u, row = q / (D / 2), c2 = q % (D / 2);
    const int col = row < s.N_src ? row : 0;
    g[u] = reinterpret_cast<const double2*>(kh + (size_t)col * D)[c2];
  }
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int q = tid + NT * u, row = q / (D / 2), c2 = q % (D / 2);
    tile[0][row * ST2 + c2] = g[u];
  }
  __syncthreads();
  for (int t = 0; t < ntile; ++t) {
    // the next tile (the last tile again on the last pass: a harmless
    // re-read into the buffer nobody reads any more)
    const int cn = 16 * (t + 1 < ntile ? t + 1 : t);
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int q = tid + NT * u, row = q / (D / 2), c2 = q % (D / 2);
      const int col = cn + row < s.N_src ? cn + row : 0;
      g[u] = reinterpret_cast<const double2*>(kh + (size_t)col * D)[c2];
    }
    double b[D / 4];
    const double2* rp = &tile[t & 1][m16 * ST2];
#pragma unroll
    for (int x = 0; x < D / 8; ++x) {
      const double2 v = rp[4 * x + k];
      b[2 * x] = v.x;
      b[2 * x + 1] = v.y;
    }
    const double4_t acc = coarse_mma<D>(a, b);
    if (16 * t + m16 < s.N_src) {
#pragma unroll
      for (int i = 0; i < 4; ++i) stats_add(acc[i] * rsq, mx[i], z[i], w[i]);
    }
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int q = tid + NT * u, row = q / (D / 2), c2 = q % (D / 2);
      tile[(t + 1) & 1][row * ST2 + c2] = g[u];
    }
    __syncthreads();
  }
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double m2 = __shfl_xor(mx[i], off, 64), z2 = __shfl_xor(z[i], off, 64),
                   w2 = __shfl_xor(w[i], off, 64);
      stats_merge(mx[i], z[i], w[i], m2, z2, w2);
    }
  }
  if (m16 == 0) {
    const double n = (double)s.N_src;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = r0 + k + 4 * i;
      if (row < s.N) sharp[(size_t)bh * s.N + row] = (w[i] / (z[i] * z[i]) - 1.0 / n) / n;
    }
  }
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
// One wave selects the k largest keys it holds (lower index wins ties).
// Lane l holds items p = l + 64u, so index order is u-major, lane-minor;
// padding items hold key 0, below every key of a real score (order_key of a
// non-NaN fp64 value is nonzero), so they are never counted (k >= 1).
// Counting uses ballots (scalar popcounts), no workgroup barrier. Returns the
// k-th largest key T; the selected items are every key > T and the first
// `need` = k - #{key > T} keys equal to T in index order.
template <int IPL>
__device__ inline unsigned long long wave_topk_threshold(const unsigned long long (&key)[IPL], int k,
                                                         int& need) {
  unsigned long long T = 0;
  for (int bit = 63; bit >= 0; --bit) {
    const unsigned long long trial = T | (1ull << bit);
    int c = 0;
#pragma unroll
    for (int u = 0; u < IPL; ++u) c += __popcll(__ballot(key[u] >= trial));
    if (c >= k) {
      T = trial;
      if (c == k) break;   // exactly k at or above T: the top k (see block_topk)
    }
  }
  int gt = 0;
#pragma unroll
  for (int u = 0; u < IPL; ++u) gt += __popcll(__ballot(key[u] > T));
  need = k - gt;
  return T;
}

// Work item g = one group of 16 consecutive flat blocks of one (batch, head)
// (one 16-row matrix-core tile). Phase 1: the matrix cores form the raw dot
// products Qc_i . Kc_j (S[i, J] up to the positive factor 1/sqrt(D), which
// does not change the order) of those rows, 16 positions of J per tile,
// tiles spread over the waves; the next tile's fragments load while the
// current tile's products run. The rows go to LDS when 16 rows of J fit
// (N_kv <= kFlatLdsCols), else to this workgroup's own slot of a global
// scratch buffer, and the grid is then persistent (kFlatSlots workgroups
// walking the groups), which bounds the scratch by the slot count, not by N.
// Phase 2: one wave per row reads its row back (lane l: positions l + 64 u)
// and selects the top k_ns.
// Each pass of the grid takes its groups in XCD-contiguous order.
constexpr int kFlatLdsWaves = 4;
constexpr int kFlatGlobalWaves = 8;
constexpr int kFlatLdsCols = 640;   // 16 rows x 640 fp64 = 80 KiB of LDS
constexpr int kFlatSlots = 256;

__host__ __device__ inline bool flat_rows_in_lds(int N_kv) { return N_kv <= kFlatLdsCols; }

// One group: flat blocks f0 .. f0 + 15 of (batch, head) bh; `srow` holds
// 16 x N_kv doubles. DB: double-buffered fragment loads (the LDS form, at
// most two waves per SIMD); the global form (twice the waves) single-buffers.
template <int D, int IPL, int NW, bool DB>
__device__ inline void flat_group(const IsaShape& s, const double* __restrict__ qc,
                                  const double* __restrict__ kc, const int32_t* __restrict__ ctx_idx,
                                  const int32_t* __restrict__ flat_idx, int32_t* __restrict__ exact,
                                  double* __restrict__ srow, int bh, int f0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m16 = lane & 15, k = lane >> 4;
  const int ntile = (s.N_kv + 15) / 16;
  const unsigned long long below = (1ull << lane) - 1ull;
  const int nr = min(16, s.n_flat - f0);
  const int32_t* frow = flat_idx + (size_t)bh * s.n_flat;
  const int32_t* ctx_row = ctx_idx + (size_t)bh * s.k_ctx;
  const double* qh = qc + (size_t)bh * s.N * D;
  const double* kh = kc + (size_t)bh * s.N * D;
  int qi = -1;
  if (m16 < nr) {
    const int i = frow[f0 + m16];
    qi = (i >= 0 && i < s.N) ? i : -1;
  }
  double a[D / 4];   // rows past the group's flat blocks read row 0; never stored
  load_frag<D>(qh + (size_t)(qi >= 0 ? qi : 0) * D, k, a);
  // lane's position p = 16 t + m16 of J; positions past N_kv read row 0
  auto col_row = [&](int t) -> const double* {
    const int p = t * 16 + m16;
    const int j = (t < ntile && p < s.N_kv) ? kept_block_id(s, ctx_row, p) : -1;
    return kh + (size_t)((j >= 0 && j < s.N) ? j : 0) * D;
  };
  auto put = [&](int t, const double4_t& acc) {
    const int p = t * 16 + m16;
    if (p < s.N_kv) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = k + 4 * i;
        if (r < nr) srow[(size_t)r * s.N_kv + p] = acc[i];
      }
    }
  };
  if constexpr (DB) {
    double b0[D / 4], b1[D / 4];
    load_frag<D>(col_row(wave), k, b0);
    for (int t = wave; t < ntile; t += 2 * NW) {
      load_frag<D>(col_row(t + NW), k, b1);
      put(t, coarse_mma<D>(a, b0));
      load_frag<D>(col_row(t + 2 * NW), k, b0);
      if (t + NW < ntile) put(t + NW, coarse_mma<D>(a, b1));
    }
  } else {
    for (int t = wave; t < ntile; t += NW) {
      double b[D / 4];
      load_frag<D>(col_row(t), k, b);
      put(t, coarse_mma<D>(a, b));
    }
  }
  __syncthreads();
  for (int r = wave; r < nr; r += NW) {
    unsigned long long key[IPL];
#pragma unroll
    for (int u = 0; u < IPL; ++u) {
      const int p = lane + 64 * u;
      key[u] = p < s.N_kv ? order_key(srow[(size_t)r * s.N_kv + p]) : 0ull;
    }
    int need;
    const unsigned long long T = wave_topk_threshold<IPL>(key, s.k_ns, need);
    // selected positions of J in ascending order, then their global block
    // ids (the map from positions to ids is increasing)
    int32_t* out = exact + ((size_t)bh * s.n_flat + f0 + r) * s.k_ns;
    int base = 0, ties = 0;
#pragma unroll
    for (int u = 0; u < IPL; ++u) {
      const bool tie = key[u] == T;
      const unsigned long long tm = __ballot(tie);
      const bool sel = key[u] > T || (tie && ties + __popcll(tm & below) < need);
      ties += __popcll(tm);
      const unsigned long long msk = __ballot(sel);
      if (sel) out[base + __popcll(msk & below)] = lane + 64 * u;
      base += __popcll(msk);
    }
    for (int q = lane; q < s.k_ns; q += 64) out[q] = kept_block_id(s, ctx_row, out[q]);
  }
}

// LDS form: one group per workgroup.
template <int D, int IPL>
__global__ __launch_bounds__(64 * kFlatLdsWaves) void flat_topk_lds_kernel(
    IsaShape s, const double* __restrict__ qc, const double* __restrict__ kc,
    const int32_t* __restrict__ ctx_idx, const int32_t* __restrict__ flat_idx,
    int32_t* __restrict__ exact) {
  extern __shared__ double lds_rows[];   // [16][N_kv]
  const int gph = (s.n_flat + 15) / 16;   // groups per (batch, head)
  const int g = xcd_order(blockIdx.x, gridDim.x);
  flat_group<D, IPL, kFlatLdsWaves, true>(s, qc, kc, ctx_idx, flat_idx, exact, lds_rows, g / gph,
                                          (g % gph) * 16);
}

// Global form: persistent; workgroup x owns rows x of the scratch and walks
// the groups x, x + gridDim.x, ... (each pass of the grid remapped on its own).
template <int D, int IPL>
__global__ __launch_bounds__(64 * kFlatGlobalWaves) void flat_topk_global_kernel(
    IsaShape s, const double* __restrict__ qc, const double* __restrict__ kc,
    const int32_t* __restrict__ ctx_idx, const int32_t* __restrict__ flat_idx,
    int32_t* __restrict__ exact, double* __restrict__ scratch) {
  double* srow = scratch + (size_t)blockIdx.x * 16 * s.N_kv;
  const int gph = (s.n_flat + 15) / 16;
  const int total = gph * s.B * s.H;
  for (int pass0 = 0; pass0 + (int)blockIdx.x < total; pass0 += gridDim.x) {
    const int npass = min((int)gridDim.x, total - pass0);
    const int g = pass0 + xcd_order(blockIdx.x, npass);
    flat_group<D, IPL, kFlatGlobalWaves, false>(s, qc, kc, ctx_idx, flat_idx, exact, srow, g / gph,
                                                (g % gph) * 16);
    __syncthreads();   // the rows' storage is reused by the next group
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

hipError_t isa_launch_sharpness(const IsaShape& s, const double* qc, const double* kc, double* sharp,
                                hipStream_t st) {
  dim3 grid((s.N + 16 * kSharpWaves - 1) / (16 * kSharpWaves), s.B * s.H);
  if (s.D == 128)
    sharpness_kernel<128><<<grid, 64 * kSharpWaves, 0, st>>>(s, qc, kc, sharp);
  else
    sharpness_kernel<64><<<grid, 64 * kSharpWaves, 0, st>>>(s, qc, kc, sharp);
  return hipGetLastError();
}

hipError_t isa_launch_split(const IsaShape& s, const double* sharp, int32_t* sharp_idx,
                            int32_t* flat_idx, hipStream_t st) {
  split_kernel<<<s.B * s.H, kSplitThreads, 0, st>>>(s, sharp, sharp_idx, flat_idx);
  return hipGetLastError();
}

namespace {

// The LDS form of the exact-set kernel keeps 16 rows of S in dynamic LDS
// beyond the default limit: raised once per instantiation and device
// (host-side only).
template <int D, int IPL>
hipError_t prepare_topk() {
  static unsigned long long done = 0;
  return isa_ensure_dyn_lds(reinterpret_cast<const void*>(&flat_topk_lds_kernel<D, IPL>),
                            16 * kFlatLdsCols * (int)sizeof(double), &done);
}

template <int D, int IPL>
hipError_t launch_flat_topk(const IsaShape& s, const double* qc, const double* kc, const int32_t* ctx_idx,
                            const int32_t* flat_idx, int32_t* flat_exact_idx, double* scratch,
                            hipStream_t st) {
  const int total = (s.n_flat + 15) / 16 * s.B * s.H;
  if (flat_rows_in_lds(s.N_kv)) {
    const hipError_t e = prepare_topk<D, IPL>();
    if (e != hipSuccess) return e;
    const size_t lds = (size_t)16 * s.N_kv * sizeof(double);
    flat_topk_lds_kernel<D, IPL><<<total, 64 * kFlatLdsWaves, lds, st>>>(s, qc, kc, ctx_idx, flat_idx,
                                                                          flat_exact_idx);
  } else {
    const int grid = total < kFlatSlots ? total : kFlatSlots;
    flat_topk_global_kernel<D, IPL><<<grid, 64 * kFlatGlobalWaves, 0, st>>>(s, qc, kc, ctx_idx, flat_idx,
                                                                            flat_exact_idx, scratch);
  }
  return hipGetLastError();
}

template <int D>
hipError_t flat_topk_for_d(const IsaShape& s, const double* qc, const double* kc, const int32_t* ctx_idx,
                           const int32_t* flat_idx, int32_t* flat_exact_idx, double* scratch,
                           hipStream_t st) {
  const int ipl = (s.N_kv + 63) / 64;
  if (ipl <= 4) return launch_flat_topk<D, 4>(s, qc, kc, ctx_idx, flat_idx, flat_exact_idx, scratch, st);
  if (ipl <= 8) return launch_flat_topk<D, 8>(s, qc, kc, ctx_idx, flat_idx, flat_exact_idx, scratch, st);
  if (ipl <= 12) return launch_flat_topk<D, 12>(s, qc, kc, ctx_idx, flat_idx, flat_exact_idx, scratch, st);
  if (ipl <= 16) return launch_flat_topk<D, 16>(s, qc, kc, ctx_idx, flat_idx, flat_exact_idx, scratch, st);
  if (ipl <= 24) return launch_flat_topk<D, 24>(s, qc, kc, ctx_idx, flat_idx, flat_exact_idx, scratch, st);
  if (ipl <= 32) return launch_flat_topk<D, 32>(s, qc, kc, ctx_idx, flat_idx, flat_exact_idx, scratch, st);
  if (ipl <= 48) return launch_flat_topk<D, 48>(s, qc, kc, ctx_idx, flat_idx, flat_exact_idx, scratch, st);
  return launch_flat_topk<D, 64>(s, qc, kc, ctx_idx, flat_idx, flat_exact_idx, scratch, st);
}

}  // namespace

size_t isa_flat_topk_scratch_bytes(const IsaShape& s) {
  if (s.n_flat == 0 || s.k_ns == 0 || flat_rows_in_lds(s.N_kv)) return 0;
  return (size_t)kFlatSlots * 16 * s.N_kv * sizeof(double);
}

hipError_t isa_launch_flat_topk(const IsaShape& s, const double* qc, const double* kc, const int32_t* ctx_idx,
                                const int32_t* flat_idx, int32_t* flat_exact_idx, double* scratch,
                                hipStream_t st) {
  if (s.n_flat == 0 || s.k_ns == 0) return hipSuccess;
  return s.D == 128 ? flat_topk_for_d<128>(s, qc, kc, ctx_idx, flat_idx, flat_exact_idx, scratch, st)
                    : flat_topk_for_d<64>(s, qc, kc, ctx_idx, flat_idx, flat_exact_idx, scratch, st);
}

hipError_t isa_select_prepare_device() {
  hipError_t e = hipSuccess;
  // LDS rows are used only while 16 rows of J fit (at most 10 keys per lane)
  for (hipError_t x : {prepare_topk<128, 4>(), prepare_topk<128, 8>(), prepare_topk<128, 12>(),
                       prepare_topk<64, 4>(), prepare_topk<64, 8>(), prepare_topk<64, 12>()})
    if (e == hipSuccess) e = x;
  return e;
}
