// Step (1) of In-context Sparse Attention: mean pooling of Q, K, V per block
// (paper.rainbus.top summary of arXiv 2605.04569, "Method steps", step (1);
// the pooled means Qc, Kc, Vc feed the coarse scores and the Taylor term).
//
// One workgroup per (block, batch*head). The kernel is HBM-bound: it streams
// each token row of Q, K and V once with 16-byte loads (8 bf16 per lane),
// accumulates in fp64 (sums of bf16 values stay exact in fp64), reduces the
// row lanes with cross-lane swaps and a small LDS stage, and divides by the
// block's valid-token count n_j. Outputs: Qc and Kc in fp64 for the
// selection path, Kc and Vc rounded to bf16 for the Taylor contraction.
#include <cmath>

#include "isa_internal.h"

namespace {

constexpr int kPoolThreads = 256;

__device__ inline void bf16x8_to_f64_add(const uint4& w, double* acc) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] += (double)__uint_as_float(u[i] << 16);
    acc[2 * i + 1] += (double)__uint_as_float(u[i] & 0xffff0000u);
  }
}

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Sum across the lanes of a wave that share the same column chunk: lanes
// l, l ^ TPR, l ^ 2*TPR, ... (TPR = threads per row, a power of two).
template <int TPR>
__device__ inline double wave_sum_rows(double x) {
#pragma unroll
  for (int off = TPR; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
  return x;
}

template <int D>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(IsaShape s, const uint16_t* __restrict__ Q,
                                                            const uint16_t* __restrict__ K,
                                                            const uint16_t* __restrict__ V,
                                                            double* __restrict__ qc,
                                                            double* __restrict__ kc,
                                                            uint16_t* __restrict__ kcb,
                                                            uint16_t* __restrict__ vcb) {
  constexpr int TPR = D / 8;                 // lanes per token row (16 B each)
  constexpr int RPI = kPoolThreads / TPR;    // rows handled per iteration
  constexpr int WAVES = kPoolThreads / 64;
  const int j = blockIdx.x;
  const int bh = blockIdx.y;
  int start, n;
  isa_block_range(s, j, start, n);
  const int c = threadIdx.x % TPR;
  const int r0 = threadIdx.x / TPR;
  double aq[8], ak[8], av[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) aq[i] = ak[i] = av[i] = 0.0;
  const size_t base = ((size_t)bh * s.L + start) * D + (size_t)c * 8;
  for (int r = r0; r < n; r += RPI) {
    const size_t off = base + (size_t)r * D;
    uint4 wq = *reinterpret_cast<const uint4*>(Q + off);
    uint4 wk = *reinterpret_cast<const uint4*>(K + off);
    uint4 wv = *reinterpret_cast<const uint4*>(V + off);
    bf16x8_to_f64_add(wq, aq);
    bf16x8_to_f64_add(wk, ak);
    bf16x8_to_f64_add(wv, av);
  }
  __shared__ double red[3][WAVES][D];
  const int wave = threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    double q = wave_sum_rows<TPR>(aq[i]);
    double k = wave_sum_rows<TPR>(ak[i]);
    double v = wave_sum_rows<TPR>(av[i]);
    if (lane < TPR) {
      red[0][wave][c * 8 + i] = q;
      red[1][wave][c * 8 + i] = k;
      red[2][wave][c * 8 + i] = v;
    }
  }
  __syncthreads();
  const double inv_n = (double)n;
  const size_t obase = ((size_t)bh * s.N + j) * D;
  for (int t = threadIdx.x; t < 3 * D; t += kPoolThreads) {
    const int which = t / D, d = t % D;
    double sum = 0.0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) sum += red[which][w][d];
    const double mean = sum / inv_n;
    if (which == 0) {
      qc[obase + d] = mean;
    } else if (which == 1) {
      kc[obase + d] = mean;
      if (kcb) kcb[obase + d] = f32_to_bf16_rne((float)mean);
    } else {
      if (vcb) vcb[obase + d] = f32_to_bf16_rne((float)mean);
    }
  }
}

// ------------------------------------------------- decoupled RoPE + step (1)
// Per-pair frequencies base^(-2i/D), passed by value (at most 64 pairs).
struct RopeFreq {
  double inv[64];
};

// cos/sin of pos * inv[i] in fp64, rounded to fp32 (one entry per position
// and pair; positions restart at 0 in the context segment, so the table
// covers max(L_src, L_ctx) positions). The frequencies come from the host's
// libm pow: an error of one ulp there is multiplied by the position, so they
// are not recomputed on the device.
__global__ void rope_table_kernel(int P, int half, RopeFreq f, float2* __restrict__ tab) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)P * half) return;
  const int pos = (int)(idx / half), i = (int)(idx % half);
  const double ang = (double)pos * f.inv[i];
  tab[idx] = make_float2((float)cos(ang), (float)sin(ang));
}

// Rotates one 16-byte chunk (4 pairs) in fp32: x' = x c - y s,
// y' = x s + y c, each product and each sum rounded on its own (contraction
// into fused multiply-adds is switched off, since it changes the result
// where the two products nearly cancel), then bf16 round-to-nearest-even.
__device__ inline uint4 rope_chunk(const uint4& w, const float2* __restrict__ cs) {
#pragma clang fp contract(off)   // the products must not fuse into the sums
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
  uint32_t o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float x = __uint_as_float(u[k] << 16), y = __uint_as_float(u[k] & 0xffff0000u);
    const float2 t = cs[k];
    const float xr = x * t.x - y * t.y;
    const float yr = x * t.y + y * t.x;
    o[k] = (uint32_t)f32_to_bf16_rne(xr) | ((uint32_t)f32_to_bf16_rne(yr) << 16);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

template <int D>
__global__ __launch_bounds__(kPoolThreads) void rope_pool_kernel(IsaShape s, const uint16_t* __restrict__ Q,
                                                                 const uint16_t* __restrict__ K,
                                                                 const uint16_t* __restrict__ V,
                                                                 const float2* __restrict__ tab,
                                                                 uint16_t* __restrict__ Qr,
                                                                 uint16_t* __restrict__ Kr,
                                                                 double* __restrict__ qc,
                                                                 double* __restrict__ kc,
                                                                 uint16_t* __restrict__ kcb,
                                                                 uint16_t* __restrict__ vcb) {
  constexpr int TPR = D / 8;
  constexpr int RPI = kPoolThreads / TPR;
  constexpr int WAVES = kPoolThreads / 64;
  // heads vary fastest so that consecutive workgroups reuse one table slice
  const int bh = blockIdx.x;
  const int j = blockIdx.y;
  int start, n;
  isa_block_range(s, j, start, n);
  const int seg0 = j < s.N_src ? 0 : s.L_src;   // first token of the segment
  const int c = threadIdx.x % TPR;
  const int r0 = threadIdx.x / TPR;
  double aq[8], ak[8], av[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) aq[i] = ak[i] = av[i] = 0.0;
  const size_t base = ((size_t)bh * s.L + start) * D + (size_t)c * 8;
  for (int r = r0; r < n; r += RPI) {
    const size_t off = base + (size_t)r * D;
    const float2* cs = tab + (size_t)(start + r - seg0) * (D / 2) + c * 4;
    const uint4 wq = rope_chunk(*reinterpret_cast<const uint4*>(Q + off), cs);
    const uint4 wk = rope_chunk(*reinterpret_cast<const uint4*>(K + off), cs);
    const uint4 wv = *reinterpret_cast<const uint4*>(V + off);
    *reinterpret_cast<uint4*>(Qr + off) = wq;
    *reinterpret_cast<uint4*>(Kr + off) = wk;
    bf16x8_to_f64_add(wq, aq);
    bf16x8_to_f64_add(wk, ak);
    bf16x8_to_f64_add(wv, av);
  }
  __shared__ double red[3][WAVES][D];
  const int wave = threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    double q = wave_sum_rows<TPR>(aq[i]);
    double k = wave_sum_rows<TPR>(ak[i]);
    double v = wave_sum_rows<TPR>(av[i]);
    if (lane < TPR) {
      red[0][wave][c * 8 + i] = q;
      red[1][wave][c * 8 + i] = k;
      red[2][wave][c * 8 + i] = v;
    }
  }
  __syncthreads();
  const size_t obase = ((size_t)bh * s.N + j) * D;
  for (int t = threadIdx.x; t < 3 * D; t += kPoolThreads) {
    const int which = t / D, d = t % D;
    double sum = 0.0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) sum += red[which][w][d];
    const double mean = sum / (double)n;
    if (which == 0) {
      qc[obase + d] = mean;
    } else if (which == 1) {
      kc[obase + d] = mean;
      if (kcb) kcb[obase + d] = f32_to_bf16_rne((float)mean);
    } else {
      if (vcb) vcb[obase + d] = f32_to_bf16_rne((float)mean);
    }
  }
}

}  // namespace

hipError_t isa_launch_rope_table(const IsaShape& s, float2* table, hipStream_t st) {
  const int P = s.L_src > s.L_ctx ? s.L_src : s.L_ctx;
  const int half = s.D / 2;
  RopeFreq f;
  for (int i = 0; i < 64; ++i) f.inv[i] = i < half ? std::pow(s.rope_base, -(2.0 * i) / (double)s.D) : 0.0;
  const size_t n = (size_t)P * half;
  rope_table_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(P, half, f, table);
  return hipGetLastError();
}

hipError_t isa_launch_rope_pool(const IsaShape& s, const uint16_t* Q, const uint16_t* K,
                                const uint16_t* V, const float2* table, uint16_t* Qr,
                                uint16_t* Kr, double* qc, double* kc, uint16_t* kc_bf16,
                                uint16_t* vc_bf16, hipStream_t st) {
  dim3 grid(s.B * s.H, s.N);
  if (s.D == 128)
    rope_pool_kernel<128><<<grid, kPoolThreads, 0, st>>>(s, Q, K, V, table, Qr, Kr, qc, kc, kc_bf16, vc_bf16);
  else
    rope_pool_kernel<64><<<grid, kPoolThreads, 0, st>>>(s, Q, K, V, table, Qr, Kr, qc, kc, kc_bf16, vc_bf16);
  return hipGetLastError();
}

hipError_t isa_launch_pool(const IsaShape& s, const uint16_t* Q, const uint16_t* K,
                           const uint16_t* V, double* qc, double* kc, uint16_t* kc_bf16,
                           uint16_t* vc_bf16, hipStream_t st) {
  dim3 grid(s.N, s.B * s.H);
  if (s.D == 128)
    pool_kernel<128><<<grid, kPoolThreads, 0, st>>>(s, Q, K, V, qc, kc, kc_bf16, vc_bf16);
  else
    pool_kernel<64><<<grid, kPoolThreads, 0, st>>>(s, Q, K, V, qc, kc, kc_bf16, vc_bf16);
  return hipGetLastError();
}
