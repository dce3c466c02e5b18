// Achievable-peak probes for the measurement harness (not part of the ISA
// operator): a kernel that keeps the bf16 matrix cores busy with
// independent v_mfma_f32_16x16x32_bf16 chains and touches no memory in its
// loop (its rate is the matrix-core throughput the chip sustains, which
// depends on the operand data through the clock), and a
// kernel that streams a large buffer from HBM with 16-byte loads (the read
// bandwidth it sustains), and a kernel that reads LDS tiles with the access
// patterns of the attention kernels' operand reads (the LDS read rate).
#include <hip/hip_runtime.h>
#include <stdint.h>

#define PROBE_API extern "C" __attribute__((visibility("default")))

namespace {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(16)));
typedef float float4_t __attribute__((__vector_size__(16)));
typedef short short4_t __attribute__((__vector_size__(8)));

constexpr int kChains = 8;   // independent accumulators per wave (hide the MFMA latency)
constexpr int kMfmaPerIter = 64;   // kChains chains x 8 operand pairs

__device__ inline uint32_t mix32(uint32_t x) {
  x ^= x >> 16; x *= 0x7feb352dU; x ^= x >> 15; x *= 0x846ca68bU; x ^= x >> 16;
  return x;
}

// The matrix cores' power, and with it the clock the chip holds, depends on
// the operand bits. mode 0: every product takes the same two operands made of
// a few small values (little bit activity); mode 1: each wave holds eight A
// and eight B operands of uniform random bf16 values in (-1, 1) and each of
// the 64 products of an iteration takes a different (A, B) pair, as the
// attention kernels' products do. When `clk` is not null, thread 0 of every
// workgroup stores the shader-clock and constant-rate (wall clock) ticks that
// elapsed over the workgroup (two 64-bit words).
__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, int mode, float* out,
                                                         unsigned long long* clk) {
  const unsigned long long c0 = __builtin_amdgcn_s_memtime(), w0 = __builtin_amdgcn_s_memrealtime();
  const int t = threadIdx.x;
  const uint32_t gt = (uint32_t)blockIdx.x * 256u + (uint32_t)t;
  bf16x8_t a[8], b[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float va, vb;
      if (mode == 0) {
        va = 0.001f * (float)((t + i) & 7);
        vb = 0.002f * (float)((t * 3 + i) & 7);
      } else {
        va = (float)(mix32(gt * 131u + k * 17u + i) >> 8) * (2.0f / 16777216.0f) - 1.0f;
        vb = (float)(mix32(gt * 977u + k * 29u + i + 7777u) >> 8) * (2.0f / 16777216.0f) - 1.0f;
      }
      a[k][i] = (__bf16)va;
      b[k][i] = (__bf16)vb;
    }
  float4_t c[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k) c[k] = float4_t{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int k = 0; k < kChains; ++k)
        // accumulate in place: the builtin form made the compiler rotate the
        // accumulators through register copies on every iteration
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c[k]) : "v"(a[(k + j) & 7]), "v"(b[k]));
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kChains; ++k) s += c[k][0] + c[k][1] + c[k][2] + c[k][3];
  out[(size_t)blockIdx.x * blockDim.x + t] = s;
  if (clk != nullptr && t == 0) {
    const unsigned long long c1 = __builtin_amdgcn_s_memtime(), w1 = __builtin_amdgcn_s_memrealtime();
    clk[2 * (size_t)blockIdx.x] = c1 - c0;
    clk[2 * (size_t)blockIdx.x + 1] = w1 - w0;
  }
}

// Streams `n16` 16-byte chunks with one load per chunk (grid-stride), adds
// their words so the loads cannot be dropped, one float per thread to `out`.
__global__ __launch_bounds__(256) void read_probe_kernel(const uint4* __restrict__ src, size_t n16,
                                                         float* __restrict__ out) {
  const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  for (size_t i = tid; i < n16; i += stride) {
    const uint4 w = src[i];
    acc += w.x ^ w.y ^ w.z ^ w.w;
  }
  out[tid] = (float)acc;
}


// LDS tiles laid out as in the attention kernels: rows of 2*128 + 32 bytes.
constexpr int kLdsStride = 288;
constexpr int kLdsRows = 80;   // 64-row tile plus a sliding offset of up to 15 rows

// mode 0: 16-byte row reads (the score operand pattern, ds_read_b128);
// mode 1: 8-byte transposed reads (the value operand pattern, ds_read_b64_tr_b16).
// 16 reads per lane per iteration; the row offset slides with the iteration
// so that no read is loop-invariant. Every access stays inside the tile.
__global__ __launch_bounds__(256) void lds_probe_kernel(int iters, int mode, float* out) {
  __shared__ __attribute__((aligned(16))) char buf[kLdsRows * kLdsStride];
  for (int i = threadIdx.x; i < kLdsRows * kLdsStride / 4; i += 256)
    reinterpret_cast<uint32_t*>(buf)[i] = (uint32_t)i * 2654435761u;
  __syncthreads();
  const int lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
  uint32_t a0 = 0, a1 = 0;
  if (mode == 0) {
    for (int it = 0; it < iters; ++it) {
      const int r0 = it & 15;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int mt = k & 3, kk = k >> 2;   // rows <= 48 + 15 + 15, bytes <= 2 * (96 + 24) + 16
        const uint4 v = *reinterpret_cast<const uint4*>(buf + (16 * mt + c16 + r0) * kLdsStride + (32 * kk + 8 * g) * 2);
        a0 ^= v.x ^ v.y;
        a1 ^= v.z ^ v.w;
      }
    }
  } else {
    const int tr_row = 4 * g + (c16 >> 2), tr_col = 4 * (c16 & 3);
    for (int it = 0; it < iters; ++it) {
      const int r0 = it & 15;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int dt = k >> 1, half = k & 1;   // rows <= 16 + 15 + 15 (+ 32 below), bytes <= 2 * (112 + 12) + 8
        const char* p = buf + (32 * (it & 1) + 16 * half + tr_row + r0) * kLdsStride + (16 * dt + tr_col) * 2;
        const short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(p));
        const uint2 w = __builtin_bit_cast(uint2, v);
        a0 ^= w.x;
        a1 ^= w.y;
      }
    }
  }
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = (float)(a0 ^ a1);
}
}  // namespace

// Reads `bytes` (a multiple of 16) from device memory `src` once with
// `blocks` workgroups of 256 threads; `out` must hold blocks * 256 floats.
PROBE_API int isa_probe_read(const void* src, size_t bytes, int blocks, float* out, void* stream) {
  if (!src || !out || blocks < 1 || bytes % 16) return -1;
  read_probe_kernel<<<blocks, 256, 0, reinterpret_cast<hipStream_t>(stream)>>>(
      reinterpret_cast<const uint4*>(src), bytes / 16, out);
  return (int)hipGetLastError();
}

// Launches `blocks` workgroups of 256 threads, each wave issuing
// iters * 64 MFMAs of 16x16x32 (16384 flops each) on operands of the given
// mode (0: constant low-activity operands, 1: random operands); `out` must
// hold blocks * 256 floats, `clk` (may be null) 2 * blocks 64-bit words.
// Returns 0 or the HIP error code (-1 for bad arguments).
PROBE_API int isa_probe_mfma_bf16(int blocks, int iters, int mode, float* out, unsigned long long* clk,
                                  void* stream) {
  if (blocks < 1 || iters < 1 || (mode != 0 && mode != 1) || !out) return -1;
  mfma_probe_kernel<<<blocks, 256, 0, reinterpret_cast<hipStream_t>(stream)>>>(iters, mode, out, clk);
  return (int)hipGetLastError();
}

// Flops one isa_probe_mfma_bf16 launch performs.
PROBE_API double isa_probe_mfma_flops(int blocks, int iters) {
  return (double)blocks * 4.0 * iters * kMfmaPerIter * 16.0 * 16.0 * 32.0 * 2.0;
}

// Rate of the constant-rate clock read by s_memrealtime on the current
// device, in kHz (0 on error).
PROBE_API int isa_probe_wallclock_khz() {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
  return khz;
}

// Launches `blocks` workgroups of 256 threads reading LDS (mode 0: 16-byte
// row reads, mode 1: 8-byte transposed reads), iters * 16 reads per thread;
// `out` must hold blocks * 256 floats. Returns 0 or the HIP error code.
PROBE_API int isa_probe_lds(int blocks, int iters, int mode, float* out, void* stream) {
  if (blocks < 1 || iters < 1 || (mode != 0 && mode != 1) || !out) return -1;
  lds_probe_kernel<<<blocks, 256, 0, reinterpret_cast<hipStream_t>(stream)>>>(iters, mode, out);
  return (int)hipGetLastError();
}

// Bytes one isa_probe_lds launch reads from LDS.
PROBE_API double isa_probe_lds_bytes(int blocks, int iters, int mode) {
  return (double)blocks * 256.0 * iters * 16.0 * (mode == 0 ? 16.0 : 8.0);
}
