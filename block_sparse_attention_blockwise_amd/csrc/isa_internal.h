// Internal declarations shared by the host entry points and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "isa.h"

// Shape of one call after validation: every count of the method's steps.
struct IsaShape {
  int B, H, L_src, L_ctx, L, D, b;
  int N_src, N_ctx, N, k_ctx, N_kv, n_flat, n_sharp, k_ns;
  float gamma;
  double rope_base;
};

// Token range [start, start + n) of global block j (source blocks first,
// then context blocks; each segment is cut on its own).
__host__ __device__ inline void isa_block_range(const IsaShape& s, int j, int& start, int& n) {
  if (j < s.N_src) {
    start = j * s.b;
    int rem = s.L_src - start;
    n = rem < s.b ? rem : s.b;
  } else {
    int jc = j - s.N_src;
    start = s.L_src + jc * s.b;
    int rem = s.L_ctx - jc * s.b;
    n = rem < s.b ? rem : s.b;
  }
}

// As isa_block_range, for a block id read from memory (a selection list in
// a workspace): an id outside [0, N) gives the empty range (start 0, n 0),
// so no token row of it is ever read.
__host__ __device__ inline void isa_block_range_checked(const IsaShape& s, int j, int& start, int& n) {
  if (j < 0 || j >= s.N) {
    start = 0;
    n = 0;
    return;
  }
  isa_block_range(s, j, start, n);
}

// Buffer loads into LDS (buffer_load_dwordx4 ... lds): a buffer resource over
// a head's rows in scalar registers, a 32-bit lane offset and a wave-uniform
// byte offset, with no address arithmetic on the vector units; reads past
// the resource's size return zero. The resource type exists only in the
// device compilation; the host pass parses the kernels but never runs them.
#if defined(__HIP_DEVICE_COMPILE__)
typedef __amdgpu_buffer_rsrc_t RowsRsrc;
#else
struct RowsRsrc { int words[4]; };
#endif

__device__ inline RowsRsrc rows_rsrc(const void* p, int bytes) {
#if defined(__HIP_DEVICE_COMPILE__)
  // both halves of the (wave-uniform) base from the first lane, so that the
  // resource lives in scalar registers
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), 0,
                                           __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
#else
  (void)p; (void)bytes;
  return RowsRsrc{};
#endif
}

// Copies 16 bytes per lane from `r` at byte offset lane_off + block_off into
// LDS at `lds` + 16 * lane (`lds` and `block_off` wave-uniform).
__device__ inline void copy16_to_lds(RowsRsrc r, char* lds, uint32_t lane_off, int block_off) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, lane_off,
                                           __builtin_amdgcn_readfirstlane(block_off), 0, 0);
#else
  (void)r; (void)lds; (void)lane_off; (void)block_off;
#endif
}


// Raises a kernel's dynamic-LDS limit on the current device, once per device
// (the attribute is per device; `done` is a per-kernel bit set of devices).
inline hipError_t isa_ensure_dyn_lds(const void* kernel, int bytes, unsigned long long* done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const unsigned long long bit = 1ull << (dev & 63);
  if (__atomic_load_n(done, __ATOMIC_ACQUIRE) & bit) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) __atomic_fetch_or(done, bit, __ATOMIC_RELEASE);
  return e;
}

// Hard limits of the kernels (see isa.h).
constexpr int ISA_MAX_SEG_BLOCKS = 4096;
constexpr int ISA_MAX_NKV = 4096;

// One-time set-up of the current device (dynamic-LDS limits of the
// attention and dQ kernels); idempotent.
hipError_t isa_attn_prepare_device();
hipError_t isa_bwd_prepare_device();
hipError_t isa_select_prepare_device();

// Launchers: each returns the first HIP error met while enqueueing.
hipError_t isa_launch_pool(const IsaShape& s, const uint16_t* Q, const uint16_t* K,
                           const uint16_t* V, double* qc, double* kc, uint16_t* kc_bf16,
                           uint16_t* vc_bf16, hipStream_t st);
hipError_t isa_launch_rope_table(const IsaShape& s, float2* table, hipStream_t st);
hipError_t isa_launch_rope_pool(const IsaShape& s, const uint16_t* Q, const uint16_t* K,
                                const uint16_t* V, const float2* table, uint16_t* Qr,
                                uint16_t* Kr, double* qc, double* kc, uint16_t* kc_bf16,
                                uint16_t* vc_bf16, hipStream_t st);
hipError_t isa_launch_ctx_topk(const IsaShape& s, const double* qc, const double* kc,
                               int32_t* ctx_idx, double* ctx_score, hipStream_t st);
hipError_t isa_launch_coarse_rows(const IsaShape& s, const double* qc, const double* kc,
                                  const int32_t* ctx_idx, double* srows, hipStream_t st);
hipError_t isa_launch_sharpness(const IsaShape& s, const double* qc, const double* kc, double* sharp,
                                hipStream_t st);
hipError_t isa_launch_split(const IsaShape& s, const double* sharp, int32_t* sharp_idx,
                            int32_t* flat_idx, hipStream_t st);
// `scratch`: isa_flat_topk_scratch_bytes(s) bytes of device memory (the
// coarse rows of the flat blocks in flight when they do not fit LDS; may be
// NULL when that size is 0).
size_t isa_flat_topk_scratch_bytes(const IsaShape& s);
hipError_t isa_launch_flat_topk(const IsaShape& s, const double* qc, const double* kc,
                                const int32_t* ctx_idx, const int32_t* flat_idx,
                                int32_t* flat_exact_idx, double* scratch, hipStream_t st);
hipError_t isa_launch_coarse_residual(const IsaShape& s, const double* srows,
                                      const uint16_t* vc_bf16, const int32_t* ctx_idx,
                                      uint16_t* O, hipStream_t st);
// `lse` (nullable, [B,H,L] fp32): log2-domain log-sum-exp of every written
// row, saved for the backward pass.
hipError_t isa_launch_sharp_attn(const IsaShape& s, const uint16_t* Q, const uint16_t* K,
                                 const uint16_t* V, const int32_t* ctx_idx,
                                 const int32_t* sharp_idx, uint16_t* O, float* lse,
                                 hipStream_t st);
hipError_t isa_launch_flat_attn(const IsaShape& s, const uint16_t* Q, const uint16_t* K,
                                const uint16_t* V, const uint16_t* kc_bf16,
                                const uint16_t* vc_bf16, const int32_t* ctx_idx,
                                const int32_t* flat_idx, const int32_t* flat_exact_idx,
                                const int32_t* flat_ord, uint16_t* O, float* lse, hipStream_t st);
// Grid order of the flat blocks (flat_ord [B,H,n_flat]) for the flat kernels.
hipError_t isa_launch_flat_order(const IsaShape& s, const int32_t* flat_exact_idx, int32_t* flat_ord,
                                 hipStream_t st);
// Buffers of the backward pass (device pointers; the forward's saved state
// and the backward's scratch live in the forward workspace).
struct IsaBwdBuffers {
  const uint16_t* Q;          // attention inputs (the rotated Q, K when RoPE is on)
  const uint16_t* K;
  const uint16_t* V;
  const uint16_t* O;
  const uint16_t* dO;
  const float* lse;
  float* delta;
  const uint16_t* kcb;
  const uint16_t* vcb;
  const int32_t* ctx_idx;
  const int32_t* sharp_idx;
  const int32_t* flat_idx;
  const int32_t* exact;
  const int32_t* flat_ord;   // nullable: flat blocks in plain order
  uint64_t* ebits;
  int32_t* inv_off;
  int32_t* inv_list;
  int32_t* chunk_ord;
  float* dkc;
  float* dvc;
  const float2* rope;         // nullable
  // residual (gamma != 0) inputs and scratch
  const double* srows;
  const double* qc;
  const double* kc;
  float* dqc;
  float* doc;
  float* ocs;
  float* dsc;
  float* pc;
  uint16_t* dQ;
  uint16_t* dK;
  uint16_t* dV;
};
hipError_t isa_launch_backward(const IsaShape& s, const IsaBwdBuffers& w, hipStream_t st);
hipError_t isa_launch_dense_attn(int B, int H, int L, int D, const uint16_t* Q,
                                 const uint16_t* K, const uint16_t* V, uint16_t* O,
                                 hipStream_t st);
