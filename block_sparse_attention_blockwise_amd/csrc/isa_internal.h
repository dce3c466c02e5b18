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

// Hard limits of the kernels (see isa.h).
constexpr int ISA_MAX_SEG_BLOCKS = 4096;
constexpr int ISA_MAX_NKV = 4096;

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
hipError_t isa_launch_sharpness(const IsaShape& s, const double* srows, double* sharp,
                                hipStream_t st);
hipError_t isa_launch_split(const IsaShape& s, const double* sharp, int32_t* sharp_idx,
                            int32_t* flat_idx, hipStream_t st);
hipError_t isa_launch_flat_topk(const IsaShape& s, const double* srows, const int32_t* ctx_idx,
                                const int32_t* flat_idx, int32_t* flat_exact_idx,
                                hipStream_t st);
hipError_t isa_launch_coarse_residual(const IsaShape& s, const double* srows,
                                      const uint16_t* vc_bf16, const int32_t* ctx_idx,
                                      uint16_t* O, hipStream_t st);
hipError_t isa_launch_sharp_attn(const IsaShape& s, const uint16_t* Q, const uint16_t* K,
                                 const uint16_t* V, const int32_t* ctx_idx,
                                 const int32_t* sharp_idx, uint16_t* O, hipStream_t st);
hipError_t isa_launch_flat_attn(const IsaShape& s, const uint16_t* Q, const uint16_t* K,
                                const uint16_t* V, const uint16_t* kc_bf16,
                                const uint16_t* vc_bf16, const int32_t* ctx_idx,
                                const int32_t* flat_idx, const int32_t* flat_exact_idx,
                                uint16_t* O, hipStream_t st);
hipError_t isa_launch_dense_attn(int B, int H, int L, int D, const uint16_t* Q,
                                 const uint16_t* K, const uint16_t* V, uint16_t* O,
                                 hipStream_t st);
