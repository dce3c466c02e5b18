// Host side of the ISA library: argument validation, the counts of the
// method's steps, workspace layout and the extern "C" entry points.
//
// The counts follow the method steps of In-context Sparse Attention as given
// in the paper.rainbus.top summary of arXiv 2605.04569, section "Method
// steps": step (1) cuts the sequence into b-token blocks, step (2) keeps
// alpha_s times the number of context blocks, step (3) sends a fraction
// alpha_f of the query blocks to the flat path, step (5) computes
// alpha_ns times the kept block count exactly per flat block. Where a
// product is fractional the count is rounded toward more exact work.
#include <cmath>
#include <cstdint>
#include <cstring>

#include <initializer_list>

#include "isa_internal.h"

namespace {

constexpr double kRoundTol = 1e-9;

int ceil_count(double x) { return (int)std::ceil(x - kRoundTol); }
int floor_count(double x) { return (int)std::floor(x + kRoundTol); }

bool ratio_ok(double a) { return !std::isnan(a) && a >= 0.0 && a <= 1.0; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Layout {
  size_t qc, kc, kcb, vcb, ctx_idx, ctx_score, sharp, sharp_idx, flat_idx, exact, flat_ord, ftk, srows;
  size_t qr, kr, rope;          // RoPE buffers (only when rope_base > 0)
  size_t lse;                   // saved by isa_forward for isa_backward
  size_t delta, dkc, dvc, ebits, inv_off, inv_list, chunk_ord;   // backward scratch
  size_t dqc, doc, ocs, dsc, pc;                     // backward of the residual (gamma != 0)
  size_t total;
};

// cos/sin table of the decoupled RoPE: one float2 per (position, pair).
size_t rope_table_bytes(const IsaShape& s) {
  if (s.rope_base == 0.0) return 0;
  const size_t P = s.L_src > s.L_ctx ? s.L_src : s.L_ctx;
  return align256(P * (size_t)(s.D / 2) * sizeof(float2));
}

// with_backward = false: only what the forward's steps read and write (no
// saved log-sum-exp, no backward scratch), the layout of the static scratch.
Layout make_layout(const IsaShape& s, bool with_backward = true) {
  const size_t bh = (size_t)s.B * s.H;
  const size_t nd = bh * s.N * s.D;
  auto at_least1 = [](size_t x) { return x ? x : (size_t)1; };
  Layout l;
  size_t o = 0;
  l.qc = o;        o = align256(o + nd * 8);
  l.kc = o;        o = align256(o + nd * 8);
  l.kcb = o;       o = align256(o + nd * 2);
  l.vcb = o;       o = align256(o + nd * 2);
  l.ctx_idx = o;   o = align256(o + at_least1(bh * s.k_ctx) * 4);
  l.ctx_score = o; o = align256(o + at_least1(bh * s.N_ctx) * 8);
  l.sharp = o;     o = align256(o + bh * s.N * 8);
  l.sharp_idx = o; o = align256(o + at_least1(bh * s.n_sharp) * 4);
  l.flat_idx = o;  o = align256(o + at_least1(bh * s.n_flat) * 4);
  l.exact = o;     o = align256(o + at_least1(bh * s.n_flat * (size_t)s.k_ns) * 4);
  l.flat_ord = o;  o = align256(o + at_least1(bh * s.n_flat) * 4);
  // exact-set rows of the flat blocks in flight (only when they do not fit LDS)
  l.ftk = o;       o = align256(o + isa_flat_topk_scratch_bytes(s));
  // coarse rows S[i, J]: only the gamma residual stores them
  l.srows = o;     o = align256(o + (s.gamma != 0.0f ? bh * s.N * (size_t)s.N_kv * 8 : 0));
  const size_t qkr = s.rope_base != 0.0 ? bh * (size_t)s.L * s.D * 2 : 0;
  l.qr = o;        o = align256(o + qkr);
  l.kr = o;        o = align256(o + qkr);
  l.rope = o;      o = align256(o + rope_table_bytes(s));
  if (!with_backward) {
    l.lse = l.delta = l.dkc = l.dvc = l.ebits = l.inv_off = l.inv_list = l.chunk_ord = 0;
    l.dqc = l.doc = l.ocs = l.dsc = l.pc = 0;
    l.total = o;
    return l;
  }
  l.lse = o;       o = align256(o + bh * s.L * 4);
  l.delta = o;     o = align256(o + bh * s.L * 4);
  l.dkc = o;       o = align256(o + bh * s.N * s.D * 4);
  l.dvc = o;       o = align256(o + bh * s.N * s.D * 4);
  l.ebits = o;     o = align256(o + bh * s.n_flat * (size_t)((s.N_kv + 63) / 64) * 8);
  l.inv_off = o;   o = align256(o + bh * (size_t)(s.N_kv + 1) * 4);
  l.inv_list = o;  o = align256(o + bh * s.n_flat * (size_t)s.k_ns * 4);
  l.chunk_ord = o; o = align256(o + bh * (size_t)s.N_kv * 4);
  const bool res = s.gamma != 0.0f;
  const size_t rnd = res ? nd * 4 : 0;
  const size_t rnk = res ? bh * s.N * (size_t)s.N_kv * 4 : 0;
  l.dqc = o;       o = align256(o + rnd);
  l.doc = o;       o = align256(o + rnd);
  l.ocs = o;       o = align256(o + rnd);
  l.dsc = o;       o = align256(o + rnk);
  l.pc = o;        o = align256(o + rnk);
  l.total = o;
  return l;
}

// Workspace of isa_sharpness_split: room for the sharpness values when the
// caller passes none, then the exact-set kernel's row scratch (the coarse
// scores of the flat blocks in flight, bounded by its slot count, not by N;
// none when 16 rows of J fit LDS). Workspace of
// isa_coarse_residual: the coarse rows S[i, J] of every query block (gamma
// != 0 only). The plan reports the larger of the two.
size_t sharp_vals_bytes(const IsaShape& s) { return align256((size_t)s.B * s.H * s.N * 8); }
size_t sharp_ws_bytes(const IsaShape& s) {
  return sharp_vals_bytes(s) + align256(isa_flat_topk_scratch_bytes(s));
}
size_t residual_ws_bytes(const IsaShape& s) {
  return s.gamma != 0.0f ? align256((size_t)s.B * s.H * s.N * (size_t)s.N_kv * 8) : 0;
}
size_t scores_bytes(const IsaShape& s) {
  const size_t a = sharp_ws_bytes(s), b = residual_ws_bytes(s);
  return a > b ? a : b;
}

// Validates the parameters and derives every count. Makes no HIP call.
// (batch, head) pairs index the second grid dimension of several launches.
constexpr int64_t kMaxHeads = 65535;

int make_shape(const isa_params_t* p, IsaShape* s) {
  if (!p || !s) return ISA_ERR_ARG;
  if (p->B < 1 || p->H < 1 || p->L_src < 1 || p->L_ctx < 0 || p->D < 1 || p->b < 1)
    return ISA_ERR_ARG;
  if (!ratio_ok(p->alpha_s) || !ratio_ok(p->alpha_f) || !ratio_ok(p->alpha_ns)) return ISA_ERR_ARG;
  // gamma is applied in fp32: it must be finite there too
  if (!std::isfinite(p->gamma) || std::fabs(p->gamma) > 3.0e38) return ISA_ERR_ARG;
  if (!(p->rope_base == 0.0 || (std::isfinite(p->rope_base) && p->rope_base > 1.0))) return ISA_ERR_ARG;
  if (p->D != 64 && p->D != 128) return ISA_ERR_UNSUPPORTED;
  if ((int64_t)p->B * p->H > kMaxHeads) return ISA_ERR_UNSUPPORTED;
  if (p->b != 32 && p->b != 64) return ISA_ERR_UNSUPPORTED;
  const int64_t N_src = ((int64_t)p->L_src + p->b - 1) / p->b;
  const int64_t N_ctx = ((int64_t)p->L_ctx + p->b - 1) / p->b;
  if (N_src > ISA_MAX_SEG_BLOCKS || N_ctx > ISA_MAX_SEG_BLOCKS) return ISA_ERR_UNSUPPORTED;
  IsaShape r;
  r.B = p->B; r.H = p->H; r.L_src = p->L_src; r.L_ctx = p->L_ctx;
  r.L = p->L_src + p->L_ctx; r.D = p->D; r.b = p->b;
  r.N_src = (int)N_src; r.N_ctx = (int)N_ctx; r.N = r.N_src + r.N_ctx;
  r.k_ctx = ceil_count(p->alpha_s * r.N_ctx);
  if (r.k_ctx > r.N_ctx) r.k_ctx = r.N_ctx;
  r.N_kv = r.N_src + r.k_ctx;
  if (r.N_kv > ISA_MAX_NKV) return ISA_ERR_UNSUPPORTED;
  r.n_flat = floor_count(p->alpha_f * r.N);
  if (r.n_flat > r.N) r.n_flat = r.N;
  r.n_sharp = r.N - r.n_flat;
  r.k_ns = ceil_count(p->alpha_ns * r.N_kv);
  if (r.k_ns > r.N_kv) r.k_ns = r.N_kv;
  r.gamma = (float)p->gamma;
  r.rope_base = p->rope_base;
  *s = r;
  return ISA_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? ISA_OK : ISA_ERR_HIP; }

// Workspace of isa_forward_noalloc: a device array of the library, one copy
// per device (each holds it until the process ends). Host code never passes
// `scratch` itself to a kernel: its name is a host-side stand-in, and the
// device copy's address comes from hipGetSymbolAddress, resolved once per
// device with that device current.
static __device__ __align__(256) unsigned char scratch[ISA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch_addr[kMaxDevices];   // device address of `scratch`, per device (null until resolved)

// The current device's copy of `scratch`.
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ISA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return ISA_ERR_UNSUPPORTED;
  void* ptr = __atomic_load_n(&g_scratch_addr[dev], __ATOMIC_ACQUIRE);
  if (ptr == nullptr) {
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return ISA_ERR_HIP;
    __atomic_store_n(&g_scratch_addr[dev], ptr, __ATOMIC_RELEASE);   // same value from any thread
  }
  *out = ptr;
  return ISA_OK;
}

hipStream_t as_stream(void* st) { return reinterpret_cast<hipStream_t>(st); }

// The kernels move token rows and workspace data in 16-byte vectors.
bool aligned16(std::initializer_list<const void*> ptrs) {
  for (const void* q : ptrs)
    if (reinterpret_cast<uintptr_t>(q) & 15u) return false;
  return true;
}

}  // namespace

extern "C" {

int isa_plan(const isa_params_t* p, isa_plan_t* out) {
  if (!out) return ISA_ERR_ARG;
  IsaShape s;
  int rc = make_shape(p, &s);
  if (rc != ISA_OK) return rc;
  out->N_src = s.N_src; out->N_ctx = s.N_ctx; out->N = s.N; out->k_ctx = s.k_ctx;
  out->N_kv = s.N_kv; out->n_flat = s.n_flat; out->n_sharp = s.n_sharp; out->k_ns = s.k_ns;
  out->workspace_bytes = make_layout(s).total;
  out->scores_bytes = scores_bytes(s);
  out->rope_bytes = rope_table_bytes(s);
  out->noalloc_bytes = make_layout(s, false).total;
  return ISA_OK;
}

int isa_pool_coarse(const isa_params_t* p, const void* Q, const void* K, const void* V,
                    double* qc, double* kc, void* kc_bf16, void* vc_bf16, void* stream) {
  IsaShape s;
  int rc = make_shape(p, &s);
  if (rc != ISA_OK) return rc;
  if (!Q || !K || !V || !qc || !kc || !aligned16({Q, K, V, qc, kc, kc_bf16, vc_bf16}))
    return ISA_ERR_ARG;
  return hip_status(isa_launch_pool(s, (const uint16_t*)Q, (const uint16_t*)K, (const uint16_t*)V,
                                    qc, kc, (uint16_t*)kc_bf16, (uint16_t*)vc_bf16,
                                    as_stream(stream)));
}

int isa_rope_pool_coarse(const isa_params_t* p, const void* Q, const void* K, const void* V,
                         void* Qr, void* Kr, double* qc, double* kc, void* kc_bf16, void* vc_bf16,
                         void* ws, size_t ws_bytes, void* stream) {
  IsaShape s;
  int rc = make_shape(p, &s);
  if (rc != ISA_OK) return rc;
  if (!Q || !K || !V || !Qr || !Kr || !qc || !kc || !ws || s.rope_base == 0.0) return ISA_ERR_ARG;
  if (!aligned16({Q, K, V, Qr, Kr, ws, qc, kc, kc_bf16, vc_bf16})) return ISA_ERR_ARG;
  if (ws_bytes < rope_table_bytes(s)) return ISA_ERR_WORKSPACE;
  hipStream_t st = as_stream(stream);
  float2* table = (float2*)ws;
  hipError_t e = isa_launch_rope_table(s, table, st);
  if (e == hipSuccess)
    e = isa_launch_rope_pool(s, (const uint16_t*)Q, (const uint16_t*)K, (const uint16_t*)V, table,
                             (uint16_t*)Qr, (uint16_t*)Kr, qc, kc, (uint16_t*)kc_bf16,
                             (uint16_t*)vc_bf16, st);
  return hip_status(e);
}

int isa_ctx_topk(const isa_params_t* p, const double* qc, const double* kc, int32_t* ctx_idx,
                 double* ctx_score, void* stream) {
  IsaShape s;
  int rc = make_shape(p, &s);
  if (rc != ISA_OK) return rc;
  if (!qc || !kc || (!ctx_idx && s.k_ctx > 0) || !aligned16({qc, kc})) return ISA_ERR_ARG;
  return hip_status(isa_launch_ctx_topk(s, qc, kc, ctx_idx, ctx_score, as_stream(stream)));
}

int isa_sharpness_split(const isa_params_t* p, const double* qc, const double* kc,
                        const int32_t* ctx_idx, double* sharpness, int32_t* sharp_idx,
                        int32_t* flat_idx, int32_t* flat_exact_idx, void* ws, size_t ws_bytes,
                        void* stream) {
  IsaShape s;
  int rc = make_shape(p, &s);
  if (rc != ISA_OK) return rc;
  if (!qc || !kc || (!ctx_idx && s.k_ctx > 0) || (!sharp_idx && s.n_sharp > 0) ||
      (!flat_idx && s.n_flat > 0) || (!flat_exact_idx && s.n_flat > 0 && s.k_ns > 0) || !ws ||
      !aligned16({qc, kc, ws}))
    return ISA_ERR_ARG;
  if (ws_bytes < sharp_ws_bytes(s)) return ISA_ERR_WORKSPACE;
  hipStream_t st = as_stream(stream);
  double* sharp = sharpness ? sharpness : (double*)ws;
  double* ftk = (double*)((char*)ws + sharp_vals_bytes(s));
  hipError_t e = isa_launch_sharpness(s, qc, kc, sharp, st);
  if (e == hipSuccess) e = isa_launch_split(s, sharp, sharp_idx, flat_idx, st);
  if (e == hipSuccess) e = isa_launch_flat_topk(s, qc, kc, ctx_idx, flat_idx, flat_exact_idx, ftk, st);
  return hip_status(e);
}

int isa_sharp_attn(const isa_params_t* p, const void* Q, const void* K, const void* V,
                   const int32_t* ctx_idx, const int32_t* sharp_idx, void* O, void* stream) {
  IsaShape s;
  int rc = make_shape(p, &s);
  if (rc != ISA_OK) return rc;
  if (!Q || !K || !V || !O || (!ctx_idx && s.k_ctx > 0) || (!sharp_idx && s.n_sharp > 0))
    return ISA_ERR_ARG;
  if (!aligned16({Q, K, V, O})) return ISA_ERR_ARG;
  return hip_status(isa_launch_sharp_attn(s, (const uint16_t*)Q, (const uint16_t*)K,
                                          (const uint16_t*)V, ctx_idx, sharp_idx, (uint16_t*)O, nullptr,
                                          as_stream(stream)));
}

int isa_flat_taylor_attn(const isa_params_t* p, const void* Q, const void* K, const void* V,
                         const void* kc_bf16, const void* vc_bf16, const int32_t* ctx_idx,
                         const int32_t* flat_idx, const int32_t* flat_exact_idx, void* O,
                         void* stream) {
  IsaShape s;
  int rc = make_shape(p, &s);
  if (rc != ISA_OK) return rc;
  if (!Q || !K || !V || !O || !kc_bf16 || !vc_bf16 || (!ctx_idx && s.k_ctx > 0) ||
      (!flat_idx && s.n_flat > 0) || (!flat_exact_idx && s.n_flat > 0 && s.k_ns > 0))
    return ISA_ERR_ARG;
  if (!aligned16({Q, K, V, O, kc_bf16, vc_bf16})) return ISA_ERR_ARG;
  return hip_status(isa_launch_flat_attn(s, (const uint16_t*)Q, (const uint16_t*)K,
                                         (const uint16_t*)V, (const uint16_t*)kc_bf16,
                                         (const uint16_t*)vc_bf16, ctx_idx, flat_idx,
                                         flat_exact_idx, nullptr, (uint16_t*)O, nullptr,
                                         as_stream(stream)));
}

int isa_coarse_residual(const isa_params_t* p, const double* qc, const double* kc,
                        const void* vc_bf16, const int32_t* ctx_idx, void* O, void* ws,
                        size_t ws_bytes, void* stream) {
  IsaShape s;
  int rc = make_shape(p, &s);
  if (rc != ISA_OK) return rc;
  if (!qc || !kc || !vc_bf16 || (!ctx_idx && s.k_ctx > 0) || !O || !ws ||
      !aligned16({qc, kc, vc_bf16, O, ws}))
    return ISA_ERR_ARG;
  if (s.gamma == 0.0f) return ISA_OK;
  if (ws_bytes < residual_ws_bytes(s)) return ISA_ERR_WORKSPACE;
  hipStream_t st = as_stream(stream);
  double* srows = (double*)ws;
  hipError_t e = isa_launch_coarse_rows(s, qc, kc, ctx_idx, srows, st);
  if (e == hipSuccess)
    e = isa_launch_coarse_residual(s, srows, (const uint16_t*)vc_bf16, ctx_idx, (uint16_t*)O, st);
  return hip_status(e);
}

}  // extern "C"

namespace {

// Steps (1)-(6) on a validated shape, intermediate data in `w` laid out as
// `l`; the row log-sum-exp is saved only when the layout has room for it.
int forward_impl(const IsaShape& s, const void* Q, const void* K, const void* V, void* O, char* w,
                 const Layout& l, const isa_debug_t* dbg, hipStream_t st) {
  double* qc = (double*)(w + l.qc);
  double* kc = (double*)(w + l.kc);
  uint16_t* kcb = (uint16_t*)(w + l.kcb);
  uint16_t* vcb = (uint16_t*)(w + l.vcb);
  int32_t* ctx_idx = (int32_t*)(w + l.ctx_idx);
  double* ctx_score = (double*)(w + l.ctx_score);
  double* sharp = (double*)(w + l.sharp);
  int32_t* sharp_idx = (int32_t*)(w + l.sharp_idx);
  int32_t* flat_idx = (int32_t*)(w + l.flat_idx);
  int32_t* exact = (int32_t*)(w + l.exact);
  double* srows = (double*)(w + l.srows);
  const uint16_t* q = (const uint16_t*)Q;
  const uint16_t* k = (const uint16_t*)K;
  const uint16_t* v = (const uint16_t*)V;

  hipError_t e = hipSuccess;
  if (s.rope_base != 0.0) {
    uint16_t* qr = (uint16_t*)(w + l.qr);
    uint16_t* kr = (uint16_t*)(w + l.kr);
    float2* table = (float2*)(w + l.rope);
    e = isa_launch_rope_table(s, table, st);
    if (e == hipSuccess) e = isa_launch_rope_pool(s, q, k, v, table, qr, kr, qc, kc, kcb, vcb, st);
    q = qr;   // every later step reads the rotated tensors
    k = kr;
  } else {
    e = isa_launch_pool(s, q, k, v, qc, kc, kcb, vcb, st);
  }
  if (e == hipSuccess) e = isa_launch_ctx_topk(s, qc, kc, ctx_idx, ctx_score, st);
  if (e == hipSuccess) e = isa_launch_sharpness(s, qc, kc, sharp, st);
  if (e == hipSuccess) e = isa_launch_split(s, sharp, sharp_idx, flat_idx, st);
  if (e == hipSuccess) e = isa_launch_flat_topk(s, qc, kc, ctx_idx, flat_idx, exact, (double*)(w + l.ftk), st);
  int32_t* flat_ord = (s.n_flat > 0 && s.k_ns > 0) ? (int32_t*)(w + l.flat_ord) : nullptr;
  if (e == hipSuccess && flat_ord) e = isa_launch_flat_order(s, exact, flat_ord, st);
  float* lse = l.lse ? (float*)(w + l.lse) : nullptr;
  if (e == hipSuccess) e = isa_launch_sharp_attn(s, q, k, v, ctx_idx, sharp_idx, (uint16_t*)O, lse, st);
  if (e == hipSuccess)
    e = isa_launch_flat_attn(s, q, k, v, kcb, vcb, ctx_idx, flat_idx, exact, flat_ord, (uint16_t*)O, lse, st);
  if (e == hipSuccess && s.gamma != 0.0f) {
    // the residual's pooled attention reads whole coarse rows (kept for the backward)
    e = isa_launch_coarse_rows(s, qc, kc, ctx_idx, srows, st);
    if (e == hipSuccess) e = isa_launch_coarse_residual(s, srows, vcb, ctx_idx, (uint16_t*)O, st);
  }
  if (e == hipSuccess && dbg) {
    const size_t bh = (size_t)s.B * s.H;
    struct { void* dst; const void* src; size_t n; } cp[] = {
        {dbg->qc, qc, bh * s.N * s.D * 8},
        {dbg->kc, kc, bh * s.N * s.D * 8},
        {dbg->ctx_score, ctx_score, bh * s.N_ctx * 8},
        {dbg->ctx_idx, ctx_idx, bh * s.k_ctx * 4},
        {dbg->sharpness, sharp, bh * s.N * 8},
        {dbg->sharp_idx, sharp_idx, bh * s.n_sharp * 4},
        {dbg->flat_idx, flat_idx, bh * s.n_flat * 4},
        {dbg->flat_exact_idx, exact, bh * s.n_flat * (size_t)s.k_ns * 4},
    };
    for (auto& c : cp) {
      if (e != hipSuccess) break;
      if (c.dst && c.n) e = hipMemcpyAsync(c.dst, c.src, c.n, hipMemcpyDeviceToDevice, st);
    }
  }
  return hip_status(e);
}

}  // namespace

extern "C" {

int isa_forward(const isa_params_t* p, const void* Q, const void* K, const void* V, void* O,
                void* ws, size_t ws_bytes, const isa_debug_t* dbg, void* stream) {
  IsaShape s;
  int rc = make_shape(p, &s);
  if (rc != ISA_OK) return rc;
  if (!Q || !K || !V || !O || !ws || !aligned16({Q, K, V, O, ws})) return ISA_ERR_ARG;
  const Layout l = make_layout(s);
  if (ws_bytes < l.total) return ISA_ERR_WORKSPACE;
  return forward_impl(s, Q, K, V, O, (char*)ws, l, dbg, as_stream(stream));
}

int isa_forward_noalloc(const isa_params_t* p, const void* Q, const void* K, const void* V,
                        void* O, const isa_debug_t* dbg, void* stream) {
  IsaShape s;
  int rc = make_shape(p, &s);
  if (rc != ISA_OK) return rc;
  if (!Q || !K || !V || !O || !aligned16({Q, K, V, O})) return ISA_ERR_ARG;
  const Layout l = make_layout(s, false);
  if (l.total > ISA_NOALLOC_SCRATCH_BYTES) return ISA_ERR_SCRATCH;
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc != ISA_OK) return rc;
  return forward_impl(s, Q, K, V, O, (char*)ws, l, dbg, as_stream(stream));
}

int isa_init(void) {
  hipError_t e = isa_attn_prepare_device();
  if (e == hipSuccess) e = isa_bwd_prepare_device();
  if (e == hipSuccess) e = isa_select_prepare_device();
  if (e != hipSuccess) return ISA_ERR_HIP;
  void* ws = nullptr;
  return scratch_address(&ws);
}

int isa_backward(const isa_params_t* p, const void* Q, const void* K, const void* V,
                 const void* O, const void* dO, void* dQ, void* dK, void* dV, void* ws,
                 size_t ws_bytes, void* stream) {
  IsaShape s;
  int rc = make_shape(p, &s);
  if (rc != ISA_OK) return rc;
  if (!Q || !K || !V || !O || !dO || !dQ || !dK || !dV || !ws) return ISA_ERR_ARG;
  if (!aligned16({Q, K, V, O, dO, dQ, dK, dV, ws})) return ISA_ERR_ARG;
  const Layout l = make_layout(s);
  if (ws_bytes < l.total) return ISA_ERR_WORKSPACE;
  char* w = (char*)ws;
  IsaBwdBuffers b{};
  const bool rope = s.rope_base != 0.0;
  b.Q = rope ? (const uint16_t*)(w + l.qr) : (const uint16_t*)Q;
  b.K = rope ? (const uint16_t*)(w + l.kr) : (const uint16_t*)K;
  b.V = (const uint16_t*)V;
  b.O = (const uint16_t*)O;
  b.dO = (const uint16_t*)dO;
  b.lse = (const float*)(w + l.lse);
  b.delta = (float*)(w + l.delta);
  b.kcb = (const uint16_t*)(w + l.kcb);
  b.vcb = (const uint16_t*)(w + l.vcb);
  b.ctx_idx = (const int32_t*)(w + l.ctx_idx);
  b.sharp_idx = (const int32_t*)(w + l.sharp_idx);
  b.flat_idx = (const int32_t*)(w + l.flat_idx);
  b.exact = (const int32_t*)(w + l.exact);
  b.flat_ord = (s.n_flat > 0 && s.k_ns > 0) ? (const int32_t*)(w + l.flat_ord) : nullptr;
  b.ebits = (uint64_t*)(w + l.ebits);
  b.inv_off = (int32_t*)(w + l.inv_off);
  b.inv_list = (int32_t*)(w + l.inv_list);
  b.chunk_ord = (int32_t*)(w + l.chunk_ord);
  b.dkc = (float*)(w + l.dkc);
  b.dvc = (float*)(w + l.dvc);
  b.rope = rope ? (const float2*)(w + l.rope) : nullptr;
  b.srows = (const double*)(w + l.srows);
  b.qc = (const double*)(w + l.qc);
  b.kc = (const double*)(w + l.kc);
  b.dqc = (float*)(w + l.dqc);
  b.doc = (float*)(w + l.doc);
  b.ocs = (float*)(w + l.ocs);
  b.dsc = (float*)(w + l.dsc);
  b.pc = (float*)(w + l.pc);
  b.dQ = (uint16_t*)dQ;
  b.dK = (uint16_t*)dK;
  b.dV = (uint16_t*)dV;
  return hip_status(isa_launch_backward(s, b, as_stream(stream)));
}

int isa_dense_attn(int32_t B, int32_t H, int32_t L, int32_t D, const void* Q, const void* K,
                   const void* V, void* O, void* stream) {
  if (B < 1 || H < 1 || L < 1 || D < 1 || !Q || !K || !V || !O) return ISA_ERR_ARG;
  if (!aligned16({Q, K, V, O})) return ISA_ERR_ARG;
  if (D != 64 && D != 128) return ISA_ERR_UNSUPPORTED;
  if ((int64_t)B * H > kMaxHeads) return ISA_ERR_UNSUPPORTED;
  // one head's rows must be addressable with 32-bit byte offsets
  if ((int64_t)L * D * 2 > (int64_t)INT32_MAX) return ISA_ERR_UNSUPPORTED;
  return hip_status(isa_launch_dense_attn(B, H, L, D, (const uint16_t*)Q, (const uint16_t*)K,
                                          (const uint16_t*)V, (uint16_t*)O, as_stream(stream)));
}

const char* isa_strerror(int status) {
  switch (status) {
    case ISA_OK: return "ok";
    case ISA_ERR_ARG: return "invalid argument (null pointer, bad shape or ratio)";
    case ISA_ERR_UNSUPPORTED: return "unsupported configuration (D, b or block counts outside the limits)";
    case ISA_ERR_WORKSPACE: return "workspace too small";
    case ISA_ERR_HIP: return "HIP launch or copy failed";
    case ISA_ERR_SCRATCH:
      return "request needs more than the library's static scratch (ISA_NOALLOC_SCRATCH_BYTES); "
             "use isa_forward with a caller workspace";
    default: return "unknown status";
  }
}

}  // extern "C"
