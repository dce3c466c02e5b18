/*
 * isa.h - C ABI of the MI355X (gfx950) In-context Sparse Attention library.
 *
 * In-context Sparse Attention (ISA) is the attention operator of the
 * LIVEditor paper (arXiv 2605.04569). The method is defined in the
 * paper.rainbus.top structured summary of that paper, section "Method steps",
 * steps (1)-(6), with the 0th-order Taylor term explained in its
 * "Prerequisites" section. The same workflow is told in the techwalker.com
 * article on the paper, sections 4 and 5. Per (batch, head) it runs:
 *   (1) cut Q/K/V into b-token blocks; mean-pool each block to Qc, Kc, Vc;
 *       coarse scores S = Qc Kc^T / sqrt(D);
 *   (2) keep the top ceil(alpha_s * N_ctx) context blocks, ranked by their
 *       coarse scores summed over the source query rows; J = all source
 *       blocks + kept context blocks;
 *   (3) sharpness M_i = Var(softmax(S[i, source columns])); the floor(alpha_f*N)
 *       least sharp query blocks are "flat", the rest "sharp";
 *   (4) sharp blocks: exact softmax attention over the tokens of J;
 *   (5) flat block i: exact attention over its top ceil(alpha_ns*|J|) blocks
 *       E_i of J (by coarse score), plus for every other block j of J the term
 *       n_j * exp(q.Kc_j / sqrt(D)) in the denominator and that weight times
 *       Vc_j in the numerator (n_j = valid tokens of block j); one softmax
 *       accumulator merges both;
 *   (6) outputs land at their token positions, plus gamma * O_coarse_i on
 *       every token of block i, where O_coarse_i is the pooled attention at
 *       block resolution over the kept blocks: softmax_j(S[i, j], j in J)
 *       applied to Vc_j. The pages leave gamma open; gamma = 0 (the default)
 *       skips the residual.
 *
 * Conventions shared by every entry point
 *   Layout:    Q, K, V, O are dense row-major [B, H, L, D] bf16 (raw 16-bit
 *              words), L = L_src + L_ctx, source tokens first. Base pointers
 *              must be 16-byte aligned.
 *   Blocks:    cut per segment: source blocks 0..N_src-1 cover tokens
 *              [j*b, min((j+1)*b, L_src)); context block N_src+j covers
 *              [L_src + j*b, min(L_src + (j+1)*b, L)). A tail block holds
 *              n_j < b tokens; its means are over those n_j tokens.
 *              Block ids are global (source then context). Every index list
 *              is sorted ascending.
 *   Counts:    N_src = ceil(L_src/b), N_ctx = ceil(L_ctx/b), N = N_src+N_ctx,
 *              k_ctx = ceil(alpha_s*N_ctx), N_kv = N_src + k_ctx,
 *              n_flat = floor(alpha_f*N), n_sharp = N - n_flat,
 *              k_ns = min(N_kv, ceil(alpha_ns*N_kv)); ceil/floor are taken
 *              with a 1e-9 tolerance (ceil(x - 1e-9), floor(x + 1e-9)).
 *   Ties:      every selection prefers the lower index among equal scores;
 *              in the split a lower index counts as sharper.
 *   Ownership: the caller allocates every buffer (device memory unless
 *              stated) and the workspace sized by isa_plan. The library never
 *              allocates or frees memory and never synchronises the host.
 *              All work is enqueued on `stream` (a hipStream_t; NULL = the
 *              default stream); results are valid once the caller
 *              synchronises that stream. Only kernels are enqueued (no
 *              memset; copies only for isa_forward's optional debug
 *              outputs), so a caller may capture isa_forward and
 *              isa_backward in a HIP graph and replay it on new contents
 *              of the same buffers, after isa_init() or one call outside
 *              the capture on the device (that sets kernel attributes).
 *   Errors:    every call returns ISA_OK (0) or a negative code. Arguments
 *              are validated on the host before anything is enqueued; on
 *              error nothing is launched or written. No call aborts or
 *              throws.
 *   State:     the library keeps two things per device, each set once and
 *              never changed after: that the attention kernels' dynamic-LDS
 *              limit has been raised, and the device address of its static
 *              scratch array (used only by isa_forward_noalloc, whose
 *              contents persist from one such call to the next). Both are set
 *              by isa_init() or by the first call that needs them on that
 *              device; the flags are atomic, so calls from several host
 *              threads are safe. Nothing else persists between calls.
 *   Numerics:  pooling and every selection score run in fp64; attention uses
 *              bf16 MFMA with fp32 accumulation; outputs are bf16
 *              (round-to-nearest-even). Identical inputs give bitwise
 *              identical outputs and selections.
 *   Alignment: Q, K, V, O, dO, dQ, dK, dV, Qr, Kr, the fp64 and bf16 block
 *              means and every workspace must start on a 16-byte boundary
 *              (the kernels move 16-byte vectors); otherwise ISA_ERR_ARG.
 *   Limits:    D in {64, 128}; b in {32, 64}; L_src >= 1; L_ctx >= 0;
 *              B, H >= 1; B * H <= 65535; N_src <= 4096; N_ctx <= 4096;
 *              N_kv <= 4096;
 *              ratios in [0, 1] (NaN rejected); gamma finite with
 *              |gamma| <= 3e38 (it is applied in fp32); rope_base 0 or
 *              finite and > 1.
 */
#ifndef ISA_H
#define ISA_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define ISA_API __attribute__((visibility("default")))
#else
#define ISA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

#define ISA_OK 0
#define ISA_ERR_ARG (-1)          /* null pointer, bad shape or ratio */
#define ISA_ERR_UNSUPPORTED (-2)  /* valid request outside the limits above */
#define ISA_ERR_WORKSPACE (-3)    /* workspace smaller than isa_plan says */
#define ISA_ERR_HIP (-4)          /* a HIP launch or copy failed */
#define ISA_ERR_SCRATCH (-5)      /* isa_forward_noalloc: the request needs more
                                     than ISA_NOALLOC_SCRATCH_BYTES */

/* Size of the device array that isa_forward_noalloc uses as its workspace
 * (one copy per device, held until the process ends): 64 MiB. */
#define ISA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

typedef struct {
  int32_t B, H;        /* batch, heads */
  int32_t L_src;       /* source tokens (first in the sequence) */
  int32_t L_ctx;       /* context tokens (after the source tokens) */
  int32_t D;           /* head dimension */
  int32_t b;           /* block size in tokens */
  double alpha_s;      /* fraction of context blocks kept (step 2) */
  double alpha_f;      /* fraction of query blocks on the flat path (step 3) */
  double alpha_ns;     /* fraction of J computed exactly per flat block (step 5) */
  double gamma;        /* weight of the low-frequency residual (step 6); 0 = off */
  double rope_base;    /* > 1: decoupled RoPE on Q and K before step 1 (read by
                          isa_forward and isa_rope_pool_coarse; the other step
                          entry points take Q and K as given, so pass them the
                          rotated tensors); 0 = off */
} isa_params_t;

typedef struct {
  int32_t N_src, N_ctx, N, k_ctx, N_kv, n_flat, n_sharp, k_ns;
  size_t workspace_bytes; /* device workspace isa_forward needs */
  size_t scores_bytes;    /* workspace isa_sharpness_split and isa_coarse_residual
                             need (the larger of the two) */
  size_t rope_bytes;      /* workspace isa_rope_pool_coarse needs (0 if RoPE off) */
  size_t noalloc_bytes;   /* scratch isa_forward_noalloc needs (it refuses the
                             call when this exceeds ISA_NOALLOC_SCRATCH_BYTES) */
} isa_plan_t;

/* Optional device buffers isa_forward fills when non-NULL (debug and tests). */
typedef struct {
  double *qc, *kc;          /* [B,H,N,D] fp64 block means of Q and K        */
  double *ctx_score;        /* [B,H,N_ctx] context importance (step 2)      */
  int32_t *ctx_idx;         /* [B,H,k_ctx] kept context blocks, global ids  */
  double *sharpness;        /* [B,H,N] M_i (step 3)                         */
  int32_t *sharp_idx;       /* [B,H,n_sharp] sharp query blocks             */
  int32_t *flat_idx;        /* [B,H,n_flat] flat query blocks               */
  int32_t *flat_exact_idx;  /* [B,H,n_flat,k_ns] E_i, row r for flat_idx[r] */
} isa_debug_t;

/* Host only: validate `p` and fill the counts and workspace sizes. Makes no
 * HIP call. Step (1)-(5) counts as stated above. */
ISA_API int isa_plan(const isa_params_t* p, isa_plan_t* out);

/* Step (1): block means. Reads Q, K, V; writes qc, kc ([B,H,N,D] fp64) and
 * kc_bf16, vc_bf16 ([B,H,N,D] bf16 copies of the K and V means, rounded to
 * nearest even, used by the Taylor term). Any output pointer except qc and
 * kc may be NULL. */
ISA_API int isa_pool_coarse(const isa_params_t* p, const void* Q, const void* K, const void* V,
                    double* qc, double* kc, void* kc_bf16, void* vc_bf16, void* stream);

/* Decoupled RoPE fused with step (1). Rotary embedding of Q and K on
 * interleaved pairs (2i, 2i+1) with angle pos * rope_base^(-2i/D), where
 * source tokens take positions 0..L_src-1 and context tokens restart at 0
 * (source and context positions are encoded independently: rainbus.top
 * summary, Novelty; techwalker article, section 6). cos/sin are computed in
 * fp64 and rounded to fp32; the rotation is fp32 (each product and sum
 * rounded); the rotated values are rounded to bf16 and written to Qr, Kr
 * ([B,H,L,D] bf16, caller-owned). The block means of Qr, Kr and V are written
 * as in isa_pool_coarse. `ws` must hold plan.rope_bytes bytes of device
 * memory. Requires rope_base != 0 (ISA_ERR_ARG otherwise). */
ISA_API int isa_rope_pool_coarse(const isa_params_t* p, const void* Q, const void* K,
                                 const void* V, void* Qr, void* Kr, double* qc, double* kc,
                                 void* kc_bf16, void* vc_bf16, void* ws, size_t ws_bytes,
                                 void* stream);

/* Step (2): context importance r_j = sum over source query blocks i of
 * S[i, N_src + j] (computed as s * (sum_i Qc_i) . Kc_{N_src+j}) and the
 * top-k_ctx context blocks. Writes ctx_idx [B,H,k_ctx] (global block ids,
 * ascending) and, if non-NULL, ctx_score [B,H,N_ctx]. */
ISA_API int isa_ctx_topk(const isa_params_t* p, const double* qc, const double* kc,
                 int32_t* ctx_idx, double* ctx_score, void* stream);

/* Steps (1) coarse scores, (3) sharpness and split, (5) exact-set choice.
 * Needs qc, kc from isa_pool_coarse and ctx_idx from isa_ctx_topk. Writes
 * sharpness [B,H,N] (may be NULL), sharp_idx [B,H,n_sharp],
 * flat_idx [B,H,n_flat] and flat_exact_idx [B,H,n_flat,k_ns] (global ids,
 * rows ascending). The coarse scores are formed where they are used and
 * never stored as a whole; `ws` (at least plan.scores_bytes bytes of device
 * memory) holds the sharpness values when `sharpness` is NULL, then, when
 * N_kv > 640 (16 rows of J no longer fit LDS), the exact-set selection's row
 * scratch: 256 x 16 x N_kv fp64 (the rows of the flat blocks in flight,
 * independent of N). */
ISA_API int isa_sharpness_split(const isa_params_t* p, const double* qc, const double* kc,
                        const int32_t* ctx_idx, double* sharpness, int32_t* sharp_idx,
                        int32_t* flat_idx, int32_t* flat_exact_idx, void* ws, size_t ws_bytes,
                        void* stream);

/* Step (4): exact attention of every valid token of the sharp blocks over
 * the tokens of J. Writes only those rows of O. */
ISA_API int isa_sharp_attn(const isa_params_t* p, const void* Q, const void* K, const void* V,
                   const int32_t* ctx_idx, const int32_t* sharp_idx, void* O, void* stream);

/* Step (5): flat rows: exact attention over the tokens of E_i plus the
 * 0th-order Taylor terms of J \ E_i (Kc, Vc in bf16), one softmax
 * accumulator. Writes only the flat rows of O. */
ISA_API int isa_flat_taylor_attn(const isa_params_t* p, const void* Q, const void* K, const void* V,
                         const void* kc_bf16, const void* vc_bf16, const int32_t* ctx_idx,
                         const int32_t* flat_idx, const int32_t* flat_exact_idx, void* O,
                         void* stream);

/* Step (6) residual: adds gamma * O_coarse_i (see above) to every token row
 * of block i of O, in place (bf16, rounded to nearest even). Needs qc, kc
 * from isa_pool_coarse, vc_bf16 (the bf16 V means) and ctx_idx. `ws` must
 * hold plan.scores_bytes bytes of device memory (the coarse rows S[i, J]
 * are formed there). Does nothing when gamma == 0. */
ISA_API int isa_coarse_residual(const isa_params_t* p, const double* qc, const double* kc,
                                const void* vc_bf16, const int32_t* ctx_idx, void* O, void* ws,
                                size_t ws_bytes, void* stream);

/* Steps (1)-(6) enqueued back to back with no host synchronisation (with
 * the decoupled RoPE first when rope_base > 0). `ws` must hold
 * plan.workspace_bytes of device memory; `dbg` may be NULL. */
ISA_API int isa_forward(const isa_params_t* p, const void* Q, const void* K, const void* V, void* O,
                void* ws, size_t ws_bytes, const isa_debug_t* dbg, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops or harnesses that forbid hipMalloc): isa_forward
 * with the workspace taken from a device array inside the library,
 * ISA_NOALLOC_SCRATCH_BYTES bytes per device, instead of a caller buffer. The
 * caller still passes Q, K, V and O (and optional dbg buffers). The call
 * allocates nothing (no hipMalloc/hipFree; only kernels, plus copies when dbg
 * is given). Refused with ISA_ERR_SCRATCH when plan.noalloc_bytes exceeds
 * ISA_NOALLOC_SCRATCH_BYTES (e.g. B = 1, H = 40, D = 128, b = 64 fits up to
 * 16384 tokens). The row log-sum-exp is not saved, so isa_backward cannot
 * follow this call. Every call on one device shares that device's array:
 * calls that overlap in time on one device (different streams, or host
 * threads without ordering) race and give undefined results; calls ordered
 * on one stream are safe. Nothing in the array needs to start at zero (every
 * value a step reads was written by an earlier step of the same call). */
ISA_API int isa_forward_noalloc(const isa_params_t* p, const void* Q, const void* K,
                                const void* V, void* O, const isa_debug_t* dbg, void* stream);

/* Optional one-time set-up of the current device (see State above): raises
 * the kernels' dynamic-LDS limits and resolves the static scratch address.
 * Idempotent. Returns ISA_ERR_HIP when no device is usable. Calling it before
 * capturing library calls in a HIP graph makes the first captured call
 * equivalent to later ones. */
ISA_API int isa_init(void);

/* Backward pass (the operator is trainable end to end: rainbus.top summary,
 * Core method and Novelty (c)). Gradients of sum(dO * O) with respect to
 * Q, K, V, with every selection of the forward held fixed (they are piecewise
 * constant): the exact terms give the usual softmax-attention gradients; the
 * 0th-order Taylor terms reach K and V through the block means (each token of
 * block j receives 1/n_j of the gradient of Kc_j, Vc_j); tokens of pruned
 * context blocks get zero gradient; with gamma != 0 the residual
 * gamma * O_coarse adds its gradient through Qc, Kc, Vc. With rope_base != 0
 * the gradients are those of the unrotated Q and K (the transposed rotation
 * is applied).
 * Q, K, V: the inputs of the isa_forward call that filled `ws` (same
 * params), O its output, dO [B,H,L,D] bf16; writes dQ, dK, dV [B,H,L,D]
 * bf16 (caller-owned, every row written). `ws` must be that call's workspace,
 * unmodified since: the forward saved its selections, each row's softmax
 * log-sum-exp and the rotated Q, K there, and the backward uses the rest of
 * it as scratch. Deterministic (fixed summation orders, no float atomics). */
ISA_API int isa_backward(const isa_params_t* p, const void* Q, const void* K, const void* V,
                         const void* O, const void* dO, void* dQ, void* dK, void* dV,
                         void* ws, size_t ws_bytes, void* stream);

/* Dense baseline: O = softmax(Q K^T / sqrt(D)) V over all L tokens (no mask),
 * bf16 in/out, same tile engine as isa_sharp_attn. D in {64, 128},
 * B * H <= 65535 and L * D * 2 < 2^31 bytes per head (else
 * ISA_ERR_UNSUPPORTED). The
 * comparison line the pages measure ISA against (rainbus.top summary,
 * "Prerequisites", SDPA and FlashAttention paragraph). */
ISA_API int isa_dense_attn(int32_t B, int32_t H, int32_t L, int32_t D, const void* Q, const void* K,
                   const void* V, void* O, void* stream);

/* Static description of a status code. */
ISA_API const char* isa_strerror(int status);

#ifdef __cplusplus
}
#endif
#endif /* ISA_H */
