/*
 * thanos.h -- C ABI of libthanos: block-wise multi-constraint pruning of one
 * linear layer (Thanos-style) on AMD Instinct MI355X (gfx950).
 *
 * Method sources (page titles and sections):
 *   [BLOG]  "Pruning LLMs with Thanos" (project blog post):
 *           "The layer-reconstruction lens" (objective ||WX - What X||_F^2,
 *           decomposition over rows), "One deletion with compensation: the OBS
 *           view" (damped Hessian, OBS update and cost), "Contribution one: solve
 *           a selected set directly" (joint update delta = -u Rhat^-1 R),
 *           "Contribution two: keep the budget global and the execution local"
 *           (dynamic residual budget), "Making irregular row masks batchable".
 *   [EXPL]  "Weight Pruning in Large Language Models: How SparseGPT, Wanda, and
 *           Semi-Structured 2:4 Sparsity ..." (explainer): "SparseGPT:
 *           Second-Order Reconstruction at Scale" (H = 2XX^T + lambda*I, one
 *           Cholesky of H^-1 per layer), "Wanda: Pruning by Weights and
 *           Activations", "N:M Semi-Structured Sparsity (2:4 Pattern)".
 *   [REPO]  "Thanos - Method of Pruning LLMs" (repository README), "Usage":
 *           --sparsity_ratio and --sparsity_type {unstructured, 2:4, 4:8}.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless the comment says "host".
 *   - Matrices are row-major. W is c x b (row = output channel, contiguous over
 *     the b inputs). X is b x n with tokens as columns; it is passed token-major
 *     as X^T [n, b] (the same bytes as column-major X), row pitch ldx elements.
 *   - The caller owns every buffer, including the workspace. The library never
 *     allocates device memory; the one entry point without a workspace argument
 *     (th_prune_layer_noalloc) uses a fixed array the library holds from load.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream).
 *     The factorisation of the Hessian also runs part of its work on a stream
 *     the library creates once per device and host thread (default priority);
 *     that work is joined back into `stream` with events, so everything the
 *     caller enqueues on `stream` afterwards sees the results.
 *     Entry points that return host values or a status that depends on device
 *     results synchronise that stream before returning.
 *   - Argument errors are reported before anything is launched. No C++
 *     exception crosses this interface. th_last_error() gives a message for the
 *     last non-OK status of the calling thread.
 *   - Calls that share a workspace or output buffers must not overlap.
 */
#ifndef THANOS_H_
#define THANOS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
typedef struct ihipStream_t* th_stream_t; /* identical to hipStream_t */

typedef enum {
  TH_OK = 0,
  TH_ERR_INVALID_ARG = 1, /* bad size, null pointer, unsupported combination */
  TH_ERR_NOT_SPD = 2,     /* the damped Hessian has a non-positive pivot */
  TH_ERR_NONFINITE = 3,   /* NaN/Inf in W or in the Hessian's diagonal */
  TH_ERR_WORKSPACE = 4,   /* workspace smaller than the size query returned */
  TH_ERR_HIP = 5          /* a HIP runtime call failed */
} th_status;

typedef enum { TH_F32 = 0, TH_BF16 = 1 } th_dtype;
typedef enum { TH_UNSTRUCTURED = 0, TH_NM = 1 } th_pattern_kind;
typedef enum { TH_SCORE_OBS = 0, TH_SCORE_WANDA = 1 } th_score;

typedef struct {
  int32_t kind; /* th_pattern_kind */
  int32_t n;    /* N:M: keep n of every m consecutive weights of a row */
  int32_t m;
} th_pattern;

typedef struct {
  /* Unstructured: fraction p in [0,1]; the layer loses
   * k_total = round-half-even(p*c*b) weights in total [BLOG, "Contribution two"].
   * N:M: ignored (the pattern fixes 1 - n/m), as with [REPO]'s --sparsity_ratio. */
  double sparsity;
  th_pattern pattern;
  /* Column block size B, 1 <= B <= 128. Blocks run left to right; finished
   * blocks are frozen [BLOG, "The scaling problem, and what SparseGPT changes"].
   * N:M needs m | B and m | b. */
  int64_t block;
  /* Damping: absolute lambda if lambda_is_relative == 0, else
   * lambda = lambda * mean(diag(2G)) (typical: 0.01, relative). */
  double lambda;
  int32_t lambda_is_relative;
  /* Score g_q in S_kq = W_kq^2 g_q: OBS g_q = 1/[(H_F)^-1]_qq over the active
   * columns F [BLOG, "One deletion with compensation"]; Wanda g_q = G_qq
   * ([EXPL, "Wanda"]; same ordering as |W| ||X_q||). */
  int32_t score;
} th_prune_params;

typedef struct {
  double lambda_used;    /* absolute damping that was applied (or derived, see below) */
  int64_t total_pruned;  /* number of weights set to zero */
  int64_t nblocks;       /* number of column blocks */
} th_stats;

/* H += 2 * X_chunk^T X_chunk on the lower triangle (entries with row >= column).
 * [EXPL, "SparseGPT: Second-Order Reconstruction at Scale"]: H = 2XX^T (+ lambda I
 * later). X_chunk: [t, b] token-major, dtype xdt (TH_BF16: products are exact in
 * fp32 and accumulate in fp32 on the matrix cores; TH_F32: fp32 FMA). ldx >= b
 * and, for TH_BF16, b % 8 == 0, ldx % 8 == 0 and a 16-byte aligned X. H: b x b fp32, zeroed by
 * the caller before the first chunk; the strict upper triangle is not touched.
 * workspace (optional, may be NULL with workspace_bytes 0; 16-byte aligned) lets
 * small b split the token range over more workgroups and large b run 384 x 256
 * tiles with the last round's tiles cut into token pieces; size from
 * th_hessian_workspace_size. The summation order is fixed, so repeated calls give
 * bit-identical H. Asynchronous. */
th_status th_hessian_accumulate(float* H, const void* X_chunk, th_dtype xdt, int64_t t,
                                int64_t b, int64_t ldx, void* workspace,
                                size_t workspace_bytes, th_stream_t stream);
th_status th_hessian_workspace_size(int64_t t, int64_t b, size_t* bytes /* host */);

/* Damping and symmetrisation of an accumulated H (= 2G on the lower triangle):
 * lambda = lambda_rel * mean(diag(H)) if lambda_is_relative else lambda;
 * H_qq += lambda; the upper triangle is overwritten by the mirror of the lower
 * [BLOG, "One deletion with compensation"]. *lambda_out (host, optional) gets the
 * absolute lambda. Synchronises the stream. */
th_status th_hessian_finalize(float* H, int64_t b, double lambda, int32_t lambda_is_relative,
                              double* lambda_out, th_stream_t stream);

/* Prune one layer [BLOG, "Contribution one" and "Contribution two"; N:M masks per
 * "The semi-structured N:M variant" paragraph of "Contribution two"].
 *   W [c,b] dtype wdt (TH_BF16 or TH_F32): read, then overwritten with What
 *     rounded to wdt (round-to-nearest-even for bf16).
 *   Exactly one of X / H is non-NULL:
 *     X [n,b] token-major (ldx = b), dtype xdt: H = 2XX^T + lambda*I is built
 *       inside (p->lambda, p->lambda_is_relative);
 *     H [b,b] fp32, full symmetric and already damped. If p->score is Wanda,
 *       G_qq is taken as (H_qq - lambda)/2 with lambda = p->lambda (absolute) or
 *       lambda_rel/(1+lambda_rel) * mean(diag H) (relative; exact for an H that
 *       th_hessian_finalize produced with the same lambda_rel).
 *   W_out_f32 [c,b] fp32 (optional): What in fp32.
 *   mask_out [c,b] uint8 (optional): 1 = pruned.
 *   workspace: >= th_prune_layer_workspace_size bytes, 256-byte aligned.
 *   stats_out (host, optional); block_counts (host, optional, nblocks entries):
 *     weights pruned in each block.
 * Returns TH_ERR_NOT_SPD if the Cholesky factorisation of the damped Hessian
 * meets a non-positive pivot, TH_ERR_NONFINITE for NaN/Inf in W or diag(H).
 * Synchronises the stream once, at the end. */
th_status th_prune_layer(void* W, th_dtype wdt, int64_t c, int64_t b, const void* X,
                         th_dtype xdt, int64_t n, const float* H, const th_prune_params* p,
                         float* W_out_f32, uint8_t* mask_out, void* workspace,
                         size_t workspace_bytes, th_stats* stats_out,
                         int64_t* block_counts, th_stream_t stream);
th_status th_prune_layer_workspace_size(int64_t c, int64_t b, int64_t n, int32_t have_x,
                                        const th_prune_params* p, size_t* bytes /* host */);

/* th_prune_layer without a workspace argument and without allocating, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation). Its device memory is one file-scope
 * array of TH_NOALLOC_SCRATCH_BYTES bytes that every GPU the library runs on holds
 * from the library's load until the process ends. th_prune_layer_workspace_size
 * bounds what a call needs (less when the caller passes W_out_f32 and mask_out):
 * square layers up to b = 1024 fit with X given, up to about b = 2000 with a
 * given H. Arguments,
 * results, synchronisation and errors as th_prune_layer; a layer that needs more
 * scratch returns TH_ERR_WORKSPACE before anything is launched. The first call on
 * a device (per host thread) looks up the array's address and creates the
 * factorisation's side stream and events; no call allocates memory. All calls on
 * one GPU share its array and every call clears what must start at zero: calls
 * that overlap on one GPU (other host threads, other streams) race and must not
 * be made. */
#define TH_NOALLOC_SCRATCH_BYTES (64u << 20)
th_status th_prune_layer_noalloc(void* W, th_dtype wdt, int64_t c, int64_t b, const void* X,
                                 th_dtype xdt, int64_t n, const float* H, const th_prune_params* p,
                                 float* W_out_f32, uint8_t* mask_out, th_stats* stats_out,
                                 int64_t* block_counts, th_stream_t stream);

/* Inverse factor of a damped Hessian, for layers that share one input (q/k/v,
 * gate/up): H^-1 = U^T U with U upper [EXPL, "SparseGPT: Second-Order
 * Reconstruction at Scale": one factorisation of the inverse Hessian per layer;
 * here per shared input]. Exactly one of X ([n,b] token-major, dtype xdt: H =
 * 2XX^T + lambda*I is built inside) / H ([b,b] fp32, full symmetric, already
 * damped) is non-NULL; lambda and lambda_is_relative as in th_prune_params.
 * U [b,b] fp32 (device, caller-owned): receives U, zero below the diagonal (with
 * X it also serves as the Hessian's scratch). *lambda_out (host, optional): the
 * absolute lambda, added (X given) or taken to be in a given H (lambda when
 * absolute, lambda/(1+lambda) * mean(diag H) when relative). workspace: >=
 * th_factor_workspace_size bytes, 256-byte aligned. Synchronises once.
 * TH_ERR_NOT_SPD / TH_ERR_NONFINITE as th_prune_layer. */
th_status th_factor(const void* X, th_dtype xdt, int64_t n, const float* H, int64_t b,
                    double lambda, int32_t lambda_is_relative, float* U, double* lambda_out,
                    void* workspace, size_t workspace_bytes, th_stream_t stream);
th_status th_factor_workspace_size(int64_t b, int64_t n, int32_t have_x, size_t* bytes /* host */);

/* th_prune_layer from a given factor U (th_factor's output; read only, copied
 * into the workspace): the same block loop, so the result is identical to
 * th_prune_layer on the H that U came from [BLOG, "Contribution one" and
 * "Contribution two"]. p->score must be TH_SCORE_OBS (the Wanda score needs
 * diag(H)); p->lambda is not used and stats_out->lambda_used is 0. Other
 * arguments, synchronisation and errors as th_prune_layer. workspace: >=
 * th_prune_layer_factored_workspace_size bytes. */
th_status th_prune_layer_factored(void* W, th_dtype wdt, int64_t c, int64_t b, const float* U,
                                  const th_prune_params* p, float* W_out_f32, uint8_t* mask_out,
                                  void* workspace, size_t workspace_bytes, th_stats* stats_out,
                                  int64_t* block_counts, th_stream_t stream);
th_status th_prune_layer_factored_workspace_size(int64_t c, int64_t b, const th_prune_params* p,
                                                 size_t* bytes /* host */);

/* The alpha variant: round-half-even(alpha*c) rows of W stay dense, the other
 * rows are pruned as a layer of their own [BLOG, "What the experiments show":
 * the alpha = 0.1 variant keeps 10% of the rows as outliers, so 50% becomes 45%].
 * Which rows is not on the pages; here the rows of largest output energy
 * s_k = sum_q W_kq^2 G_qq (fp64 sums, ranked by their fp32 value, ties to the
 * higher row index), with G_qq from X's column norms (th_column_sq_norms) or
 * from a given damped H as (H_qq - lambda)/2. Arguments as th_prune_layer, plus
 * alpha in [0, 1] and dense_rows_out [c] uint8 (device, optional): 1 = kept
 * dense. Dense rows are left unchanged (mask 0); block_counts and stats count
 * the pruned rows only. workspace: >= th_prune_layer_alpha_workspace_size
 * bytes. Synchronisation and errors as th_prune_layer (a non-finite weight in
 * any row gives TH_ERR_NONFINITE). */
th_status th_prune_layer_alpha(void* W, th_dtype wdt, int64_t c, int64_t b, const void* X,
                               th_dtype xdt, int64_t n, const float* H, const th_prune_params* p,
                               double alpha, float* W_out_f32, uint8_t* mask_out,
                               uint8_t* dense_rows_out, void* workspace, size_t workspace_bytes,
                               th_stats* stats_out, int64_t* block_counts, th_stream_t stream);
th_status th_prune_layer_alpha_workspace_size(int64_t c, int64_t b, int64_t n, int32_t have_x,
                                              const th_prune_params* p, double alpha,
                                              size_t* bytes /* host */);

/* Input of down_proj from a gated feed-forward: Y = silu(X W_gate^T) * (X W_up^T)
 * with silu(z) = z/(1+e^-z) [BLOG, "The compression target: linear layers":
 * feed-forward projections joined by a nonlinearity; gate/up/down as in LLaMA].
 * X [n,d] token-major, W_gate and W_up [f,d] row-major, Y [n,f]; all bf16 (dt
 * must be TH_BF16), device, caller-owned. Products on the bf16 matrix cores with
 * fp32 sums, silu and the product in fp32, Y rounded to nearest even. Needs
 * d % 8 == 0 and 16-byte aligned X, W_gate, W_up. Asynchronous on the stream. */
th_status th_gated_ffn_input(const void* X, const void* W_gate, const void* W_up, th_dtype dt,
                             int64_t n, int64_t d, int64_t f, void* Y, th_stream_t stream);

/* Comparator: the column-sequential schedule of SparseGPT on the same Hessian and
 * factor [BLOG, "The scaling problem, and what SparseGPT changes": left to right,
 * every row at once, finished columns frozen, compensation only into active
 * columns, masks refreshed per block; EXPL, "SparseGPT: Second-Order
 * Reconstruction at Scale": pruning w_kq subtracts (w_kq/[H^-1]_qq) times row q
 * of H^-1 over the active columns from the rest of row k]. With H^-1 = U^T U that
 * update is (w_kq/U_qq) U_{q,q:}. Mask of block J chosen at block start from the
 * score w_kq^2/U_qq^2 (the cost of deleting w_kq alone when column q is
 * processed): unstructured, the block's round-half-even(p*c*|J|) lowest
 * (score, flat index k*b+q) — an equal quota per block, unlike th_prune_layer's
 * global budget; N:M, the m-n lowest (score, column) of every aligned group.
 * Arguments, layout, ownership, synchronisation and errors as th_prune_layer;
 * p->score must be TH_SCORE_OBS (else TH_ERR_INVALID_ARG). workspace: >=
 * th_prune_sparsegpt_workspace_size bytes, 256-byte aligned. block_counts get
 * the weights pruned in each block. */
th_status th_prune_sparsegpt(void* W, th_dtype wdt, int64_t c, int64_t b, const void* X,
                             th_dtype xdt, int64_t n, const float* H, const th_prune_params* p,
                             float* W_out_f32, uint8_t* mask_out, void* workspace,
                             size_t workspace_bytes, th_stats* stats_out,
                             int64_t* block_counts, th_stream_t stream);
th_status th_prune_sparsegpt_workspace_size(int64_t c, int64_t b, int64_t n, int32_t have_x,
                                            const th_prune_params* p, size_t* bytes /* host */);

/* E = ||(W - What) X||_F^2 = sum_k D_k G D_k^T and E / ||W X||_F^2
 * [BLOG, "The layer-reconstruction lens"]. W and What: [c,b] dtype wdt. Exactly
 * one of X ([n,b] token-major, dtype xdt) or G ([b,b] fp32, full symmetric,
 * undamped XX^T) is non-NULL. Products on the fp32 matrix cores, sums in fp64.
 * err_out, rel_err_out: host. Synchronises the stream. */
th_status th_reconstruction_error(const void* W, const void* What, th_dtype wdt, int64_t c,
                                  int64_t b, const void* X, th_dtype xdt, int64_t n,
                                  const float* G, void* workspace, size_t workspace_bytes,
                                  double* err_out, double* rel_err_out, th_stream_t stream);
th_status th_reconstruction_error_workspace_size(int64_t c, int64_t b, int32_t have_x,
                                                 size_t* bytes /* host */);

/* ---- Entry points for parity tests: one step of the path on given inputs ---- */

/* N:M selection on given scores [c, blk] fp32: in every aligned group of m
 * columns, mark the m-n lowest (score, column) pairs (ties: lower column first)
 * [BLOG, "The compression target: linear layers"; EXPL, "N:M ..."].
 * mask_blk [c, blk] uint8, 1 = pruned. Asynchronous. */
th_status th_debug_select_nm(const float* scores, int64_t c, int64_t blk, int32_t n, int32_t m,
                             uint8_t* mask_blk, th_stream_t stream);

/* Global residual-budget selection on given scores [c, f] fp32 (f = b_full - j0
 * active columns, row pitch f): the r lowest keys (score, k*b_full + j0 + q)
 * form the candidate set; mask_blk [c, blk] (uint8, row pitch blk) gets the
 * candidates in the first blk columns, s_k [c] (int32, optional) their count per
 * row [BLOG, "Contribution two"]. workspace: >= 64 KiB. Synchronises. */
th_status th_debug_select_global(const float* scores, int64_t c, int64_t f, int64_t b_full,
                                 int64_t j0, int64_t blk, int64_t r, uint8_t* mask_blk,
                                 int32_t* s_k, void* workspace, size_t workspace_bytes,
                                 th_stream_t stream);

/* ---- Comparators without compensation ------------------------------------
 * [EXPL, "Wanda: Pruning by Weights and Activations"]: score |W_kq| * ||X_q||_2,
 * thresholds computed per output row, no update of the remaining weights.
 * [EXPL, "The Failure of Magnitude Pruning in Large Transformers"]: rank by
 * |W_kq| and remove the smallest (compared here per output row, like Wanda).
 * [BLOG, "Why magnitude alone misses important weights"]: W_kq^2 G_qq (G = X X^T)
 * orders like the Wanda score. [EXPL, "N:M Semi-Structured Sparsity (2:4
 * Pattern)"]: both enforce the pattern within every aligned group of m. */
typedef enum { TH_BASE_MAGNITUDE = 0, TH_BASE_WANDA = 1 } th_baseline;

/* gdiag[q] = G_qq = sum_t X_tq^2 (fp64 accumulation in a fixed order, rounded to
 * fp32). X token-major [n, b] (row pitch ldx >= b), bf16 or fp32; gdiag: b floats.
 * workspace (device) >= th_column_sq_norms_workspace_size bytes. Asynchronous. */
th_status th_column_sq_norms_workspace_size(int64_t n, int64_t b, size_t* bytes /* host */);
th_status th_column_sq_norms(const void* X, th_dtype xdt, int64_t n, int64_t b, int64_t ldx,
                             float* gdiag, void* workspace, size_t workspace_bytes,
                             th_stream_t stream);

/* Prune W (c x b, bf16 or fp32) in place: the pruned entries become exactly 0,
 * every other entry is left unchanged. Key of (k, q): w^2 rounded to fp32, times
 * gdiag[q] (Wanda; gdiag required, device, b floats) or times 1 (magnitude;
 * gdiag ignored), rounded to fp32; among equal keys the lower column is pruned
 * first. Unstructured (p->pattern.kind): every row loses its round-half-even(
 * p->sparsity * b) smallest keys. N:M: in every aligned group of m along a row,
 * the m-n smallest (1 <= m <= 128, m | b). p->block, lambda and score are not
 * used. mask_out (optional, device, c x b uint8): 1 = pruned. Asynchronous. */
th_status th_prune_baseline(void* W, th_dtype wdt, int64_t c, int64_t b, th_baseline method,
                            const float* gdiag, const th_prune_params* p, uint8_t* mask_out,
                            th_stream_t stream);

/* U = upper-triangular factor with H^-1 = U^T U (U = chol_upper(H^-1), the factor
 * [EXPL, "SparseGPT"] computes once per layer), from a damped, full symmetric H
 * [b,b] fp32. U [b,b] fp32 (strict lower triangle zero). workspace: >= b*b*4 +
 * 2*ceil(b/128)*128*256*4 + 2*2*3*256*ceil(b/256)*256 + 65536 bytes
 * (TH_ERR_WORKSPACE if smaller). Returns
 * TH_ERR_NOT_SPD on a non-positive pivot.
 * Synchronises. */
th_status th_debug_factor(const float* H, int64_t b, float* U, void* workspace,
                          size_t workspace_bytes, th_stream_t stream);

/* H += 2 X^T X on the lower triangle through the 384 x 256 rectangles that
 * th_hessian_accumulate takes for large layers (bf16 X, [EXPL, "SparseGPT:
 * Second-Order Reconstruction at Scale"]), with the work split fixed here
 * instead of by the device: whole tiles in rounds of P workgroups, each remaining
 * tile cut into m pieces of consecutive 32-token stages whose sums are added in a
 * fixed order (m = 0: chosen as for the device's compute units; m = 1: those
 * tiles whole as well). Arguments as th_hessian_accumulate with t >= 32 and
 * ldx < 2^25; 1 <= P <= 4096, 0 <= m <= t / 32; workspace: >= (number of cut
 * tiles) * (m * 98304 + 1) * 4 bytes (TH_ERR_WORKSPACE if smaller;
 * ceil(b/384) * ceil(b/256) * (m * 98304 + 1) * 4 always suffices), 16-byte
 * aligned. Asynchronous. */
th_status th_debug_syrk_rect(float* H, const void* X_chunk, int64_t t, int64_t b, int64_t ldx,
                             int32_t P, int32_t m, void* workspace, size_t workspace_bytes,
                             th_stream_t stream);

/* W[:, col0:col_end] -= Z[:, 0:K] R[r0:r0+K, col0:col_end] on operands split once into
 * three bf16 planes and 256 x 256 tiles, the update the N:M block loop applies to
 * the columns past each group of eight blocks ["Pruning LLMs with Thanos", section
 * "Contribution one: solve a selected set directly": every block's compensation
 * reaches all still-active columns]. W [c, b] fp32 (pitch b), Z [c, ldz] fp32,
 * R [>= r0+K, b] fp32, all device. K % 16 == 0, 0 <= col0 < col_end <= b, ldz >= K.
 * The tiles of a last, partial round of one workgroup per compute unit run in
 * pieces of consecutive k stages whose sums are subtracted in a fixed order.
 * workspace: the split planes, Y = 3 * ceil(K/64)*64 * (ceil(c/256) +
 * ceil((col_end-col0)/256)) * 256 * 2 bytes rounded up to a multiple of 256, then
 * 256 piece slots of 256 KB: >= Y + 67108864 bytes (TH_ERR_WORKSPACE if smaller),
 * 16-byte aligned. Asynchronous. */
th_status th_debug_far_update(float* W, int64_t c, int64_t b, const float* Z, int64_t ldz,
                              const float* R, int64_t r0, int64_t K, int64_t col0,
                              int64_t col_end, void* workspace, size_t workspace_bytes,
                              th_stream_t stream);

/* Message for the last non-OK status on this thread (never NULL). */
const char* th_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* THANOS_H_ */
