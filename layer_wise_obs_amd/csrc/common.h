// Shared definitions of the libthanos HIP sources (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/thanos.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

namespace th {

constexpr int kMaxBlock = 128;  // largest column block B the kernels tile for
constexpr int kSelBits = 11;    // radix-select digit width
constexpr int kSelBins = 1 << kSelBits;
constexpr int kSelCopies = 4;   // global histogram copies (workgroup i adds to copy i % 4)

// Device-side state of one th_prune_layer call (lives in the workspace).
struct DevState {
  unsigned long long prefix;   // resolved high bits of the threshold key
  unsigned long long tbound;   // selection: key < tbound
  long long rrem;              // rank still to find inside the current bucket
  long long pruned;            // weights pruned so far (all blocks)
  long long budget;            // k_total
  int shift;                   // bit position of the next digit
  int done;                    // threshold found for this block
  int not_spd;                 // a pivot was <= 0 or not finite
  int nonfinite;               // NaN/Inf met in W or diag(H)
  double lambda;               // absolute damping used
  double diag_mean;            // mean(diag(2G))
  int cand_state;              // candidate list: 0 not built, 1 valid, 2 not usable
  int cand_over;               // a workgroup's candidates did not fit its segment
  // Copies of the digit histogram, summed by the pick: a quarter of the
  // workgroups adds to each, so fewer atomics meet on one address.
  alignas(16) unsigned int hist[kSelCopies][kSelBins];
};
static_assert(offsetof(DevState, hist) % 16 == 0, "16-byte loads of the histogram");

// Score S = w^2 * g in fp32, with g = 1/[A_F]_qq (OBS) or G_qq (Wanda).
// One definition for every kernel that ranks weights, so that keys computed
// in different passes are bit-identical.
__device__ __forceinline__ float score_of(float w, float g) {
  float w2 = __fmul_rn(w, w);
  return __fmul_rn(w2, g);
}

// N:M selection: whether entry e is among the m-n lowest (score, column) of its
// aligned group of m in sc[] (ties: the lower column is pruned first).
__device__ __forceinline__ bool nm_pruned(const float* sc, int e, int n, int m) {
  const int g0 = (e / m) * m;
  const float se = sc[e];
  int rank = 0;
  for (int t = 0; t < m; ++t) {
    const int q = g0 + t;
    const float sq = sc[q];
    rank += (q != e) && ((sq < se) || (sq == se && q < e));
  }
  return rank < m - n;
}

__device__ __forceinline__ unsigned long long make_key(float s, unsigned int flat) {
  return ((unsigned long long)__float_as_uint(s) << 32) | (unsigned long long)flat;
}

__device__ __forceinline__ float bf16_to_f32(unsigned short h) {
  return __uint_as_float(((unsigned int)h) << 16);
}

__device__ __forceinline__ unsigned short f32_to_bf16_rne(float f) {
  unsigned int u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) {  // inf or nan
    return (unsigned short)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  }
  u += 0x7fffu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}

// Wave-level LDS ordering: every LDS access of this wave issued before the call
// has completed, and the compiler does not move LDS accesses across it.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_wave_barrier();
  __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E). Used where
// register arrays must be indexed by constants in fully unrolled code.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Value of v in lane `lane` (lane must be wave-uniform).
__device__ __forceinline__ float bcast(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------- launchers
// hessian.hip
int syrk_bf16_splits(int64_t t, int64_t b);
// workspace (floats) of the bf16 syrk for t tokens of b features: 0 when none helps
size_t syrk_bf16_workspace_floats(int64_t t, int64_t b);
hipError_t launch_syrk_bf16(float* H, const unsigned short* X, int64_t t, int64_t b, int64_t ldx,
                            float* partials, int splits, hipStream_t s);
// the 384 x 256 rectangles, whole tiles in rounds of P workgroups and the rest cut
// into m pieces each (m = 0: chosen); part holds syrk_rect_workspace_floats
size_t syrk_rect_workspace_floats(int64_t t, int64_t b, int P, int m);
hipError_t launch_syrk_rect(float* H, const unsigned short* X, int64_t t, int64_t b, int64_t ldx,
                            float* part, int P, int m, hipStream_t s, bool overwrite);
// H = 2 X^T X on the lower triangle (the rectangles write every lower entry;
// otherwise H is cleared first and accumulated into)
hipError_t launch_syrk_bf16_set(float* H, const unsigned short* X, int64_t t, int64_t b,
                                int64_t ldx, float* partials, int splits, hipStream_t s);
hipError_t launch_syrk_f32(float* H, const float* X, int64_t t, int64_t b, int64_t ldx,
                           hipStream_t s);
hipError_t launch_lambda(const float* H, int64_t b, double lam, int rel, int h_is_damped,
                         DevState* st, hipStream_t s);
hipError_t launch_damp_mirror(float* H, int64_t b, float lam, hipStream_t s);
hipError_t launch_flip_lower(const float* H, float* S, int64_t b, const DevState* st,
                             int add_lambda, hipStream_t s);
hipError_t launch_wanda_diag(const float* H, int64_t b, const DevState* st, int h_is_damped,
                             float* gdiag, hipStream_t s);

// baseline.hip
int colsq_splits(int64_t n);
hipError_t launch_column_sq_norms(const void* X, th_dtype xdt, int64_t n, int64_t b, int64_t ldx,
                                  double* part, float* g, hipStream_t s);
hipError_t launch_baseline_rows(void* W, th_dtype wdt, int64_t c, int64_t b, const float* g,
                                int64_t krow, uint8_t* mask, hipStream_t s);
hipError_t launch_baseline_nm(void* W, th_dtype wdt, int64_t c, int64_t b, const float* g, int n,
                              int m, uint8_t* mask, hipStream_t s);

// factor.hip
// panel: chol_panel_floats(b) floats. Part of the work runs on a library-owned
// stream of the current device, joined back into s before the call returns.
size_t chol_panel_floats(int64_t b);
hipError_t launch_chol_inv_inplace(float* S, int64_t b, float* panel, DevState* st,
                                   hipStream_t s);
// U = the reversal of S's lower triangle, zero below the diagonal: everywhere when
// zero_block is 0, else only inside the diagonal blocks of that size (what the
// per-block slices read; the rest of the strict lower triangle is left as is)
hipError_t launch_reverse(const float* S, float* U, int64_t b, int64_t zero_block, hipStream_t s);


// prep.hip
// The per-block preparation, for blocks jlo .. jhi-1 of size B:
hipError_t launch_save_diag_blocks(const float* U, int64_t b, int64_t B, float* Ublk, float* UblkT,
                                   int jlo, int jhi, hipStream_t s);
hipError_t launch_transform_rows(float* R, int64_t b, int64_t B, const float* UblkT, int jlo,
                                 int jhi, hipStream_t s);
// Dpart[r][q] = sum over rows i <= q of block r of U_iq^2 (fp64), then
// D[r][q] = 1 / sum_{r' >= r} Dpart[r'][q] once every block's part is in
hipError_t launch_colnorm_partial(const float* U, int64_t b, int64_t B, double* Dpart, int jlo,
                                  int jhi, hipStream_t s);
hipError_t launch_colnorm_scan(const double* Dpart, int64_t b, int64_t B, float* D, hipStream_t s);
// D[r][q] = sum_{i = rB .. q} U_iq^2 (fp64 sums); scratch (optional, e.g. the free
// S buffer) of at least ceil(b/B)*b doubles selects the two-pass coalesced version.
hipError_t launch_block_inverses(const float* Ublk, int64_t b, int64_t B, float* Nblk, int jlo,
                                 int jhi, hipStream_t s);

// select.hip
// budget += add_budget, then r = budget - pruned keys are to be found among ncand.
hipError_t launch_select_init(DevState* st, long long add_budget, long long ncand,
                              hipStream_t s);
// One radix pass over the keys of W[:, j0:j1) with score weights g, then the pick.
// Candidate list of the global selection: one segment of `quota` keys per
// workgroup of the pass grid, and a count per segment.
int64_t select_segments(int64_t c);
int64_t select_quota(int64_t c, int64_t b);
// cand / cand_n: select_segments(c) * quota keys and select_segments(c) counts, or
// nullptr (every pass then reads W).
hipError_t launch_select_pass(const float* W, int64_t c, int64_t b, int64_t j0, int64_t j1,
                              const float* g, DevState* st, hipStream_t s,
                              unsigned long long* cand = nullptr, unsigned int* cand_n = nullptr,
                              int64_t quota = 0);
hipError_t launch_select_pick(DevState* st, hipStream_t s);
hipError_t launch_select_scores_pass(const float* scores, int64_t c, int64_t f,
                                     int64_t b_full, int64_t j0, DevState* st, hipStream_t s);

// solve.hip
hipError_t launch_solve_nm(const float* W, int64_t c, int64_t b, int64_t j0, int64_t B, int n,
                           int m, const float* R, const float* gW, const float* Nblk, float* Z,
                           int64_t ldz, uint8_t* mask, DevState* st, unsigned long long* blk_count,
                           hipStream_t s);
// N:M with the group's block-local compensation folded in (route A and 4-aligned
// widths only: solve_nm_local_applies). Reads W[:, J] less Z[:, 0:j0-r0] R[r0:j0, J] (Z: the
// group's coefficients, whose first column belongs to block row r0), writes the
// block's final W[:, J], its mask and its coefficients Z[:, j0-r0 : j0-r0+B];
// with Wout, also the final W[:, J] in dtype wdt (c x b, row-major). group_end:
// the end column of the block's group (the next block's reads of R are prefetched
// when it lies inside).
bool solve_nm_local_applies(int64_t b, int64_t B, int n, int m);
hipError_t launch_solve_nm_local(float* W, int64_t c, int64_t b, int64_t j0, int64_t B, int n,
                                 int m, const float* R, const float* gW, float* Z, int64_t ldz,
                                 int64_t r0, uint8_t* mask, DevState* st,
                                 unsigned long long* blk_count, void* Wout, th_dtype wdt,
                                 int64_t group_end, hipStream_t s);
hipError_t launch_solve_unstructured(const float* W, int64_t c, int64_t b, int64_t j0, int64_t B,
                                     const float* R, const float* Nblk, const float* g,
                                     float* Z, uint8_t* mask, DevState* st,
                                     unsigned long long* blk_count, hipStream_t s);
hipError_t launch_debug_select_nm(const float* scores, int64_t c, int64_t blk, int n, int m,
                                  uint8_t* mask, hipStream_t s);
hipError_t launch_debug_mask_from_scores(const float* scores, int64_t c, int64_t f,
                                         int64_t b_full, int64_t j0, int64_t blk,
                                         const DevState* st, uint8_t* mask, int32_t* s_k,
                                         hipStream_t s);

// sparsegpt.hip
hipError_t launch_sgpt_gdiag(const float* U, int64_t b, float* g, hipStream_t s);
hipError_t launch_sgpt_errors(const float* W, int64_t c, int64_t b, int64_t j0, int64_t B, int n,
                              int m, int unstructured, const float* U, const float* g, float* E,
                              int64_t lde, uint8_t* mask, DevState* st,
                              unsigned long long* blk_count, hipStream_t s);

// ffn.hip
hipError_t launch_gated_ffn(const unsigned short* X, const unsigned short* Wg,
                            const unsigned short* Wu, unsigned short* Y, int64_t n, int64_t d,
                            int64_t f, hipStream_t s);

// rows.hip
hipError_t launch_row_energy(const void* W, th_dtype wdt, int64_t c, int64_t b, const float* g,
                             float* s, hipStream_t st);
hipError_t launch_row_index(const float* s, int64_t c, const DevState* sel, int32_t* idx,
                            int32_t* rowmap, uint8_t* dense_out, DevState* layer,
                            hipStream_t st);
hipError_t launch_gather_rows(const void* W, th_dtype wdt, int64_t b, const int32_t* rowmap,
                              int64_t cp, float* Wf, DevState* dst, hipStream_t st);
hipError_t launch_scatter_rows(void* W, th_dtype wdt, int64_t c, int64_t b, const int32_t* idx,
                               const float* Wf, const uint8_t* mc, float* Wout, uint8_t* mask,
                               hipStream_t st);

// update.hip
// W[:, col0:col_end) -= Z[:, 0:K] R[r0:r0+K, col0:col_end) (Z pitch ldz); entries of
// columns [mask_j0, mask_j0 + mask_w) with mask set are then zeroed. With hist set,
// the new values of columns >= hist_j0 also add the first radix digit of their
// selection keys (score_of(w, gn[col]), top 11 bits of the 64-bit key) to hist.
hipError_t launch_update(float* W, int64_t c, int64_t b, int64_t r0, int64_t K, int64_t ldz,
                         int64_t col0, int64_t col_end, const float* Z, const float* R,
                         const uint8_t* mask, int64_t mask_j0, int64_t mask_w, hipStream_t s,
                         const float* gn = nullptr, int64_t hist_j0 = 0,
                         unsigned int* hist = nullptr);
// Whether launch_update runs on 128 x 128 tiles (else 64 x 64) for this range.
bool update_large_tiles(int64_t c, int64_t col0, int64_t col_end);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);
// far_x3.hip: W[:, col0:col_end] -= Z[:, 0:K] R[r0:r0+K, col0:col_end] on operands
// split once into bf16 planes (Y: far_x3_elems(c, col_end - col0, K) bf16, the
// planes followed by the slots of tiles run in pieces)
bool far_x3_applies(int64_t c, int64_t ncols, int64_t K);
size_t far_x3_elems(int64_t c, int64_t ncols_max, int64_t K);
hipError_t launch_far_update(float* W, int64_t c, int64_t b, int64_t r0, int64_t K, int64_t ldz,
                             int64_t col0, int64_t col_end, const float* Z, const float* R,
                             unsigned short* Y, hipStream_t s);

hipError_t launch_to_f32(const void* src, th_dtype dt, int64_t count, float* dst,
                         DevState* st, hipStream_t s);
hipError_t launch_from_f32(const float* src, int64_t count, th_dtype dt, void* dst,
                           hipStream_t s);
hipError_t launch_diff_f32(const void* W, const void* What, th_dtype dt, int64_t count,
                           float* D, hipStream_t s);
hipError_t launch_quadform(const float* D, int64_t c, int64_t b, const float* G,
                           double* partials, int64_t* nparts, hipStream_t s);
hipError_t launch_sum_partials(const double* partials, int64_t n, double* out, hipStream_t s);

}  // namespace th
