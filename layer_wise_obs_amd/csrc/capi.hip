// C ABI of libthanos: argument checks, workspace layout and the per-layer host sequence.
//
// th_prune_layer runs the whole per-layer path on one stream:
//   Hessian (X given):  H = 2 X^T X (lower)  -> lambda on the device
//   factor:             S = P H P (+lambda), in-place Cholesky + inverse, U = reverse(S)
//   slices:             Ublk, [D], [N], R[J,F] = U_JJ^T U[J,F]
//   block loop (left to right, "Pruning LLMs with Thanos", section "The scaling
//   problem, and what SparseGPT changes"):
//       unstructured: threshold by radix select over F, solve, update W[:, F]
//       N:M:          select + solve in one kernel, update W[:, J .. end of the
//                     super-block]; the rest of F once per super-block
//   output:             What cast back to the input dtype
// th_prune_sparsegpt (comparator) shares the Hessian and the factor, then runs the
// column-sequential schedule: per block a block-local mask, the per-row error
// recurrence, and the same update GEMM with U in place of the slices.
// The budget, the threshold and every count stay on the device; the host
// synchronises once, at the end, to read the status flags.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"

using namespace th;

namespace {

thread_local std::string g_last_error = "no error";

th_status fail(th_status s, const char* msg) {
  g_last_error = msg;
  return s;
}

th_status hip_fail(hipError_t e, const char* where) {
  g_last_error = std::string(where) + ": " + hipGetErrorString(e);
  return TH_ERR_HIP;
}

#define TH_HIP(call, where)                      \
  do {                                           \
    hipError_t e_ = (call);                      \
    if (e_ != hipSuccess) return hip_fail(e_, where); \
  } while (0)

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* p) : base((char*)p) {}
  template <class T>
  T* take(size_t count) {
    T* p = base ? (T*)(base + off) : nullptr;
    off = align256(off + count * sizeof(T));
    return p;
  }
};

struct PruneLayout {
  DevState* st;
  unsigned long long* counts;
  float* S;
  float* R;
  float* P;
  float* Ublk;
  float* UblkT;
  float* Nblk;
  float* D;
  double* Dpart;  // per-block parts of D's column sums (fp64)
  float* gW;
  float* Z;
  float* Wf;
  uint8_t* mask;
  float* syrk_part;
  unsigned short* Yfar;      // N:M: the far-column update's split operands
  unsigned long long* cand;  // unstructured: candidate keys of the selection
  unsigned int* cand_n;      // and their count per segment
  int64_t cand_quota;        // keys per segment
  size_t bytes;
};

// N:M masks depend only on the block's own columns, so a block's compensation
// of columns beyond its super-block (kSuperBlocks consecutive blocks) can wait:
// it is applied once per super-block as one GEMM with K = kSuperBlocks * B.
constexpr int64_t kSuperBlocks = 8;

int64_t super_pitch(int64_t b, int64_t B) {
  const int64_t full = cdiv(b, B) * B;
  const int64_t sb = kSuperBlocks * B;
  return full < sb ? full : sb;
}

int64_t z_pitch(int64_t b, const th_prune_params* p) {
  if (p->pattern.kind != TH_NM) return p->block;
  return super_pitch(b, p->block);
}

bool needs_complement(const th_prune_params* p) {
  if (p->block <= 64) return false;
  if (p->pattern.kind == TH_UNSTRUCTURED) return true;
  return (p->block / p->pattern.m) * (p->pattern.m - p->pattern.n) > 64;
}

// sgpt: the column-sequential comparator's layout (U only, no slices; gW holds the
// score weights 1/U_qq^2; E in Z with the super-block pitch for both patterns).
// factor: false when U is given (no panel buffer).
PruneLayout layout_prune(void* ws, int64_t c, int64_t b, int64_t n, bool have_x,
                         const th_prune_params* p, bool need_wf, bool need_mask, th_dtype xdt,
                         bool sgpt = false, bool factor = true) {
  Carve cv(ws);
  PruneLayout L;
  const int64_t B = p->block;
  const int64_t nblk = cdiv(b, B);
  L.st = cv.take<DevState>(1);
  L.counts = cv.take<unsigned long long>(nblk);
  L.S = cv.take<float>((size_t)b * b);
  L.R = cv.take<float>((size_t)b * b);
  L.P = factor ? cv.take<float>(chol_panel_floats(b)) : nullptr;
  L.Ublk = sgpt ? nullptr : cv.take<float>((size_t)nblk * B * B);
  L.UblkT = sgpt ? nullptr : cv.take<float>((size_t)nblk * B * B);
  L.Nblk = (!sgpt && needs_complement(p)) ? cv.take<float>((size_t)nblk * B * B) : nullptr;
  const bool unstr = p->pattern.kind == TH_UNSTRUCTURED;
  const bool colnorm = !sgpt && unstr && p->score == TH_SCORE_OBS;
  L.D = colnorm ? cv.take<float>((size_t)nblk * b) : nullptr;
  L.Dpart = colnorm ? cv.take<double>((size_t)nblk * b) : nullptr;
  L.gW = (sgpt || p->score == TH_SCORE_WANDA) ? cv.take<float>((size_t)b) : nullptr;
  L.Z = cv.take<float>((size_t)c * (sgpt ? super_pitch(b, B) : z_pitch(b, p)));
  // the first group's far columns are the widest
  const int64_t ldz = sgpt ? 0 : z_pitch(b, p);
  L.Yfar = (!sgpt && !unstr && b > ldz && far_x3_applies(c, b - ldz, ldz))
               ? cv.take<unsigned short>(far_x3_elems(c, b - ldz, ldz))
               : nullptr;
  L.Wf = need_wf ? cv.take<float>((size_t)c * b) : nullptr;
  L.mask = need_mask ? cv.take<uint8_t>((size_t)c * b) : nullptr;
  L.cand = nullptr;
  L.cand_n = nullptr;
  L.cand_quota = 0;
  if (!sgpt && unstr) {
    L.cand_quota = select_quota(c, b);
    L.cand = cv.take<unsigned long long>((size_t)(select_segments(c) * L.cand_quota));
    L.cand_n = cv.take<unsigned int>((size_t)select_segments(c));
  }
  L.syrk_part = nullptr;
  if (have_x && xdt == TH_BF16) {
    const size_t nf = syrk_bf16_workspace_floats(n, b);
    if (nf > 0) L.syrk_part = cv.take<float>(nf);
  }
  L.bytes = cv.off;
  return L;
}

th_status check_params(int64_t c, int64_t b, const th_prune_params* p) {
  if (!p) return fail(TH_ERR_INVALID_ARG, "params is NULL");
  if (c < 1 || b < 1) return fail(TH_ERR_INVALID_ARG, "c and b must be >= 1");
  if (c * b >= (int64_t)1 << 32) return fail(TH_ERR_INVALID_ARG, "c*b must be < 2^32");
  if (p->block < 1 || p->block > kMaxBlock)
    return fail(TH_ERR_INVALID_ARG, "block must be in [1, 128]");
  if (p->score != TH_SCORE_OBS && p->score != TH_SCORE_WANDA)
    return fail(TH_ERR_INVALID_ARG, "unknown score");
  if (p->pattern.kind == TH_UNSTRUCTURED) {
    if (!(p->sparsity >= 0.0 && p->sparsity <= 1.0))
      return fail(TH_ERR_INVALID_ARG, "sparsity must be in [0, 1]");
  } else if (p->pattern.kind == TH_NM) {
    const int n = p->pattern.n, m = p->pattern.m;
    if (m < 1 || n < 0 || n > m) return fail(TH_ERR_INVALID_ARG, "N:M needs 0 <= n <= m, m >= 1");
    if (p->block % m || b % m) return fail(TH_ERR_INVALID_ARG, "N:M needs m | block and m | b");
  } else {
    return fail(TH_ERR_INVALID_ARG, "unknown pattern kind");
  }
  if (!(p->lambda >= 0.0) || !std::isfinite(p->lambda))
    return fail(TH_ERR_INVALID_ARG, "lambda must be finite and >= 0");
  return TH_OK;
}

bool dtype_ok(th_dtype d) { return d == TH_F32 || d == TH_BF16; }

// Stands for "no workspace argument" in the shared checks (the allocation-free
// entry point brings its own); never dereferenced.
const char kNoWorkspaceTag = 0;
const void* const kNoWorkspace = &kNoWorkspaceTag;

// Checks shared by the layer entry points (before anything is enqueued).
th_status check_layer_args(const void* W, th_dtype wdt, int64_t c, int64_t b, const void* X,
                           th_dtype xdt, int64_t n, const float* H, const th_prune_params* p,
                           const void* workspace) {
  th_status chk = check_params(c, b, p);
  if (chk != TH_OK) return chk;
  if (!W) return fail(TH_ERR_INVALID_ARG, "W is NULL");
  if ((X == nullptr) == (H == nullptr)) return fail(TH_ERR_INVALID_ARG, "pass exactly one of X, H");
  if (!dtype_ok(wdt) || (X && !dtype_ok(xdt))) return fail(TH_ERR_INVALID_ARG, "unknown dtype");
  if (X && n < 1) return fail(TH_ERR_INVALID_ARG, "n must be >= 1");
  if (X && xdt == TH_BF16 && (b % 8 || ((uintptr_t)X & 15)))
    return fail(TH_ERR_INVALID_ARG, "bf16 X needs b % 8 == 0 and 16-byte alignment");
  if (workspace == kNoWorkspace) return TH_OK;
  if (!workspace) return fail(TH_ERR_INVALID_ARG, "workspace is NULL");
  if ((uintptr_t)workspace & 255) return fail(TH_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return TH_OK;
}

th_status accumulate_into(float* H, const void* X, th_dtype xdt, int64_t t, int64_t b,
                          int64_t ldx, float* part, hipStream_t s) {
  if (xdt == TH_BF16) {
    const int splits = part ? syrk_bf16_splits(t, b) : 1;
    TH_HIP(launch_syrk_bf16(H, (const unsigned short*)X, t, b, ldx, part, splits, s), "syrk_bf16");
  } else {
    TH_HIP(launch_syrk_f32(H, (const float*)X, t, b, ldx, s), "syrk_f32");
  }
  return TH_OK;
}

// Damped H (from X through the syrk, or given), its flipped lower triangle in S,
// then U with H^-1 = U^T U in R (in-place Cholesky and inverse of S, reversed).
// Wanda's G_qq goes to L.gW when the score asks for it.
// The per-block slices of U (in R) for blocks jlo .. jhi-1: the diagonal blocks
// (and their transposes), the column norms' parts and the block inverses when the
// layer needs them, then the transformed rows R[J, F] = U_JJ^T U[J, F] in place.
// Each block reads and writes only its own rows of R.
hipError_t slices_for(const PruneLayout& L, int64_t b, int64_t B, int jlo, int jhi,
                      hipStream_t s) {
  hipError_t e = launch_save_diag_blocks(L.R, b, B, L.Ublk, L.UblkT, jlo, jhi, s);
  if (e == hipSuccess && L.D) e = launch_colnorm_partial(L.R, b, B, L.Dpart, jlo, jhi, s);
  if (e == hipSuccess && L.Nblk) e = launch_block_inverses(L.Ublk, b, B, L.Nblk, jlo, jhi, s);
  if (e == hipSuccess) e = launch_transform_rows(L.R, b, B, L.UblkT, jlo, jhi, s);
  return e;
}

// zero_block: 0 leaves U exactly upper triangular in R; B (the block loop's block
// size) zeroes below the diagonal only inside the diagonal blocks, all that the
// per-block slices read, and prepares those slices too.
th_status inverse_factor(const void* X, th_dtype xdt, int64_t n, const float* H, int64_t b,
                         const th_prune_params* p, const PruneLayout& L, hipStream_t s,
                         int64_t zero_block) {
  const bool obs = p->score == TH_SCORE_OBS;
  if (X) {
    float* Hb = L.R;  // R is free until the factor is reversed into it
    if (xdt == TH_BF16) {
      const int splits = L.syrk_part ? syrk_bf16_splits(n, b) : 1;
      TH_HIP(launch_syrk_bf16_set(Hb, (const unsigned short*)X, n, b, b, L.syrk_part, splits, s),
             "syrk_bf16");
    } else {
      TH_HIP(launch_zero(Hb, (size_t)b * b * sizeof(float), s), "clear H");
      th_status a = accumulate_into(Hb, X, xdt, n, b, b, L.syrk_part, s);
      if (a != TH_OK) return a;
    }
    TH_HIP(launch_lambda(Hb, b, p->lambda, p->lambda_is_relative, 0, L.st, s), "lambda");
    if (!obs) TH_HIP(launch_wanda_diag(Hb, b, L.st, 0, L.gW, s), "wanda diag");
    TH_HIP(launch_flip_lower(Hb, L.S, b, L.st, 1, s), "flip");
  } else {
    TH_HIP(launch_lambda(H, b, p->lambda, p->lambda_is_relative, 1, L.st, s), "lambda");
    if (!obs) TH_HIP(launch_wanda_diag(H, b, L.st, 1, L.gW, s), "wanda diag");
    TH_HIP(launch_flip_lower(H, L.S, b, L.st, 0, s), "flip");
  }
  if (zero_block == 0) {
    TH_HIP(launch_chol_inv_inplace(L.S, b, L.P, L.st, s), "cholesky/inverse");
    TH_HIP(launch_reverse(L.S, L.R, b, 0, s), "reverse");
    return TH_OK;
  }
  TH_HIP(launch_chol_inv_inplace(L.S, b, L.P, L.st, s), "cholesky/inverse");
  TH_HIP(launch_reverse(L.S, L.R, b, zero_block, s), "reverse");
  TH_HIP(slices_for(L, b, zero_block, 0, (int)cdiv(b, zero_block), s), "slices");
  return TH_OK;
}

// The one synchronisation of a layer call: device state and per-block counts to
// the host, then the status flags.
th_status finish_layer(const PruneLayout& L, int64_t nblk, th_stats* stats_out,
                       int64_t* block_counts, hipStream_t s) {
  DevState host;
  TH_HIP(hipMemcpyAsync(&host, L.st, offsetof(DevState, hist), hipMemcpyDeviceToHost, s), "state");
  // counts are non-negative and below 2^63: the same bytes as int64_t
  static_assert(sizeof(unsigned long long) == sizeof(int64_t), "count width");
  if (block_counts)
    TH_HIP(hipMemcpyAsync(block_counts, L.counts, nblk * sizeof(unsigned long long),
                          hipMemcpyDeviceToHost, s),
           "counts");
  TH_HIP(hipStreamSynchronize(s), "sync");
  if (stats_out) {
    stats_out->lambda_used = host.lambda;
    stats_out->total_pruned = host.pruned;
    stats_out->nblocks = nblk;
  }
  if (host.nonfinite) return fail(TH_ERR_NONFINITE, "non-finite value in W or diag(H)");
  if (host.not_spd) return fail(TH_ERR_NOT_SPD, "damped Hessian is not positive definite");
  return TH_OK;
}

// Cleared device state (budget 0) and counts, W in fp32.
th_status begin_layer(const PruneLayout& L, const void* W, th_dtype wdt, int64_t c, int64_t b,
                      const th_prune_params* p, float* Wf, hipStream_t s) {
  const int64_t nblk = cdiv(b, p->block);
  TH_HIP(launch_zero(L.st, sizeof(DevState), s), "clear state");
  TH_HIP(launch_zero(L.counts, nblk * sizeof(unsigned long long), s), "clear counts");
  TH_HIP(launch_to_f32(W, wdt, c * b, Wf, L.st, s), "W to fp32");
  return TH_OK;
}

// The per-block slices of U (in L.R) and the block loop: What in Wf, the mask,
// per-block counts and the pruned total in the device state.
// prepared: inverse_factor (with zero_block = B) has already made the slices.
th_status prune_blocks(const PruneLayout& L, int64_t c, int64_t b, const th_prune_params* p,
                       float* Wf, uint8_t* mask, hipStream_t s, bool prepared,
                       void* Wout = nullptr, th_dtype wdt = TH_F32, bool* cast_done = nullptr) {
  const int64_t B = p->block;
  const int64_t nblk = cdiv(b, B);
  const bool unstr = p->pattern.kind == TH_UNSTRUCTURED;
  const bool obs = p->score == TH_SCORE_OBS;
  if (!prepared) TH_HIP(slices_for(L, b, B, 0, (int)nblk, s), "slices");
  if (L.D) TH_HIP(launch_colnorm_scan(L.Dpart, b, B, L.D, s), "column norms");

  const int64_t ldz = z_pitch(b, p);
  // the layer's budget k_total = round-half-even(p c b) joins at the first block
  const long long k_total = unstr ? (long long)std::nearbyint(p->sparsity * (double)c * (double)b) : 0;
  bool next_digit_done = false;  // the previous update counted this block's first digit
  // N:M with at most 64 pruned per block row (every block takes route A): the
  // block-local compensation runs inside the solve (one launch per block)
  const bool local = !unstr && solve_nm_local_applies(b, B, p->pattern.n, p->pattern.m);
  // there every block's solve writes its final columns, in the output dtype too
  if (cast_done) *cast_done = local && Wout;
  for (int64_t blk = 0; blk < nblk; ++blk) {
    const int64_t j0 = blk * B;
    const int64_t Bb = (b - j0) < B ? (b - j0) : B;
    const float* Nb = L.Nblk ? L.Nblk + blk * B * B : nullptr;
    if (unstr) {
      // the global selection scores every active column, so W[:, F] is updated in full
      const float* g = obs ? L.D + blk * b : L.gW;
      int first_pass = 0;
      if (!next_digit_done) {
        TH_HIP(launch_select_init(L.st, blk == 0 ? k_total : 0, (long long)(c * (b - j0)), s),
               "select init");
      } else {
        // this block's selection was set up before the previous block's update, which
        // also counted the first digit of its keys: the first pick needs no pass
        TH_HIP(launch_select_pick(L.st, s), "select pick");
        first_pass = 1;
      }
      for (int pass = first_pass; pass < 6; ++pass) {
        TH_HIP(launch_select_pass(Wf, c, b, j0, b, g, L.st, s, L.cand, L.cand_n, L.cand_quota),
               "select pass");
        TH_HIP(launch_select_pick(L.st, s), "select pick");
      }
      TH_HIP(launch_solve_unstructured(Wf, c, b, j0, B, L.R, Nb, g, L.Z, mask, L.st,
                                       L.counts + blk, s),
             "solve");
      const int64_t jn = j0 + Bb;  // the next block's active region starts here
      // On 128 x 128 tiles the update also counts the first key digit of the next
      // block (it writes all of that block's active region); on the small 64 x 64
      // tiles of the late blocks a separate pass is cheaper.
      next_digit_done = jn < b && update_large_tiles(c, j0, b);
      if (next_digit_done) {
        // after the solve (it reads this block's threshold and adds to the pruned
        // count), before the update that fills the histogram
        TH_HIP(launch_select_init(L.st, 0, (long long)(c * (b - jn)), s), "select init");
        unsigned int* hist = (unsigned int*)((char*)L.st + offsetof(DevState, hist));
        TH_HIP(launch_update(Wf, c, b, j0, Bb, B, j0, b, L.Z, L.R, mask, j0, Bb, s,
                             obs ? L.D + (blk + 1) * b : L.gW, jn, hist),
               "update");
      } else {
        TH_HIP(launch_update(Wf, c, b, j0, Bb, B, j0, b, L.Z, L.R, mask, j0, Bb, s), "update");
      }
    } else {
      const int64_t per = ldz / B;  // blocks per super-block
      const int64_t sb0 = (blk / per) * ldz;
      const int64_t s1 = (sb0 + ldz) < b ? (sb0 + ldz) : b;
      float* Zb = L.Z + (blk % per) * B;
      if (local) {
        // left-looking inside the group: the solve subtracts the earlier blocks'
        // compensation from its rows first and writes the block's final weights
        TH_HIP(launch_solve_nm_local(Wf, c, b, j0, B, p->pattern.n, p->pattern.m, L.R,
                                     obs ? nullptr : L.gW, Zb, ldz, sb0, mask, L.st,
                                     L.counts + blk, Wout, wdt, s1, s),
               "solve");
      } else {
        TH_HIP(launch_solve_nm(Wf, c, b, j0, B, p->pattern.n, p->pattern.m, L.R,
                               obs ? nullptr : L.gW, Nb, Zb, ldz, mask, L.st, L.counts + blk, s),
               "solve");
        TH_HIP(launch_update(Wf, c, b, j0, Bb, ldz, j0, s1, Zb, L.R, mask, j0, Bb, s), "update");
      }
      if (j0 + Bb == s1 && s1 < b) {  // last block of the super-block: the deferred columns
        if (L.Yfar && far_x3_applies(c, b - s1, s1 - sb0))
          TH_HIP(launch_far_update(Wf, c, b, sb0, s1 - sb0, ldz, s1, b, L.Z, L.R, L.Yfar, s),
                 "deferred update");
        else
          TH_HIP(launch_update(Wf, c, b, sb0, s1 - sb0, ldz, s1, b, L.Z, L.R, mask, 0, 0, s),
                 "deferred update");
      }
    }
  }
  return TH_OK;
}

}  // namespace

extern "C" {

const char* th_last_error(void) { return g_last_error.c_str(); }

th_status th_hessian_workspace_size(int64_t t, int64_t b, size_t* bytes) {
  if (!bytes || t < 0 || b < 1) return fail(TH_ERR_INVALID_ARG, "bad arguments");
  *bytes = syrk_bf16_workspace_floats(t, b) * sizeof(float);
  return TH_OK;
}

th_status th_hessian_accumulate(float* H, const void* X, th_dtype xdt, int64_t t, int64_t b,
                                int64_t ldx, void* workspace, size_t workspace_bytes,
                                th_stream_t stream) {
  if (!H || !X) return fail(TH_ERR_INVALID_ARG, "H and X must be non-NULL");
  if (t < 0 || b < 1 || ldx < b) return fail(TH_ERR_INVALID_ARG, "need t >= 0, b >= 1, ldx >= b");
  if (!dtype_ok(xdt)) return fail(TH_ERR_INVALID_ARG, "unknown dtype");
  if (xdt == TH_BF16 && (ldx % 8 || b % 8 || ((uintptr_t)X & 15)))
    return fail(TH_ERR_INVALID_ARG, "bf16 X needs b % 8 == 0, ldx % 8 == 0 and 16-byte alignment");
  size_t need = 0;
  th_hessian_workspace_size(t, b, &need);
  float* part = nullptr;
  if (workspace && need > 0) {
    if (workspace_bytes < need) return fail(TH_ERR_WORKSPACE, "workspace too small");
    if ((uintptr_t)workspace & 15) return fail(TH_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    part = (float*)workspace;
  }
  return accumulate_into(H, X, xdt, t, b, ldx, part, (hipStream_t)stream);
}

th_status th_hessian_finalize(float* H, int64_t b, double lambda, int32_t rel, double* lambda_out,
                              th_stream_t stream) {
  if (!H || b < 1) return fail(TH_ERR_INVALID_ARG, "bad arguments");
  if (!(lambda >= 0.0) || !std::isfinite(lambda)) return fail(TH_ERR_INVALID_ARG, "bad lambda");
  hipStream_t s = (hipStream_t)stream;
  std::vector<float> diag((size_t)b);
  TH_HIP(hipMemcpy2DAsync(diag.data(), sizeof(float), H, (size_t)(b + 1) * sizeof(float),
                          sizeof(float), (size_t)b, hipMemcpyDeviceToHost, s),
         "copy diag");
  TH_HIP(hipStreamSynchronize(s), "sync");
  double sum = 0.0;
  for (int64_t q = 0; q < b; ++q) {
    if (!std::isfinite(diag[q])) return fail(TH_ERR_NONFINITE, "non-finite Hessian diagonal");
    sum += diag[q];
  }
  const double lam = rel ? lambda * (sum / (double)b) : lambda;
  TH_HIP(launch_damp_mirror(H, b, (float)lam, s), "damp_mirror");
  TH_HIP(hipStreamSynchronize(s), "sync");
  if (lambda_out) *lambda_out = lam;
  return TH_OK;
}

th_status th_prune_layer_workspace_size(int64_t c, int64_t b, int64_t n, int32_t have_x,
                                        const th_prune_params* p, size_t* bytes) {
  if (!bytes) return fail(TH_ERR_INVALID_ARG, "bytes is NULL");
  th_status st = check_params(c, b, p);
  if (st != TH_OK) return st;
  // worst case: no caller-provided fp32 output or mask, bf16 X
  PruneLayout L = layout_prune(nullptr, c, b, n, have_x != 0, p, true, true, TH_BF16);
  *bytes = L.bytes;
  return TH_OK;
}

th_status th_prune_layer(void* W, th_dtype wdt, int64_t c, int64_t b, const void* X, th_dtype xdt,
                         int64_t n, const float* H, const th_prune_params* p, float* W_out_f32,
                         uint8_t* mask_out, void* workspace, size_t workspace_bytes,
                         th_stats* stats_out, int64_t* block_counts, th_stream_t stream) {
  th_status chk = check_layer_args(W, wdt, c, b, X, xdt, n, H, p, workspace);
  if (chk != TH_OK) return chk;
  PruneLayout L = layout_prune(workspace, c, b, n, X != nullptr, p, W_out_f32 == nullptr,
                               mask_out == nullptr, xdt);
  if (workspace_bytes < L.bytes) return fail(TH_ERR_WORKSPACE, "workspace too small");
  hipStream_t s = (hipStream_t)stream;
  const int64_t B = p->block;
  const int64_t nblk = cdiv(b, B);
  float* Wf = W_out_f32 ? W_out_f32 : L.Wf;
  uint8_t* mask = mask_out ? mask_out : L.mask;

  th_status st0 = begin_layer(L, W, wdt, c, b, p, Wf, s);
  if (st0 != TH_OK) return st0;
  th_status pre = inverse_factor(X, xdt, n, H, b, p, L, s, p->block);
  if (pre != TH_OK) return pre;

  bool cast_done = false;
  th_status blocks = prune_blocks(L, c, b, p, Wf, mask, s, true, W, wdt, &cast_done);
  if (blocks != TH_OK) return blocks;
  if (!cast_done) TH_HIP(launch_from_f32(Wf, c * b, wdt, W, s), "cast back");
  return finish_layer(L, nblk, stats_out, block_counts, s);
}

// --------------------------------------------- allocation-free layer step

namespace {
// Device memory of the allocation-free entry point: a file-scope array that each
// GPU holds from the library's load until the process ends. Host code never uses
// its name as an address: the per-device address comes from hipGetSymbolAddress.
constexpr size_t kScratchBytes = (size_t)TH_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

// The scratch array's address on the current device, looked up once per device
// (with that device current) and kept.
th_status scratch_on_current_device(void** out) {
  int dev = -1;
  TH_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(TH_ERR_INVALID_ARG, "device index out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    TH_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (!p || ((uintptr_t)p & 255)) return fail(TH_ERR_HIP, "scratch address not 256-byte aligned");
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return TH_OK;
}
}  // namespace

th_status th_prune_layer_noalloc(void* W, th_dtype wdt, int64_t c, int64_t b, const void* X,
                                 th_dtype xdt, int64_t n, const float* H,
                                 const th_prune_params* p, float* W_out_f32, uint8_t* mask_out,
                                 th_stats* stats_out, int64_t* block_counts, th_stream_t stream) {
  th_status chk = check_layer_args(W, wdt, c, b, X, xdt, n, H, p, kNoWorkspace);
  if (chk != TH_OK) return chk;
  const size_t need = layout_prune(nullptr, c, b, n, X != nullptr, p, W_out_f32 == nullptr,
                                   mask_out == nullptr, xdt)
                          .bytes;
  if (need > kScratchBytes) {
    g_last_error = "the layer needs " + std::to_string(need) +
                   " bytes of scratch; th_prune_layer_noalloc holds " +
                   std::to_string(kScratchBytes) + " (use th_prune_layer with a workspace)";
    return TH_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  th_status st = scratch_on_current_device(&ws);
  if (st != TH_OK) return st;
  return th_prune_layer(W, wdt, c, b, X, xdt, n, H, p, W_out_f32, mask_out, ws, kScratchBytes,
                        stats_out, block_counts, stream);
}

th_status th_prune_sparsegpt_workspace_size(int64_t c, int64_t b, int64_t n, int32_t have_x,
                                            const th_prune_params* p, size_t* bytes) {
  if (!bytes) return fail(TH_ERR_INVALID_ARG, "bytes is NULL");
  th_status st = check_params(c, b, p);
  if (st != TH_OK) return st;
  PruneLayout L = layout_prune(nullptr, c, b, n, have_x != 0, p, true, true, TH_BF16, true);
  *bytes = L.bytes;
  return TH_OK;
}

th_status th_prune_sparsegpt(void* W, th_dtype wdt, int64_t c, int64_t b, const void* X,
                             th_dtype xdt, int64_t n, const float* H, const th_prune_params* p,
                             float* W_out_f32, uint8_t* mask_out, void* workspace,
                             size_t workspace_bytes, th_stats* stats_out, int64_t* block_counts,
                             th_stream_t stream) {
  th_status chk = check_layer_args(W, wdt, c, b, X, xdt, n, H, p, workspace);
  if (chk != TH_OK) return chk;
  if (p->score != TH_SCORE_OBS)
    return fail(TH_ERR_INVALID_ARG, "the column-sequential comparator takes the OBS score only");
  PruneLayout L = layout_prune(workspace, c, b, n, X != nullptr, p, W_out_f32 == nullptr,
                               mask_out == nullptr, xdt, true);
  if (workspace_bytes < L.bytes) return fail(TH_ERR_WORKSPACE, "workspace too small");
  hipStream_t s = (hipStream_t)stream;
  const int64_t B = p->block;
  const int64_t nblk = cdiv(b, B);
  float* Wf = W_out_f32 ? W_out_f32 : L.Wf;
  uint8_t* mask = mask_out ? mask_out : L.mask;
  const bool unstr = p->pattern.kind == TH_UNSTRUCTURED;

  th_status st0 = begin_layer(L, W, wdt, c, b, p, Wf, s);  // the budget grows block by block
  if (st0 != TH_OK) return st0;
  th_status pre = inverse_factor(X, xdt, n, H, b, p, L, s, 0);
  if (pre != TH_OK) return pre;
  TH_HIP(launch_sgpt_gdiag(L.R, b, L.gW, s), "score weights");

  // Both masks depend only on the block's own columns, so compensation beyond the
  // super-block waits and is applied once per super-block (K = its width).
  const int64_t ldz = super_pitch(b, B);
  const int64_t per = ldz / B;
  for (int64_t blk = 0; blk < nblk; ++blk) {
    const int64_t j0 = blk * B;
    const int64_t Bb = (b - j0) < B ? (b - j0) : B;
    const int64_t sb0 = (blk / per) * ldz;
    const int64_t s1 = (sb0 + ldz) < b ? (sb0 + ldz) : b;
    float* Eb = L.Z + (blk % per) * B;
    if (unstr) {  // the block's quota: round-half-even(p * c * |J|)
      const long long quota = (long long)std::nearbyint(p->sparsity * (double)c * (double)Bb);
      TH_HIP(launch_select_init(L.st, quota, (long long)(c * Bb), s), "select init");
      for (int pass = 0; pass < 6; ++pass) {
        TH_HIP(launch_select_pass(Wf, c, b, j0, j0 + Bb, L.gW, L.st, s), "select pass");
        TH_HIP(launch_select_pick(L.st, s), "select pick");
      }
    }
    TH_HIP(launch_sgpt_errors(Wf, c, b, j0, B, p->pattern.n, p->pattern.m, unstr ? 1 : 0, L.R,
                              L.gW, Eb, ldz, mask, L.st, L.counts + blk, s),
           "errors");
    TH_HIP(launch_update(Wf, c, b, j0, Bb, ldz, j0, s1, Eb, L.R, mask, j0, Bb, s), "update");
    if (j0 + Bb == s1 && s1 < b)
      TH_HIP(launch_update(Wf, c, b, sb0, s1 - sb0, ldz, s1, b, L.Z, L.R, mask, 0, 0, s),
             "deferred update");
  }
  TH_HIP(launch_from_f32(Wf, c * b, wdt, W, s), "cast back");
  return finish_layer(L, nblk, stats_out, block_counts, s);
}

// ----------------------------------------------------------- shared factor

namespace {
struct FactorLayout {
  DevState* st;
  float* S;
  float* P;
  float* syrk_part;
  size_t bytes;
};

FactorLayout layout_factor(void* ws, int64_t b, int64_t n, bool have_x, th_dtype xdt) {
  Carve cv(ws);
  FactorLayout F;
  F.st = cv.take<DevState>(1);
  F.S = cv.take<float>((size_t)b * b);
  F.P = cv.take<float>(chol_panel_floats(b));
  F.syrk_part = nullptr;
  if (have_x && xdt == TH_BF16) {
    const size_t nf = syrk_bf16_workspace_floats(n, b);
    if (nf > 0) F.syrk_part = cv.take<float>(nf);
  }
  F.bytes = cv.off;
  return F;
}
}  // namespace

th_status th_factor_workspace_size(int64_t b, int64_t n, int32_t have_x, size_t* bytes) {
  if (!bytes || b < 1) return fail(TH_ERR_INVALID_ARG, "bad arguments");
  *bytes = layout_factor(nullptr, b, n, have_x != 0, TH_BF16).bytes;
  return TH_OK;
}

th_status th_factor(const void* X, th_dtype xdt, int64_t n, const float* H, int64_t b,
                    double lambda, int32_t lambda_is_relative, float* U, double* lambda_out,
                    void* workspace, size_t workspace_bytes, th_stream_t stream) {
  if (!U || b < 1) return fail(TH_ERR_INVALID_ARG, "U is NULL or b < 1");
  if ((X == nullptr) == (H == nullptr)) return fail(TH_ERR_INVALID_ARG, "pass exactly one of X, H");
  if (X && (!dtype_ok(xdt) || n < 1)) return fail(TH_ERR_INVALID_ARG, "bad X");
  if (X && xdt == TH_BF16 && (b % 8 || ((uintptr_t)X & 15)))
    return fail(TH_ERR_INVALID_ARG, "bf16 X needs b % 8 == 0 and 16-byte alignment");
  if (!(lambda >= 0.0) || !std::isfinite(lambda))
    return fail(TH_ERR_INVALID_ARG, "lambda must be finite and >= 0");
  if (!workspace || ((uintptr_t)workspace & 255))
    return fail(TH_ERR_INVALID_ARG, "workspace must be non-NULL and 256-byte aligned");
  FactorLayout F = layout_factor(workspace, b, n, X != nullptr, xdt);
  if (workspace_bytes < F.bytes) return fail(TH_ERR_WORKSPACE, "workspace too small");
  hipStream_t s = (hipStream_t)stream;
  th_prune_params p{};
  p.lambda = lambda;
  p.lambda_is_relative = lambda_is_relative;
  p.score = TH_SCORE_OBS;
  PruneLayout L{};
  L.st = F.st;
  L.S = F.S;
  L.R = U;  // H from X accumulates in U, which then receives the factor
  L.P = F.P;
  L.syrk_part = F.syrk_part;
  TH_HIP(launch_zero(F.st, sizeof(DevState), s), "clear state");
  th_status pre = inverse_factor(X, xdt, n, H, b, &p, L, s, 0);  // U is the output
  if (pre != TH_OK) return pre;
  DevState host;
  TH_HIP(hipMemcpyAsync(&host, F.st, offsetof(DevState, hist), hipMemcpyDeviceToHost, s), "state");
  TH_HIP(hipStreamSynchronize(s), "sync");
  if (lambda_out) *lambda_out = host.lambda;
  if (host.nonfinite) return fail(TH_ERR_NONFINITE, "non-finite value in diag(H)");
  if (host.not_spd) return fail(TH_ERR_NOT_SPD, "damped Hessian is not positive definite");
  return TH_OK;
}

th_status th_prune_layer_factored_workspace_size(int64_t c, int64_t b, const th_prune_params* p,
                                                 size_t* bytes) {
  if (!bytes) return fail(TH_ERR_INVALID_ARG, "bytes is NULL");
  th_status st = check_params(c, b, p);
  if (st != TH_OK) return st;
  *bytes = layout_prune(nullptr, c, b, 0, false, p, true, true, TH_BF16, false, false).bytes;
  return TH_OK;
}

th_status th_prune_layer_factored(void* W, th_dtype wdt, int64_t c, int64_t b, const float* U,
                                  const th_prune_params* p, float* W_out_f32, uint8_t* mask_out,
                                  void* workspace, size_t workspace_bytes, th_stats* stats_out,
                                  int64_t* block_counts, th_stream_t stream) {
  // U stands in for H in the shared checks (exactly one of X and H)
  th_status chk = check_layer_args(W, wdt, c, b, nullptr, TH_BF16, 0, U, p, workspace);
  if (chk != TH_OK) return chk;
  if (p->score != TH_SCORE_OBS)
    return fail(TH_ERR_INVALID_ARG, "a given factor takes the OBS score only");
  PruneLayout L = layout_prune(workspace, c, b, 0, false, p, W_out_f32 == nullptr,
                               mask_out == nullptr, TH_BF16, false, false);
  if (workspace_bytes < L.bytes) return fail(TH_ERR_WORKSPACE, "workspace too small");
  hipStream_t s = (hipStream_t)stream;
  float* Wf = W_out_f32 ? W_out_f32 : L.Wf;
  uint8_t* mask = mask_out ? mask_out : L.mask;
  th_status st0 = begin_layer(L, W, wdt, c, b, p, Wf, s);
  if (st0 != TH_OK) return st0;
  // the slices are formed in place, so the caller's factor is copied first
  TH_HIP(hipMemcpyAsync(L.R, U, (size_t)b * b * sizeof(float), hipMemcpyDeviceToDevice, s), "U");
  bool cast_done = false;
  th_status blocks = prune_blocks(L, c, b, p, Wf, mask, s, false, W, wdt, &cast_done);
  if (blocks != TH_OK) return blocks;
  if (!cast_done) TH_HIP(launch_from_f32(Wf, c * b, wdt, W, s), "cast back");
  return finish_layer(L, cdiv(b, p->block), stats_out, block_counts, s);
}

// ------------------------------------------------------- alpha outlier rows

namespace {
struct AlphaLayout {
  PruneLayout L;  // the compact layer (c - r rows), with its own fp32 W and mask
  DevState* sel;  // state of the row selection (the layer keeps L.st)
  float* scores;
  int32_t* idx;
  int32_t* rowmap;
  float* gdiag;
  double* colsq;
  size_t bytes;
};

AlphaLayout layout_alpha(void* ws, int64_t c, int64_t cp, int64_t b, int64_t n, bool have_x,
                         const th_prune_params* p, th_dtype xdt) {
  AlphaLayout A;
  A.L = layout_prune(ws, cp < 1 ? 1 : cp, b, n, have_x, p, true, true, xdt);
  Carve cv(ws);
  cv.off = A.L.bytes;
  A.sel = cv.take<DevState>(1);
  A.scores = cv.take<float>((size_t)c);
  A.idx = cv.take<int32_t>((size_t)c);
  A.rowmap = cv.take<int32_t>((size_t)c);
  A.gdiag = cv.take<float>((size_t)b);
  A.colsq = have_x ? cv.take<double>((size_t)colsq_splits(n) * b) : nullptr;
  A.bytes = cv.off;
  return A;
}
}  // namespace

th_status th_prune_layer_alpha_workspace_size(int64_t c, int64_t b, int64_t n, int32_t have_x,
                                              const th_prune_params* p, double alpha,
                                              size_t* bytes) {
  if (!bytes) return fail(TH_ERR_INVALID_ARG, "bytes is NULL");
  th_status st = check_params(c, b, p);
  if (st != TH_OK) return st;
  if (!(alpha >= 0.0 && alpha <= 1.0)) return fail(TH_ERR_INVALID_ARG, "alpha must be in [0, 1]");
  const int64_t cp = c - (int64_t)std::nearbyint(alpha * (double)c);
  *bytes = layout_alpha(nullptr, c, cp, b, n, have_x != 0, p, TH_BF16).bytes;
  return TH_OK;
}

th_status th_prune_layer_alpha(void* W, th_dtype wdt, int64_t c, int64_t b, const void* X,
                               th_dtype xdt, int64_t n, const float* H, const th_prune_params* p,
                               double alpha, float* W_out_f32, uint8_t* mask_out,
                               uint8_t* dense_rows_out, void* workspace, size_t workspace_bytes,
                               th_stats* stats_out, int64_t* block_counts, th_stream_t stream) {
  th_status chk = check_layer_args(W, wdt, c, b, X, xdt, n, H, p, workspace);
  if (chk != TH_OK) return chk;
  if (!(alpha >= 0.0 && alpha <= 1.0)) return fail(TH_ERR_INVALID_ARG, "alpha must be in [0, 1]");
  if (c >= ((int64_t)1 << 31)) return fail(TH_ERR_INVALID_ARG, "c must be < 2^31");
  const int64_t r = (int64_t)std::nearbyint(alpha * (double)c);  // rows kept dense
  const int64_t cp = c - r;
  AlphaLayout A = layout_alpha(workspace, c, cp, b, n, X != nullptr, p, xdt);
  if (workspace_bytes < A.bytes) return fail(TH_ERR_WORKSPACE, "workspace too small");
  const PruneLayout& L = A.L;
  hipStream_t s = (hipStream_t)stream;
  const int64_t nblk = cdiv(b, p->block);

  TH_HIP(launch_zero(L.st, sizeof(DevState), s), "clear state");
  TH_HIP(launch_zero(A.sel, sizeof(DevState), s), "clear selection state");
  TH_HIP(launch_zero(L.counts, nblk * sizeof(unsigned long long), s), "clear counts");
  // G_qq: column norms of X, or (H_qq - lambda)/2 of a damped H
  if (X) {
    TH_HIP(launch_column_sq_norms(X, xdt, n, b, b, A.colsq, A.gdiag, s), "column norms");
  } else {
    TH_HIP(launch_lambda(H, b, p->lambda, p->lambda_is_relative, 1, A.sel, s), "lambda");
    TH_HIP(launch_wanda_diag(H, b, A.sel, 1, A.gdiag, s), "G diagonal");
  }
  // the c - r rows of smallest (energy, row) are pruned, the rest stay dense; a
  // non-finite energy (a non-finite weight) raises the layer's flag
  TH_HIP(launch_row_energy(W, wdt, c, b, A.gdiag, A.scores, s), "row energy");
  TH_HIP(launch_select_init(A.sel, (long long)cp, (long long)c, s), "select init");
  for (int pass = 0; pass < 6; ++pass) {
    TH_HIP(launch_select_scores_pass(A.scores, c, 1, 1, 0, A.sel, s), "select pass");
    TH_HIP(launch_select_pick(A.sel, s), "select pick");
  }
  TH_HIP(launch_row_index(A.scores, c, A.sel, A.idx, A.rowmap, dense_rows_out, L.st, s),
         "row index");

  // the layer step on the compact rows
  if (cp > 0) TH_HIP(launch_gather_rows(W, wdt, b, A.rowmap, cp, L.Wf, L.st, s), "gather");
  th_status pre = inverse_factor(X, xdt, n, H, b, p, L, s, p->block);
  if (pre != TH_OK) return pre;
  if (cp > 0) {
    th_status blocks = prune_blocks(L, cp, b, p, L.Wf, L.mask, s, true);
    if (blocks != TH_OK) return blocks;
  }
  TH_HIP(launch_scatter_rows(W, wdt, c, b, A.idx, L.Wf, L.mask, W_out_f32, mask_out, s),
         "scatter");
  return finish_layer(L, nblk, stats_out, block_counts, s);
}

// ------------------------------------------------------ gated feed-forward

th_status th_gated_ffn_input(const void* X, const void* W_gate, const void* W_up, th_dtype dt,
                             int64_t n, int64_t d, int64_t f, void* Y, th_stream_t stream) {
  if (!X || !W_gate || !W_up || !Y) return fail(TH_ERR_INVALID_ARG, "NULL argument");
  if (dt != TH_BF16) return fail(TH_ERR_INVALID_ARG, "bf16 only");
  if (n < 1 || d < 8 || f < 1 || d % 8) return fail(TH_ERR_INVALID_ARG, "needs n, f >= 1, d % 8 == 0");
  if (cdiv(n, 256) * cdiv(f, 128) >= ((int64_t)1 << 30))
    return fail(TH_ERR_INVALID_ARG, "n * f too large for one launch");
  if (((uintptr_t)X | (uintptr_t)W_gate | (uintptr_t)W_up) & 15)
    return fail(TH_ERR_INVALID_ARG, "X, W_gate and W_up must be 16-byte aligned");
  TH_HIP(launch_gated_ffn((const unsigned short*)X, (const unsigned short*)W_gate,
                          (const unsigned short*)W_up, (unsigned short*)Y, n, d, f,
                          (hipStream_t)stream),
         "gated ffn");
  return TH_OK;
}

th_status th_reconstruction_error_workspace_size(int64_t c, int64_t b, int32_t have_x,
                                                 size_t* bytes) {
  if (!bytes || c < 1 || b < 1) return fail(TH_ERR_INVALID_ARG, "bad arguments");
  Carve cv(nullptr);
  cv.take<float>((size_t)c * b);
  cv.take<float>((size_t)c * b);
  if (have_x) cv.take<float>((size_t)b * b);
  cv.take<double>((size_t)cdiv(c, 128) * cdiv(b, 128));
  cv.take<double>(2);
  *bytes = cv.off;
  return TH_OK;
}

th_status th_reconstruction_error(const void* W, const void* What, th_dtype wdt, int64_t c,
                                  int64_t b, const void* X, th_dtype xdt, int64_t n,
                                  const float* G, void* workspace, size_t workspace_bytes,
                                  double* err_out, double* rel_err_out, th_stream_t stream) {
  if (!W || !What || !workspace) return fail(TH_ERR_INVALID_ARG, "NULL argument");
  if (c < 1 || b < 1) return fail(TH_ERR_INVALID_ARG, "c and b must be >= 1");
  if ((X == nullptr) == (G == nullptr)) return fail(TH_ERR_INVALID_ARG, "pass exactly one of X, G");
  if (!dtype_ok(wdt) || (X && !dtype_ok(xdt))) return fail(TH_ERR_INVALID_ARG, "unknown dtype");
  if (X && xdt == TH_BF16 && (b % 8 || ((uintptr_t)X & 15)))
    return fail(TH_ERR_INVALID_ARG, "bf16 X needs b % 8 == 0 and 16-byte alignment");
  size_t need = 0;
  th_reconstruction_error_workspace_size(c, b, X != nullptr, &need);
  if (workspace_bytes < need) return fail(TH_ERR_WORKSPACE, "workspace too small");
  hipStream_t s = (hipStream_t)stream;
  Carve cv(workspace);
  float* D = cv.take<float>((size_t)c * b);
  float* Wf = cv.take<float>((size_t)c * b);
  float* Gb = X ? cv.take<float>((size_t)b * b) : nullptr;
  double* parts = cv.take<double>((size_t)cdiv(c, 128) * cdiv(b, 128));
  double* out = cv.take<double>(2);
  double scale = 1.0;
  if (X) {
    TH_HIP(launch_zero(Gb, (size_t)b * b * sizeof(float), s), "clear G");
    th_status a = accumulate_into(Gb, X, xdt, n, b, b, nullptr, s);  // 2G, lower
    if (a != TH_OK) return a;
    TH_HIP(launch_damp_mirror(Gb, b, 0.f, s), "mirror");
    G = Gb;
    scale = 0.5;
  }
  TH_HIP(launch_diff_f32(W, What, wdt, c * b, D, s), "diff");
  TH_HIP(launch_to_f32(W, wdt, c * b, Wf, nullptr, s), "W to fp32");
  int64_t np = 0;
  TH_HIP(launch_quadform(D, c, b, G, parts, &np, s), "quadform");
  TH_HIP(launch_sum_partials(parts, np, out, s), "sum");
  TH_HIP(launch_quadform(Wf, c, b, G, parts, &np, s), "quadform");
  TH_HIP(launch_sum_partials(parts, np, out + 1, s), "sum");
  double host[2];
  TH_HIP(hipMemcpyAsync(host, out, sizeof(host), hipMemcpyDeviceToHost, s), "copy");
  TH_HIP(hipStreamSynchronize(s), "sync");
  const double E = host[0] * scale, base = host[1] * scale;
  if (err_out) *err_out = E;
  if (rel_err_out) *rel_err_out = base > 0 ? E / base : 0.0;
  return TH_OK;
}

th_status th_debug_select_nm(const float* scores, int64_t c, int64_t blk, int32_t n, int32_t m,
                             uint8_t* mask_blk, th_stream_t stream) {
  if (!scores || !mask_blk || c < 1 || blk < 1 || blk > 1024)
    return fail(TH_ERR_INVALID_ARG, "bad arguments (blk must be in [1, 1024])");
  if (m < 1 || n < 0 || n > m || blk % m) return fail(TH_ERR_INVALID_ARG, "bad N:M");
  TH_HIP(launch_debug_select_nm(scores, c, blk, n, m, mask_blk, (hipStream_t)stream), "select nm");
  return TH_OK;
}

th_status th_debug_select_global(const float* scores, int64_t c, int64_t f, int64_t b_full,
                                 int64_t j0, int64_t blk, int64_t r, uint8_t* mask_blk,
                                 int32_t* s_k, void* workspace, size_t workspace_bytes,
                                 th_stream_t stream) {
  if (!scores || !mask_blk || !workspace) return fail(TH_ERR_INVALID_ARG, "NULL argument");
  if (c < 1 || f < 1 || blk < 1 || blk > f || j0 < 0 || j0 + f > b_full || c * b_full >= ((int64_t)1 << 32))
    return fail(TH_ERR_INVALID_ARG, "bad sizes");
  if (workspace_bytes < sizeof(DevState)) return fail(TH_ERR_WORKSPACE, "workspace too small");
  hipStream_t s = (hipStream_t)stream;
  DevState* st = (DevState*)workspace;
  TH_HIP(hipMemsetAsync(st, 0, sizeof(DevState), s), "memset");
  TH_HIP(launch_select_init(st, (long long)r, (long long)(c * f), s), "init");  // budget = r
  for (int pass = 0; pass < 6; ++pass) {
    TH_HIP(launch_select_scores_pass(scores, c, f, b_full, j0, st, s), "pass");
    TH_HIP(launch_select_pick(st, s), "pick");
  }
  TH_HIP(launch_debug_mask_from_scores(scores, c, f, b_full, j0, blk, st, mask_blk, s_k, s), "mask");
  TH_HIP(hipStreamSynchronize(s), "sync");
  return TH_OK;
}

th_status th_column_sq_norms_workspace_size(int64_t n, int64_t b, size_t* bytes) {
  if (!bytes || n < 1 || b < 1) return fail(TH_ERR_INVALID_ARG, "bad arguments");
  *bytes = (size_t)colsq_splits(n) * (size_t)b * sizeof(double);
  return TH_OK;
}

th_status th_column_sq_norms(const void* X, th_dtype xdt, int64_t n, int64_t b, int64_t ldx,
                             float* gdiag, void* workspace, size_t workspace_bytes,
                             th_stream_t stream) {
  if (!X || !gdiag || n < 1 || b < 1 || ldx < b || !dtype_ok(xdt))
    return fail(TH_ERR_INVALID_ARG, "bad arguments");
  size_t need = 0;
  th_column_sq_norms_workspace_size(n, b, &need);
  if (!workspace || workspace_bytes < need) return fail(TH_ERR_WORKSPACE, "workspace too small");
  TH_HIP(launch_column_sq_norms(X, xdt, n, b, ldx, (double*)workspace, gdiag, (hipStream_t)stream),
         "column norms");
  return TH_OK;
}

th_status th_prune_baseline(void* W, th_dtype wdt, int64_t c, int64_t b, th_baseline method,
                            const float* gdiag, const th_prune_params* p, uint8_t* mask_out,
                            th_stream_t stream) {
  if (!W || !p || !dtype_ok(wdt)) return fail(TH_ERR_INVALID_ARG, "bad arguments");
  if (c < 1 || b < 1) return fail(TH_ERR_INVALID_ARG, "c and b must be >= 1");
  if (c * b >= (int64_t)1 << 32) return fail(TH_ERR_INVALID_ARG, "c*b must be < 2^32");
  if (method != TH_BASE_MAGNITUDE && method != TH_BASE_WANDA)
    return fail(TH_ERR_INVALID_ARG, "unknown baseline method");
  if (method == TH_BASE_WANDA && !gdiag)
    return fail(TH_ERR_INVALID_ARG, "Wanda needs the squared column norms gdiag");
  const float* g = method == TH_BASE_WANDA ? gdiag : nullptr;
  hipStream_t s = (hipStream_t)stream;
  if (p->pattern.kind == TH_UNSTRUCTURED) {
    if (!(p->sparsity >= 0.0 && p->sparsity <= 1.0))
      return fail(TH_ERR_INVALID_ARG, "sparsity must be in [0, 1]");
    // every row loses round-half-even(p * b) weights
    const int64_t krow = (int64_t)std::nearbyint(p->sparsity * (double)b);
    TH_HIP(launch_baseline_rows(W, wdt, c, b, g, krow, mask_out, s), "baseline rows");
  } else if (p->pattern.kind == TH_NM) {
    const int n = p->pattern.n, m = p->pattern.m;
    if (m < 1 || m > kMaxBlock || n < 0 || n > m)
      return fail(TH_ERR_INVALID_ARG, "N:M needs 0 <= n <= m, 1 <= m <= 128");
    if (b % m) return fail(TH_ERR_INVALID_ARG, "N:M needs m | b");
    TH_HIP(launch_baseline_nm(W, wdt, c, b, g, n, m, mask_out, s), "baseline N:M");
  } else {
    return fail(TH_ERR_INVALID_ARG, "unknown pattern kind");
  }
  return TH_OK;
}

th_status th_debug_factor(const float* H, int64_t b, float* U, void* workspace,
                          size_t workspace_bytes, th_stream_t stream) {
  if (!H || !U || !workspace || b < 1) return fail(TH_ERR_INVALID_ARG, "bad arguments");
  Carve cv(workspace);
  DevState* st = cv.take<DevState>(1);
  float* S = cv.take<float>((size_t)b * b);
  float* P = cv.take<float>(chol_panel_floats(b));
  if (workspace_bytes < cv.off) return fail(TH_ERR_WORKSPACE, "workspace too small");
  hipStream_t s = (hipStream_t)stream;
  TH_HIP(hipMemsetAsync(st, 0, sizeof(DevState), s), "memset");
  TH_HIP(launch_flip_lower(H, S, b, st, 0, s), "flip");
  TH_HIP(launch_chol_inv_inplace(S, b, P, st, s), "cholesky/inverse");
  TH_HIP(launch_reverse(S, U, b, 0, s), "reverse");
  int flag = 0;
  TH_HIP(hipMemcpyAsync(&flag, &st->not_spd, sizeof(int), hipMemcpyDeviceToHost, s), "flag");
  TH_HIP(hipStreamSynchronize(s), "sync");
  if (flag) return fail(TH_ERR_NOT_SPD, "damped Hessian is not positive definite");
  return TH_OK;
}

th_status th_debug_syrk_rect(float* H, const void* X, int64_t t, int64_t b, int64_t ldx, int32_t P,
                             int32_t m, void* workspace, size_t workspace_bytes,
                             th_stream_t stream) {
  if (!H || !X) return fail(TH_ERR_INVALID_ARG, "NULL argument");
  if (t < 32 || b < 1 || ldx < b || ldx >= ((int64_t)1 << 25) || P < 1 || P > 4096 || m < 0 ||
      m > t / 32)
    return fail(TH_ERR_INVALID_ARG,
                "need t >= 32, 1 <= b <= ldx < 2^25, 1 <= P <= 4096, 0 <= m <= t / 32");
  if (ldx % 8 || b % 8 || ((uintptr_t)X & 15))
    return fail(TH_ERR_INVALID_ARG, "bf16 X needs b % 8 == 0, ldx % 8 == 0 and 16-byte alignment");
  const size_t need = syrk_rect_workspace_floats(t, b, P, m) * sizeof(float);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(TH_ERR_WORKSPACE, "workspace too small");
  if ((uintptr_t)workspace & 15) return fail(TH_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  TH_HIP(launch_syrk_rect(H, (const unsigned short*)X, t, b, ldx, (float*)workspace, P, m,
                          (hipStream_t)stream, false),
         "syrk rectangles");
  return TH_OK;
}

th_status th_debug_far_update(float* W, int64_t c, int64_t b, const float* Z, int64_t ldz,
                              const float* R, int64_t r0, int64_t K, int64_t col0,
                              int64_t col_end, void* workspace, size_t workspace_bytes,
                              th_stream_t stream) {
  if (!W || !Z || !R || !workspace) return fail(TH_ERR_INVALID_ARG, "NULL argument");
  if (c < 1 || b < 1 || K < 16 || K % 16 || ldz < K || r0 < 0 || col0 < 0 || col_end <= col0 ||
      col_end > b)
    return fail(TH_ERR_INVALID_ARG, "bad shape");
  if ((uintptr_t)workspace & 15) return fail(TH_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  if (workspace_bytes < far_x3_elems(c, col_end - col0, K) * sizeof(unsigned short))
    return fail(TH_ERR_WORKSPACE, "workspace too small");
  TH_HIP(launch_far_update(W, c, b, r0, K, ldz, col0, col_end, Z, R, (unsigned short*)workspace,
                           (hipStream_t)stream),
         "far update");
  return TH_OK;
}

}  // extern "C"
