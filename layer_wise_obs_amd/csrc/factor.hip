// Factor and invert the damped Hessian once per layer.
//
// What the block loop needs is U, upper triangular with H^-1 = U^T U (the factor
// the explainer's section "SparseGPT: Second-Order Reconstruction at Scale"
// computes once per layer; "Pruning LLMs with Thanos", section "Contribution one",
// takes R and R-hat from the inverse Hessian). U = V^-1 where H = V V^T with V
// upper ("reverse" Cholesky). With P the reversal permutation, P H P = L L^T is
// an ordinary lower Cholesky factorisation and U = P L^-1 P.
//
// The factorisation and the triangular inverse run in one right-looking sweep
// over 128-wide block columns, in place on S = P H P (lower triangle):
//   before step k:  S[k:,k:] = Schur complement,  S[k:,:k] = partial rows of L^-1,
//                   S[:k,:k] = final rows of L^-1.
//   step k:  (1) one workgroup factors the diagonal block (fp32, registers and
//                LDS): X_kk = L_kk^-1, written back over the block;
//            (2) panel:  Lp_i = S[i,k] X_kk^T for block rows i > k (to a buffer),
//                        S[k,:k] = X_kk S[k,:k] (row k of L^-1 is now final);
//            (3) trailing, one GEMM over all tiles (i > k, j <= i):
//                S[i,j] -= Lp_i [ X row k | -/X_kk | Lp_j^T ]  (j < k | j = k | j > k),
//                where column block k is overwritten with -Lp_i X_kk.
//   Steps run in pairs: step k updates only block row and column k+1, block k+1
//   is factored, and then one K = 256 GEMM applies both steps to everything else
//   (half the C traffic per flop of two K = 128 updates). That GEMM is split in
//   two: the tiles the next pair's factorisation reads first (block rows and
//   columns k+2, k+3) run on the caller's stream, the rest on a second stream as
//   a persistent kernel of one workgroup per compute unit, so that the next
//   pair's diagonal blocks, panels and row/column update (a chain of small,
//   latency-bound kernels) run beside the bulk of the update. Each diagonal
//   factorisation after the first shares a launch with the update that precedes
//   it on the chain (block row and column k+1, or the look-ahead set): its
//   workgroup updates the diagonal tile straight into LDS and factors it while
//   the launch's other workgroups update the remaining tiles. The rest set reads
//   the pair's operands once more, pre-split into bf16 planes (rest_x3.h): its
//   tiles are a symmetric rank-256 product like the Hessian's syrk and run on
//   that kernel's pipeline, 256 x 256 per workgroup.
// The panel and trailing GEMMs run on the bf16 matrix cores with three-way split
// fp32 operands (gemm_x3.h: errors of the order of fp32 accumulation, at about a
// third of the fp32 matrix-core time); the diagonal blocks stay in fp32.
// At the end S holds L^-1 (lower); U is the element-wise reversal of S.
#include "gemm_x3.h"
#include "rest_x3.h"

namespace th {

namespace {

constexpr int kNb = 128;
constexpr int kBase = 32;  // block-column width of the sweep inside the diagonal block
constexpr int kBase16 = 16;  // register base case
constexpr int kPP16 = kBase16 + 1;
constexpr int kPP = kBase + 1;  // LDS pitch of a 32 x 32 panel tile
constexpr int kSP = kNb + 1;  // LDS pitch (floats) of the 128 x 128 diagonal block

// Copy of the lane id that the compiler cannot hoist or share across the
// unrolled steps (keeps per-step lane masks short-lived).
__device__ __forceinline__ int fresh_lane() {
  int l = threadIdx.x & 63;
  __asm__ volatile("" : "+v"(l));
  return l;
}

// Accumulator layout of one 32x32 MFMA block (lane l, register q):
// row 8*(q/4) + 4*(l/32) + (q%4), column l%32.
template <class F>
__device__ __forceinline__ void tile_foreach(const f32x16_t& acc, F&& f) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int q = 0; q < 16; ++q) f(8 * (q >> 2) + 4 * (lane >> 5) + (q & 3), lane & 31, acc[q]);
}

template <class F>
__device__ __forceinline__ void tile_foreach_idx(f32x16_t& acc, F&& f) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int q = 0; q < 16; ++q) f(q, 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3), lane & 31);
}

// One wave, 16 x 16 SPD block `a` (lower triangle, pitch lda): X = L^-1 with
// a = L L^T written to `x` (pitch ldx, zeros above the diagonal; x may be a).
// Lanes 16..63 shadow lanes 0..15. Branch-free and fully unrolled:
// Pass 1, right-looking Cholesky, lane i holds row i; step j reads column j of
//   the (symmetric) trailing block from lane c's register j with v_readlane.
//   Lane i keeps L[i][j] in Lc[j].
// Pass 2, right-looking forward substitution L X = I, lane c holds column c of
//   X; L[i][m] is lane i's Lc[m], read with v_readlane.
__device__ __forceinline__ void wave_chol_inv16(const float* a, int lda, float* x, int ldx,
                                                int& flag) {
  float Lc[kBase16], rsv[kBase16];
  {
    const int row = threadIdx.x & 15;
    float reg[kBase16];
    static_for<0, kBase16>([&](auto C) __attribute__((always_inline)) {
      constexpr int c = C;
      reg[c] = (c <= row) ? a[row * lda + c] : a[c * lda + row];
    });
    static_for<0, kBase16>([&](auto J) __attribute__((always_inline)) {
      constexpr int j = J;
      const int ln = fresh_lane() & 15;
      const float p0 = bcast(reg[j], j);
      const bool ok = (p0 > 0.f) && (p0 < 3.0e38f);
      flag |= ok ? 0 : 1;
      const float p = ok ? p0 : 1.f;
      const float rs = __builtin_amdgcn_rsqf(p);
      const float sp = p * rs;
      rsv[j] = rs;
      const float rj = reg[j];
      const float f = (ln > j) ? rj * (rs * rs) : 0.f;
      float lv = rj * rs;
      lv = (ln > j) ? lv : 0.f;
      Lc[j] = (ln == j) ? sp : lv;
      static_for<j + 1, kBase16>([&](auto C) __attribute__((always_inline)) {
        constexpr int c = C;
        reg[c] = fmaf(-f, bcast(rj, c), reg[c]);
      });
    });
  }
  const int col = fresh_lane() & 15;
  float acc[kBase16];
  static_for<0, kBase16>([&](auto I) __attribute__((always_inline)) {
    constexpr int i = I;
    acc[i] = (col == i) ? 1.f : 0.f;
  });
  static_for<0, kBase16>([&](auto M) __attribute__((always_inline)) {
    constexpr int m = M;
    const float xm = acc[m] * rsv[m];
    acc[m] = xm;
    static_for<m + 1, kBase16>([&](auto I) __attribute__((always_inline)) {
      constexpr int i = I;
      acc[i] = fmaf(-bcast(Lc[m], i), xm, acc[i]);
    });
  });
  wave_sync();  // every lane has read `a` before `x` (possibly the same) is written
  static_for<0, kBase16>([&](auto I) __attribute__((always_inline)) {
    constexpr int i = I;
    x[i * ldx + col] = (i >= col) ? acc[i] : 0.f;
  });
  wave_sync();
}

// 16 x 16 = acc + sum_k A(i, k) B(k, j), k < 16, on v_mfma_f32_16x16x4_f32
// (A: lane l holds A[l%16][l/16]; B: B[l/16][l%16]; D register r of lane l is
// D[4*(l/16) + r][l%16]).
template <class FA, class FB>
__device__ __forceinline__ f32x4_t mfma16(f32x4_t acc, FA&& a, FB&& bop) {
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, kq = lane >> 4;
#pragma unroll
  for (int k0 = 0; k0 < kBase16; k0 += 4)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a(i, k0 + kq), bop(k0 + kq, i), acc, 0, 0, 0);
  return acc;
}

template <class F>
__device__ __forceinline__ void foreach16(const f32x4_t& acc, F&& f) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int r = 0; r < 4; ++r) f(4 * (lane >> 4) + r, lane & 15, acc[r]);
}

// One wave, 32 x 32 SPD block d (lower triangle, pitch kSP) -> X = L^-1 in place
// (zeros above the diagonal), split 2 x 2 into 16-blocks:
//   X11 = chol_inv(A11);  L21 = A21 X11^T;  A22 -= L21 L21^T;  X22 = chol_inv(A22);
//   X21 = -X22 (L21 X11).
// tmp: 16 x kPP16 floats of LDS scratch.
__device__ __forceinline__ void wave_chol_inv32(float* d, float* tmp, int* bad) {
  int flag = 0;
  float* A21 = d + 16 * kSP;
  float* A22 = d + 16 * kSP + 16;
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  wave_chol_inv16(d, kSP, d, kSP, flag);
  {  // L21 = A21 X11^T over A21
    f32x4_t acc = mfma16(zero, [&](int i, int k) { return A21[i * kSP + k]; },
                         [&](int k, int j) { return d[j * kSP + k]; });
    wave_sync();
    foreach16(acc, [&](int i, int j, float v) { A21[i * kSP + j] = v; });
    wave_sync();
  }
  {  // A22 -= L21 L21^T
    f32x4_t acc;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = -A22[(4 * (lane >> 4) + r) * kSP + (lane & 15)];
    acc = mfma16(acc, [&](int i, int k) { return A21[i * kSP + k]; },
                 [&](int k, int j) { return A21[j * kSP + k]; });
    foreach16(acc, [&](int i, int j, float v) { A22[i * kSP + j] = -v; });
    wave_sync();
  }
  wave_chol_inv16(A22, kSP, A22, kSP, flag);
  {  // T = L21 X11 -> tmp
    f32x4_t acc = mfma16(zero, [&](int i, int k) { return A21[i * kSP + k]; },
                         [&](int k, int j) { return d[k * kSP + j]; });
    foreach16(acc, [&](int i, int j, float v) { tmp[i * kPP16 + j] = v; });
    wave_sync();
  }
  {  // X21 = -X22 T over A21; the upper-right block of X is zero
    f32x4_t acc = mfma16(zero, [&](int i, int k) { return A22[i * kSP + k]; },
                         [&](int k, int j) { return tmp[k * kPP16 + j]; });
    foreach16(acc, [&](int i, int j, float v) {
      A21[i * kSP + j] = -v;
      d[i * kSP + 16 + j] = 0.f;
    });
    wave_sync();
  }
  if (flag && (threadIdx.x & 63) == 0) *bad = 1;
}

// 32 x 32 tile (this wave) of init - sum_m A(i, m) B(m, j), m < 32, operands in LDS.
template <class FA, class FB>
__device__ __forceinline__ f32x16_t lds_mfma_tile32(f32x16_t acc, FA&& a, FB&& bop) {
  const int lane = threadIdx.x & 63;
  const int i = lane & 31, kk = lane >> 5;
#pragma unroll
  for (int m = 0; m < kBase; m += 2)
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(-a(i, m + kk), bop(m + kk, i), acc, 0, 0, 0);
  return acc;
}

// (1) Diagonal block: X_kk = L_kk^-1 with A_kk = L_kk L_kk^T, fp32, 256 threads,
// the whole block in LDS. The same right-looking in-place sweep as the layer's
// factorisation, over four 32-wide block columns t = 0..3:
//   base:     X_tt = chol_inv(A_tt)                       (one wave)
//   panel:    Lp_i = A_it X_tt^T (i > t);  A_tj = X_tt A_tj (j < t)
//   trailing: A_ij -= Lp_i [ A_tj | X_tt (overwrite) | Lp_j^T ]  (j < t | j = t | j > t)
// The base case of step t + 1 needs only tile (t+1, t+1) of step t's trailing
// update, so wave 0 updates that tile and factors it while the other waves
// finish the step.
// A block narrower than 128 (the last one) is padded with the identity.
// LDS of a diagonal factorisation (the split-operand GEMM of the fused launches
// below stages its operands in the same space before the block is formed there).
struct DiagLds {
  float sS[kNb * kSP];
  float sP[3 * kBase * kPP];
  float sT[kBase16 * kPP16];
  int bad;
};
static_assert(sizeof(DiagLds) >= (size_t)kX3LdsBytes, "GEMM staging fits in the diagonal LDS");

// The block of S at (k0, k0) into sS: lower triangle, identity padding past nbk.
__device__ __forceinline__ void diag_load(const float* __restrict__ S, int64_t b, int64_t k0,
                                          int nbk, float* sS) {
  const int tid = threadIdx.x;
  // all 64 loads of a thread in flight at once (addresses clamped into the block)
  constexpr int kPer = kNb * kNb / 256;
  float v[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int idx = e * 256 + tid, i = idx >> 7, j = idx & (kNb - 1);
    const int ii = i < nbk ? i : nbk - 1, jj = j < nbk ? j : nbk - 1;
    v[e] = S[(k0 + ii) * b + k0 + jj];
  }
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int idx = e * 256 + tid, i = idx >> 7, j = idx & (kNb - 1);
    const float pad = (i == j) ? 1.f : 0.f;
    sS[i * kSP + j] = (i < nbk && j < nbk && j <= i) ? v[e] : pad;
  }
}

// The accumulators of a 128 x 128 GEMM tile (the updated diagonal block) into sS,
// as diag_load would have read them from S.
__device__ __forceinline__ void diag_from_acc(const f32x16_t (&acc)[2][2], int nbk, float* sS) {
  gemm_foreach(acc, [&](int r, int c, float v) {
    const float pad = (r == c) ? 1.f : 0.f;
    sS[r * kSP + c] = (r < nbk && c < nbk && c <= r) ? v : pad;
  });
}

// Factor the block in sS (all 256 threads; sS complete and visible): X = L^-1
// written back over the block of S at (k0, k0), zeros above the diagonal.
__device__ __forceinline__ void diag_factor_body(float* __restrict__ S, int64_t b, int64_t k0,
                                                 int nbk, DevState* st, DiagLds& L) {
  float* const sS = L.sS;
  float* const sP = L.sP;
  float* const sT = L.sT;
  int& bad = L.bad;
  const int tid = threadIdx.x, wave = tid >> 6;
  auto blk = [&](int i, int j) { return sS + (kBase * i) * kSP + kBase * j; };
  // trailing tile q of step t: (i, j), t < i < 4, 0 <= j <= i, row-major order
  auto trailing_tile = [&](int t, int q) {
    int i = t + 1, rem = q;
    while (rem > i) { rem -= i + 1; ++i; }
    const int j = rem;
    float* C = blk(i, j);
    const float* Lpi = sP + (i - 1) * kBase * kPP;
    f32x16_t acc;
    tile_foreach_idx(acc, [&](int q2, int rr, int cc) {
      acc[q2] = (j == t) ? 0.f : C[rr * kSP + cc];
    });
    if (j <= t) {
      const float* Btj = blk(t, j);
      acc = lds_mfma_tile32(
          acc, [&](int ii, int m) { return Lpi[ii * kPP + m]; },
          [&](int m, int jj) { return Btj[m * kSP + jj]; });
    } else {
      const float* Lpj = sP + (j - 1) * kBase * kPP;
      acc = lds_mfma_tile32(
          acc, [&](int ii, int m) { return Lpi[ii * kPP + m]; },
          [&](int m, int jj) { return Lpj[jj * kPP + m]; });
    }
    tile_foreach(acc, [&](int rr, int cc, float x) { C[rr * kSP + cc] = x; });
  };
  if (wave == 0) wave_chol_inv32(blk(0, 0), sT, &bad);
  __syncthreads();
  for (int t = 0; t < 4; ++t) {
    const float* Dtt = blk(t, t);
    if (wave < 3) {  // 3 - t rows of Lp, t blocks of row t
      f32x16_t acc;
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[q] = 0.f;
      if (wave < 3 - t) {
        const int i = t + 1 + wave;
        const float* Ait = blk(i, t);
        acc = lds_mfma_tile32(
            acc, [&](int ii, int m) { return -Ait[ii * kSP + m]; },
            [&](int m, int jj) { return Dtt[jj * kSP + m]; });
        float* P = sP + (i - 1) * kBase * kPP;
        tile_foreach(acc, [&](int rr, int cc, float x) { P[rr * kPP + cc] = x; });
      } else {
        float* Atj = blk(t, wave - (3 - t));
        acc = lds_mfma_tile32(
            acc, [&](int ii, int m) { return -Dtt[ii * kSP + m]; },
            [&](int m, int jj) { return Atj[m * kSP + jj]; });
        tile_foreach(acc, [&](int rr, int cc, float x) { Atj[rr * kSP + cc] = x; });
      }
    }
    __syncthreads();
    if (t == 3) break;
    // Lookahead: wave 0 updates the next diagonal block (tile t + 1 of the
    // step) and factors it while waves 1..3 update the other tiles.
    const int ntile = (4 + t + 2) * (3 - t) / 2;
    if (wave == 0) {
      trailing_tile(t, t + 1);
      wave_sync();
      wave_chol_inv32(blk(t + 1, t + 1), sT, &bad);
    } else {
      for (int u = wave - 1; u < ntile - 1; u += 3) trailing_tile(t, u <= t ? u : u + 1);
    }
    __syncthreads();
  }
#pragma unroll 16
  for (int e = 0; e < kNb * kNb / 256; ++e) {
    const int idx = e * 256 + tid, i = idx >> 7, j = idx & (kNb - 1);
    const float v = (j <= i) ? sS[i * kSP + j] : 0.f;
    if (i < nbk && j < nbk) S[(k0 + i) * b + k0 + j] = v;
  }
  if (tid == 0 && bad) st->not_spd = 1;
}

__global__ __launch_bounds__(256) void diag_factor_kernel(float* __restrict__ S, int64_t b,
                                                          int64_t k0, int nbk, DevState* st) {
  // This kernel and the panel and row/column updates form the serial chain that
  // runs beside the rest set of the previous pair: their waves issue first.
  __builtin_amdgcn_s_setprio(3);
  __shared__ DiagLds L;
  if (threadIdx.x == 0) L.bad = 0;
  diag_load(S, b, k0, nbk, L.sS);
  __syncthreads();
  diag_factor_body(S, b, k0, nbk, st, L);
}

// Panel rows Lp_i live in a buffer of pitch kPP2 = 256: the panel of an even step
// in columns 0..127, of an odd step in 128..255, so the two panels of a pair of
// steps form one K = 256 operand.
constexpr int kPP2 = 2 * kNb;

// (2) Panel: blockIdx.x < nrow -> Lp for block row k+1+blockIdx.x;
//            otherwise column tile (blockIdx.x - nrow) of row k: S[k,j] = X_kk S[k,j].
__global__ __launch_bounds__(256, 2) void panel_kernel(float* __restrict__ S, int64_t b, int k,
                                                    int nbk, int nrow, float* __restrict__ P) {
  // on the serial chain (see diag_factor_kernel)
  __builtin_amdgcn_s_setprio(2);
  __shared__ __attribute__((aligned(16))) unsigned char smem[kX3LdsBytes];
  const int64_t k0 = (int64_t)k * kNb;
  f32x16_t acc[2][2];
  gemm_zero(acc);
  const float* Xkk = S + k0 * b + k0;
  if ((int)blockIdx.x < nrow) {
    const int64_t i0 = k0 + kNb + (int64_t)blockIdx.x * kNb;
    const int rows = (int)((b - i0) < kNb ? (b - i0) : kNb);
    float* Pk = P + (k & 1) * kNb;
    // A[i][kk] = S[i0+i][k0+kk]; B[kk][jj] = X_kk[jj][kk]
    gemm_tile_x3<true>(S + i0 * b + k0, b, rows, Xkk, b, nbk, nbk, acc, smem);
    gemm_foreach(acc, [&](int r, int c, float v) {
      if (r < rows && c < nbk) Pk[(i0 + r) * kPP2 + c] = v;
    });
  } else {
    const int64_t j0 = (int64_t)(blockIdx.x - nrow) * kNb;
    // A = X_kk (k-contig), B[kk][jj] = S[k0+kk][j0+jj]
    gemm_tile_x3<false>(Xkk, b, nbk, S + k0 * b + j0, b, kNb, nbk, acc, smem);
    gemm_foreach(acc, [&](int r, int c, float v) {
      if (r < nbk) S[(k0 + r) * b + j0 + c] = v;
    });
  }
}

// One tile (i, j), i > k, j <= i, of step k's trailing update:
//   C = S[i,j] - Lp_i [ X row k | X_kk | Lp_j^T ]   (j < k | j = k, C from zero | j > k)
__device__ __forceinline__ void trailing_tile(float* __restrict__ S, int64_t b, int k, int nbk,
                                              int i, int j, const float* __restrict__ P,
                                              unsigned char* smem) {
  const int64_t k0 = (int64_t)k * kNb, i0 = (int64_t)i * kNb, j0 = (int64_t)j * kNb;
  const int rows = (int)((b - i0) < kNb ? (b - i0) : kNb);
  const int cols = (int)((b - j0) < kNb ? (b - j0) : kNb);
  const float* Pk = P + (k & 1) * kNb;
  f32x16_t acc[2][2];
  float* C = S + i0 * b + j0;
  if (j == k) gemm_zero(acc);
  else gemm_load_c(acc, C, b, rows, cols);
  const float* A = Pk + i0 * kPP2;  // Lp_i, k-contig
  if (j <= k) {
    // B[kk][jj] = S[k0+kk][j0+jj]  (X row k for j < k, X_kk for j == k)
    gemm_tile_x3<false>(A, kPP2, rows, S + k0 * b + j0, b, cols, nbk, acc, smem, true);
  } else {
    // B[kk][jj] = Lp_j[jj][kk]
    gemm_tile_x3<true>(A, kPP2, rows, Pk + j0 * kPP2, kPP2, cols, nbk, acc, smem, true);
  }
  gemm_foreach(acc, [&](int r, int c, float v) {
    if (r < rows && c < cols) C[(int64_t)r * b + c] = v;
  });
}

// (3a') Step k's update of block row and column k+1 and the factorisation of
// block k+1 in one launch: workgroup 0 updates the diagonal tile (k+1, k+1) straight
// into LDS and factors it while the others update the rest of block row and
// column k+1 (read next by the panel of step k+1). Workgroup t >= 1 takes
// tile q = t - 1 (below the diagonal one) or q = t (past it), where tile q < k+2
// is (k+1, q) and otherwise (q, k+1).
__global__ __launch_bounds__(256, 2) void next_diag_kernel(float* __restrict__ S, int64_t b, int k,
                                                         int nblk, const float* __restrict__ P,
                                                         DevState* st) {
  __shared__ __attribute__((aligned(16))) DiagLds L;
  unsigned char* const smem = (unsigned char*)&L;
  if (blockIdx.x == 0) {
    __builtin_amdgcn_s_setprio(3);
    const int64_t i0 = (int64_t)(k + 1) * kNb;
    const int nbk = (int)((b - i0) < kNb ? (b - i0) : kNb);
    const float* Pk = P + (k & 1) * kNb;
    f32x16_t acc[2][2];
    gemm_load_c(acc, S + i0 * b + i0, b, nbk, nbk);
    gemm_tile_x3<true>(Pk + i0 * kPP2, kPP2, nbk, Pk + i0 * kPP2, kPP2, nbk, kNb, acc, smem, true);
    __syncthreads();  // the staging space is free again
    if (threadIdx.x == 0) L.bad = 0;
    diag_from_acc(acc, nbk, L.sS);
    __syncthreads();
    diag_factor_body(S, b, i0, nbk, st, L);
    return;
  }
  __builtin_amdgcn_s_setprio(2);
  const int t = (int)blockIdx.x - 1;
  const int q = t < k + 1 ? t : t + 1;
  if (q >= nblk) return;
  const int i = q <= k + 1 ? k + 1 : q, j = q <= k + 1 ? q : k + 1;
  trailing_tile(S, b, k, kNb, i, j, P, smem);
}

// (3b) The rest of steps k and k+1 together (k even, both blocks full): tile
// (i, j), i > k+1, j <= i, with K = 256 from the two panels [Lp_i(k) | Lp_i(k+1)]:
//   j <  k  : S[i,j] -= [Lp_i(k) Lp_i(k+1)] [S[k,j] ; S[k+1,j]]   (the final X rows)
//   j == k  : S[i,k]  = -[Lp_i(k) Lp_i(k+1)] [X_kk ; S[k+1,k]]
//   j == k+1: S[i,k+1] = -Lp_i(k+1) X_{k+1,k+1}                    (K = 128)
//   j >  k+1: S[i,j] -= [Lp_i(k) Lp_i(k+1)] [Lp_j(k)^T ; Lp_j(k+1)^T]
// Rows k and k+1 of S are adjacent, so every B operand is one contiguous slab.
__device__ __forceinline__ void pair_tile(float* __restrict__ S, int64_t b, int k, int i, int j,
                                          const float* __restrict__ P, unsigned char* smem) {
  const int64_t k0 = (int64_t)k * kNb, i0 = (int64_t)i * kNb, j0 = (int64_t)j * kNb;
  const int rows = (int)((b - i0) < kNb ? (b - i0) : kNb);
  const int cols = (int)((b - j0) < kNb ? (b - j0) : kNb);
  f32x16_t acc[2][2];
  float* C = S + i0 * b + j0;
  if (j == k || j == k + 1) gemm_zero(acc);
  else gemm_load_c(acc, C, b, rows, cols);
  const float* A = P + i0 * kPP2;
  if (j == k + 1) {
    gemm_tile_x3<false>(A + kNb, kPP2, rows, S + (k0 + kNb) * b + j0, b, cols, kNb, acc,
                               smem, true);
  } else if (j <= k) {
    gemm_tile_x3<false>(A, kPP2, rows, S + k0 * b + j0, b, cols, 2 * kNb, acc, smem, true);
  } else {
    gemm_tile_x3<true>(A, kPP2, rows, P + j0 * kPP2, kPP2, cols, 2 * kNb, acc, smem, true);
  }
  gemm_foreach(acc, [&](int r, int c, float v) {
    if (r < rows && c < cols) C[(int64_t)r * b + c] = v;
  });
}

// The pair's tiles split in two sets. "Look-ahead": block rows k+2 and k+3
// (every j <= i) and block columns k+2, k+3 below them -- everything the
// factorisation of blocks k+2 and k+3 reads. "Rest": all other tiles (i >= k+4,
// j not in {k+2, k+3}), which the next pair's trailing update is the first to
// read. The rest runs on a second stream while the next pair's diagonal blocks
// and panels run behind the look-ahead set.
__host__ __device__ inline int64_t look_tiles(int k, int nblk) {
  const int kk = k + 2;
  if (kk >= nblk) return 0;
  int64_t n = kk + 1;                                   // row kk
  if (kk + 1 < nblk) n += kk + 2;                       // row kk+1
  if (kk + 2 < nblk) n += 2 * (int64_t)(nblk - kk - 2); // columns kk, kk+1 below
  return n;
}

// The look-ahead set of pair (k, k+1) and the factorisation of block k+2 in one
// launch: workgroup 0 applies both steps to the diagonal tile (k+2, k+2) straight
// into LDS (K = 256) and factors it while the others run the rest of the
// look-ahead set; workgroup t >= 1 takes the set's tile t - 1 below the diagonal
// one and tile t past it.
__global__ __launch_bounds__(256, 2) void look_diag_kernel(float* __restrict__ S, int64_t b, int k,
                                                         int nblk, const float* __restrict__ P,
                                                         DevState* st) {
  __shared__ __attribute__((aligned(16))) DiagLds L;
  unsigned char* const smem = (unsigned char*)&L;
  const int kk = k + 2;
  if (blockIdx.x == 0) {
    __builtin_amdgcn_s_setprio(3);
    const int64_t i0 = (int64_t)kk * kNb;
    const int nbk = (int)((b - i0) < kNb ? (b - i0) : kNb);
    f32x16_t acc[2][2];
    gemm_load_c(acc, S + i0 * b + i0, b, nbk, nbk);
    gemm_tile_x3<true>(P + i0 * kPP2, kPP2, nbk, P + i0 * kPP2, kPP2, nbk, 2 * kNb, acc, smem,
                       true);
    __syncthreads();  // the staging space is free again
    if (threadIdx.x == 0) L.bad = 0;
    diag_from_acc(acc, nbk, L.sS);
    __syncthreads();
    diag_factor_body(S, b, i0, nbk, st, L);
    return;
  }
  __builtin_amdgcn_s_setprio(2);
  int q = (int)blockIdx.x - 1, i, j;
  if (q >= kk) ++q;  // (kk, kk) is workgroup 0's
  if (q <= kk) {
    i = kk; j = q;
  } else if (kk + 1 < nblk && q <= 2 * kk + 2) {
    i = kk + 1; j = q - (kk + 1);
  } else {
    q -= (kk + 1) + (kk + 1 < nblk ? kk + 2 : 0);
    i = kk + 2 + (q >> 1); j = kk + (q & 1);
    if (i >= nblk) return;
  }
  pair_tile(S, b, k, i, j, P, smem);
}

// U[a][c] = S[b-1-a][b-1-c] for c >= a (a flat reversal); 0 below the diagonal,
// everywhere (zb = 0) or only inside the diagonal blocks of size zb. Block (a, y):
// row a, columns 1024 y .. 1024 y + 1023, four per thread (16-byte accesses when
// b % 4 == 0).
__global__ __launch_bounds__(256) void reverse_kernel(const float* __restrict__ S,
                                                      float* __restrict__ U, int64_t b,
                                                      int64_t zb) {
  const int64_t a = blockIdx.x;
  const int64_t c0 = (int64_t)blockIdx.y * 1024 + threadIdx.x * 4;
  if (c0 >= b) return;
  const int64_t zfrom = zb == 0 ? 0 : a / zb * zb;  // zeros in columns [zfrom, a)
  if (c0 + 3 < zfrom) return;
  float* dst = U + a * b + c0;
  const float* src = S + (b - 1 - a) * b + (b - 1 - c0);  // src[-q] is column c0 + q
  if ((b & 3) == 0 && c0 + 3 < b) {
    if (c0 >= a) {
      const f32x4_t x = *(const f32x4_t*)(src - 3);
      *(f32x4_t*)dst = f32x4_t{x[3], x[2], x[1], x[0]};
      return;
    }
    if (c0 + 3 < a && c0 >= zfrom) {
      *(f32x4_t*)dst = f32x4_t{0.f, 0.f, 0.f, 0.f};
      return;
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t c = c0 + q;
    if (c >= b) break;
    if (c >= a) dst[q] = src[-q];
    else if (c >= zfrom) dst[q] = 0.f;
  }
}

}  // namespace

namespace {

// Two more streams and three events per device and host thread (created on
// first use, kept until the process ends). Default priority, non-blocking. s2
// runs the rest sets one after the other; s3 builds each pair's split operands
// while the previous rest set still runs. `slots` is the rest set's persistent
// grid: one workgroup per compute unit, so that every unit keeps room (LDS and
// registers) for one workgroup of the next pair's diagonal factor, panels and
// row/column update, which run beside it.
struct SideStream {
  hipStream_t s2 = nullptr, s3 = nullptr;
  hipEvent_t chain = nullptr, built = nullptr, rest = nullptr;
  int slots = 0;
};

hipError_t side_stream(SideStream*& out) {
  constexpr int kMaxDev = 64;
  thread_local SideStream tab[kMaxDev];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  SideStream& t = tab[dev];
  if (!t.s2) {
    int ncu = 0;
    if ((e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
      return e;
    if ((e = hipEventCreateWithFlags(&t.chain, hipEventDisableTiming)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&t.built, hipEventDisableTiming)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&t.rest, hipEventDisableTiming)) != hipSuccess) return e;
    if ((e = hipStreamCreateWithFlags(&t.s3, hipStreamNonBlocking)) != hipSuccess) return e;
    if ((e = hipStreamCreateWithFlags(&t.s2, hipStreamNonBlocking)) != hipSuccess) return e;
    t.slots = ncu > 0 ? ncu : 1;
  }
  out = &t;
  return hipSuccess;
}

}  // namespace

// Two panel buffers, then two pre-split Y buffers (bf16, x3_y_elems each).
size_t chol_panel_floats(int64_t b) {
  return 2 * (size_t)cdiv(b, kNb) * kNb * kPP2 + (size_t)x3_y_elems(b);
}

hipError_t launch_chol_inv_inplace(float* S, int64_t b, float* P, DevState* st, hipStream_t s) {
  const int nblk = (int)cdiv(b, kNb);
  SideStream* side = nullptr;
  hipError_t e = side_stream(side);
  if (e != hipSuccess) return e;
  // Two panel buffers: pair p writes buffer p % 2 while the rest set of pair
  // p - 1 may still read the other one; the same for the split Y buffers.
  const size_t pbuf = (size_t)cdiv(b, kNb) * kNb * kPP2;
  unsigned short* Ybase = (unsigned short*)(P + 2 * pbuf);
  const int64_t ldy = x3_ldy(b);
  const int npr = (int)cdiv(nblk, 2);
  auto factor = [&](int k) -> hipError_t {
    const int64_t k0 = (int64_t)k * kNb;
    const int nbk = (int)((b - k0) < kNb ? (b - k0) : kNb);
    hipLaunchKernelGGL(diag_factor_kernel, dim3(1), dim3(256), 0, s, S, b, k0, nbk, st);
    return hipGetLastError();
  };
  auto panel = [&](int k, float* Pp) -> hipError_t {
    const int64_t k0 = (int64_t)k * kNb;
    const int nbk = (int)((b - k0) < kNb ? (b - k0) : kNb);
    const int nrow = nblk - k - 1;
    if (nrow + k > 0) {
      hipLaunchKernelGGL(panel_kernel, dim3(nrow + k), dim3(256), 0, s, S, b, k, nbk, nrow, Pp);
      return hipGetLastError();
    }
    return hipSuccess;
  };
  // Steps in pairs (k, k+1): block row and column k+1 first, then one K = 256
  // update of everything else, split into the look-ahead set (stream s) and the
  // rest set (stream s2, on operands split on stream s3). The next pair's
  // diagonal blocks and panels wait only for the look-ahead set; the next pair's
  // look-ahead set waits for the rest set. The rest sets follow each other on s2
  // without a cross-stream wait: each waits only for its operands, which are
  // built beside the previous rest set. An odd last block is a single step.
  //
  // Buffer reuse: Y[p % 2] is written by the split of pair p after the chain of
  // pair p, which follows the look-ahead set of pair p - 1, which waited for the
  // rest set of pair p - 2 (the last reader of Y[p % 2]); P[p % 2] is rewritten
  // by the chain of pair p + 2, after the look-ahead set of pair p + 1, which
  // waited for the rest set of pair p, which waited for the split of pair p (the
  // last reader of P[p % 2] besides the look-ahead set of pair p on stream s).
  bool rest_pending = false;
  bool factored = false;  // block k's factor came with the previous look-ahead set
  for (int k = 0, pair = 0; k < nblk; k += 2, ++pair) {
    float* Pp = P + (size_t)(pair & 1) * pbuf;
    if (!factored && (e = factor(k)) != hipSuccess) return e;
    if ((e = panel(k, Pp)) != hipSuccess) return e;
    if (k + 1 >= nblk) break;
    // block row and column k+1, with block k+1 factored beside them
    hipLaunchKernelGGL(next_diag_kernel, dim3((unsigned)nblk), dim3(256), 0, s, S, b, k, nblk, Pp,
                       st);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = panel(k + 1, Pp)) != hipSuccess) return e;
    // rest set: 256 x 256 tiles over block-row pairs from (k+4)/2 (pair-row pi has
    // pi tiles: pair-columns 0..pi without (k+2)/2)
    int64_t nrest = 0;
    for (int pi = (k + 4) / 2; pi < npr; ++pi) nrest += pi;
    bool rest_now = false;
    if (nrest > 0) {
      // rows k, k+1 of S and the pair's panel buffer are final once the chain
      // reaches this point: no later step of the chain writes them before the
      // rest set has run, and the previous rest set does not touch them
      unsigned short* Yp = Ybase + (size_t)(pair & 1) * (size_t)x3_y_elems(b);
      if ((e = hipEventRecord(side->chain, s)) != hipSuccess) return e;
      if ((e = hipStreamWaitEvent(side->s3, side->chain, 0)) != hipSuccess) return e;
      hipLaunchKernelGGL(ybuild_kernel, dim3((unsigned)(ldy / 64), kX3Rows / 64), dim3(256), 0,
                         side->s3, S, b, k, Pp, Yp, ldy);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if ((e = hipEventRecord(side->built, side->s3)) != hipSuccess) return e;
      if ((e = hipStreamWaitEvent(side->s2, side->built, 0)) != hipSuccess) return e;
      // One workgroup per compute unit on 7/8 of the units: the rest keep room for
      // the next pair's chain (1/4, 1/16 and none were slower on the 11008 layer).
      // A tile takes about as long however many run beside it, so the set costs
      // whole rounds: where a grid that leaves 3/32 of the units free saves a
      // round, take it (leaving 1/16 or 1/32 free there was slower: the chain
      // beside it slows down); the grid is then spread evenly over the rounds.
      const int64_t slots = side->slots - side->slots / 8;
      const int64_t wide = side->slots - 3 * side->slots / 32;
      int64_t rounds = cdiv(nrest, slots);
      if (rounds > 1 && cdiv(nrest, rounds - 1) <= wide) --rounds;
      const int64_t grid = cdiv(nrest, rounds);
      hipLaunchKernelGGL(rest_x3_kernel, dim3((unsigned)grid), dim3(256), 0, side->s2, S, b, k, Yp,
                         ldy, nrest);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      rest_now = true;
    }
    // the previous pair's rest set covers tiles of this pair's look-ahead set
    if (rest_pending) {
      if ((e = hipStreamWaitEvent(s, side->rest, 0)) != hipSuccess) return e;
      rest_pending = false;
    }
    if (rest_now) {
      if ((e = hipEventRecord(side->rest, side->s2)) != hipSuccess) return e;
      rest_pending = true;
    }
    // the look-ahead set, with block k+2 factored beside it
    const int64_t nlook = look_tiles(k, nblk);
    factored = nlook > 0;
    if (nlook > 0) {
      hipLaunchKernelGGL(look_diag_kernel, dim3((unsigned)nlook), dim3(256), 0, s, S, b, k, nblk,
                         Pp, st);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  if (rest_pending) e = hipStreamWaitEvent(s, side->rest, 0);
  return e;
}

hipError_t launch_reverse(const float* S, float* U, int64_t b, int64_t zero_block, hipStream_t s) {
  hipLaunchKernelGGL(reverse_kernel, dim3((unsigned)b, (unsigned)cdiv(b, 1024)), dim3(256), 0, s, S,
                     U, b, zero_block);
  return hipGetLastError();
}

}  // namespace th
