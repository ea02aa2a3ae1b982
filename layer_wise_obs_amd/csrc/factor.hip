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
//            (3) trailing, one fp32 MFMA GEMM over all tiles (i > k, j <= i):
//                S[i,j] -= Lp_i [ X row k | -/X_kk | Lp_j^T ]  (j < k | j = k | j > k),
//                where column block k is overwritten with -Lp_i X_kk.
// At the end S holds L^-1 (lower); U is the element-wise reversal of S.
#include "gemm_f32.h"

namespace th {

namespace {

constexpr int kNb = 128;
constexpr int kHalf = 64;
constexpr int kSP = kNb + 1;  // LDS pitch (floats) of the 128 x 128 diagonal block

// Copy of the lane id that the compiler cannot hoist or share across the
// unrolled steps (keeps per-step lane masks short-lived).
__device__ __forceinline__ int fresh_lane() {
  int l = threadIdx.x & 63;
  __asm__ volatile("" : "+v"(l));
  return l;
}

// One wave, 64 x 64 SPD block A (lower triangle read from sm, pitch kSP):
// L = chol(A) into sl and X = L^-1 into sx (both pitch kSP, zeros above the
// diagonal). All steps are branch-free and fully unrolled so that the row
// stays in registers.
// Pass 1, right-looking Cholesky, lane i holds row i: step j needs column j of
//   the (still symmetric) trailing block -- lane c's register j, read with
//   v_readlane.
// Pass 2, forward substitution L X = I, lane j holds column j of X: row i of L
//   is read as an LDS broadcast; no synchronisation inside the loop.
__device__ __forceinline__ void wave_chol_inv64(const float* sm, float* sx, float* sl,
                                                float* scol, int* bad) {
  int flag = 0;
  {
    const int lane = threadIdx.x & 63;
    float reg[kHalf];
    static_for<0, kHalf>([&](auto C) __attribute__((always_inline)) {
      constexpr int c = C;
      reg[c] = (c <= lane) ? sm[lane * kSP + c] : sm[c * kSP + lane];
    });
    static_for<0, kHalf>([&](auto J) __attribute__((always_inline)) {
      constexpr int j = J;
      const int ln = fresh_lane();
      const float p0 = bcast(reg[j], j);
      const bool ok = (p0 > 0.f) && (p0 < 3.0e38f);
      flag |= ok ? 0 : 1;
      const float p = ok ? p0 : 1.f;
      const float sp = __builtin_sqrtf(p);
      const float rs = __builtin_amdgcn_rcpf(sp);
      const float rj = reg[j];
      const float f = (ln > j) ? rj * (rs * rs) : 0.f;
      float lv = rj * rs;
      lv = (ln > j) ? lv : 0.f;
      lv = (ln == j) ? sp : lv;
      sl[ln * kSP + j] = lv;
      static_for<j + 1, kHalf>([&](auto C) __attribute__((always_inline)) {
        constexpr int c = C;
        reg[c] = fmaf(-f, bcast(rj, c), reg[c]);
      });
    });
    wave_sync();
  }
  {
    float x[kHalf];
    static_for<0, kHalf>([&](auto I) __attribute__((always_inline)) {
      constexpr int i = I;
      const int ln = fresh_lane();
      float acc = (ln == i) ? 1.f : 0.f;
      static_for<0, i>([&](auto M) __attribute__((always_inline)) {
        constexpr int m = M;
        acc = fmaf(-sl[i * kSP + m], x[m], acc);
      });
      x[i] = acc * __builtin_amdgcn_rcpf(sl[i * kSP + i]);
    });
    const int lane = threadIdx.x & 63;
    static_for<0, kHalf>([&](auto I) __attribute__((always_inline)) {
      constexpr int i = I;
      sx[i * kSP + lane] = (i >= lane) ? x[i] : 0.f;
    });
  }
  if (flag && (threadIdx.x & 63) == 0) *bad = 1;
}

// 32 x 32 tile (this wave) of sum_m A(i, m) B(m, j), m < K, operands in LDS.
template <class FA, class FB>
__device__ __forceinline__ f32x16_t lds_mfma_tile(FA&& a, FB&& bop, int K) {
  const int lane = threadIdx.x & 63;
  const int i = lane & 31, kk = lane >> 5;
  f32x16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  for (int m = 0; m < K; m += 2)
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a(i, m + kk), bop(m + kk, i), acc, 0, 0, 0);
  return acc;
}

template <class F>
__device__ __forceinline__ void tile_foreach(const f32x16_t& acc, F&& f) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int r = 0; r < 16; ++r) f(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3), lane & 31, acc[r]);
}

// (1) Diagonal block: X_kk = L_kk^-1 with A_kk = L_kk L_kk^T, fp32, 256 threads.
// Split 2 x 2 into 64-blocks:  X11 = chol_inv(A11);  L21 = A21 X11^T;
// A22 -= L21 L21^T;  X22 = chol_inv(A22);  X21 = -X22 (L21 X11).
// A block narrower than 128 (the last one) is padded with the identity.
__global__ __launch_bounds__(256) void diag_factor_kernel(float* __restrict__ S, int64_t b,
                                                          int64_t k0, int nbk, DevState* st) {
  __shared__ float sA[kNb * kSP];
  __shared__ float sX[kNb * kSP];
  __shared__ float scol[kHalf];
  __shared__ int bad;
  const int tid = threadIdx.x, wave = tid >> 6;
  if (tid == 0) bad = 0;
  for (int e = tid; e < kNb * kNb; e += blockDim.x) {
    const int i = e / kNb, j = e % kNb;
    float v = (i == j) ? 1.f : 0.f;
    if (i < nbk && j < nbk && j <= i) v = S[(k0 + i) * b + k0 + j];
    sA[i * kSP + j] = v;
  }
  __syncthreads();
  // L11 scratch: the (not yet needed) rows 64.. of sX, columns 0..63
  if (wave == 0) wave_chol_inv64(sA, sX, sX + kHalf * kSP, scol, &bad);
  __syncthreads();
  const int ti = wave >> 1, tj = wave & 1;
  float* A21 = sA + kHalf * kSP;         // rows 64.., cols 0..63
  float* A22 = sA + kHalf * kSP + kHalf;  // rows 64.., cols 64..
  {  // L21 = A21 X11^T  (stored over A21)
    f32x16_t acc = lds_mfma_tile(
        [&](int i, int m) { return A21[(32 * ti + i) * kSP + m]; },
        [&](int m, int j) { return sX[(32 * tj + j) * kSP + m]; }, kHalf);
    __syncthreads();
    tile_foreach(acc, [&](int r, int c, float v) { A21[(32 * ti + r) * kSP + 32 * tj + c] = v; });
  }
  __syncthreads();
  {  // A22 -= L21 L21^T
    f32x16_t acc = lds_mfma_tile(
        [&](int i, int m) { return A21[(32 * ti + i) * kSP + m]; },
        [&](int m, int j) { return A21[(32 * tj + j) * kSP + m]; }, kHalf);
    tile_foreach(acc, [&](int r, int c, float v) { A22[(32 * ti + r) * kSP + 32 * tj + c] -= v; });
  }
  __syncthreads();
  float* X22 = sX + kHalf * kSP + kHalf;
  // L22 scratch: rows 64.. of sX, columns 0..63 (T is written after this)
  if (wave == 0) wave_chol_inv64(A22, X22, sX + kHalf * kSP, scol, &bad);
  __syncthreads();
  float* T = sX + kHalf * kSP;  // rows 64.., cols 0..63 of sX: T = L21 X11
  {
    f32x16_t acc = lds_mfma_tile(
        [&](int i, int m) { return A21[(32 * ti + i) * kSP + m]; },
        [&](int m, int j) { return sX[m * kSP + 32 * tj + j]; }, kHalf);
    tile_foreach(acc, [&](int r, int c, float v) { T[(32 * ti + r) * kSP + 32 * tj + c] = v; });
  }
  __syncthreads();
  {  // X21 = -X22 T  (stored over A21)
    f32x16_t acc = lds_mfma_tile(
        [&](int i, int m) { return X22[(32 * ti + i) * kSP + m]; },
        [&](int m, int j) { return T[m * kSP + 32 * tj + j]; }, kHalf);
    tile_foreach(acc, [&](int r, int c, float v) { A21[(32 * ti + r) * kSP + 32 * tj + c] = -v; });
  }
  __syncthreads();
  for (int e = tid; e < nbk * nbk; e += blockDim.x) {
    const int i = e / nbk, j = e % nbk;
    float v = 0.f;
    if (j <= i) v = (i >= kHalf && j < kHalf) ? sA[i * kSP + j] : sX[i * kSP + j];
    S[(k0 + i) * b + k0 + j] = v;
  }
  if (tid == 0 && bad) st->not_spd = 1;
}

// (2) Panel: blockIdx.x < nrow -> Lp for block row k+1+blockIdx.x;
//            otherwise column tile (blockIdx.x - nrow) of row k: S[k,j] = X_kk S[k,j].
__global__ __launch_bounds__(256, 2) void panel_kernel(float* __restrict__ S, int64_t b, int k,
                                                    int nbk, int nrow, float* __restrict__ P) {
  __shared__ __attribute__((aligned(16))) float smem[kGemmLdsFloats];
  const int64_t k0 = (int64_t)k * kNb;
  f32x16_t acc[2][2];
  gemm_zero(acc);
  const float* Xkk = S + k0 * b + k0;
  if ((int)blockIdx.x < nrow) {
    const int64_t i0 = k0 + kNb + (int64_t)blockIdx.x * kNb;
    const int rows = (int)((b - i0) < kNb ? (b - i0) : kNb);
    // A[i][kk] = S[i0+i][k0+kk]; B[kk][jj] = X_kk[jj][kk]
    gemm_tile_f32<true, true>(S + i0 * b + k0, b, rows, Xkk, b, nbk, nbk, acc, smem);
    gemm_foreach(acc, [&](int r, int c, float v) {
      if (r < rows && c < nbk) P[(i0 + r) * kNb + c] = v;
    });
  } else {
    const int64_t j0 = (int64_t)(blockIdx.x - nrow) * kNb;
    // A = X_kk (k-contig), B[kk][jj] = S[k0+kk][j0+jj]
    gemm_tile_f32<true, false>(Xkk, b, nbk, S + k0 * b + j0, b, kNb, nbk, acc, smem);
    gemm_foreach(acc, [&](int r, int c, float v) {
      if (r < nbk) S[(k0 + r) * b + j0 + c] = v;
    });
  }
}

// (3) Trailing update over tiles (i, j), k < i < nblk, 0 <= j <= i.
__global__ __launch_bounds__(256, 2) void trailing_kernel(float* __restrict__ S, int64_t b, int k,
                                                       int nbk, int nblk,
                                                       const float* __restrict__ P) {
  __shared__ __attribute__((aligned(16))) float smem[kGemmLdsFloats];
  int rem = blockIdx.x, i = k + 1;
  while (rem > i) { rem -= i + 1; ++i; }
  const int j = rem;
  if (i >= nblk) return;
  const int64_t k0 = (int64_t)k * kNb, i0 = (int64_t)i * kNb, j0 = (int64_t)j * kNb;
  const int rows = (int)((b - i0) < kNb ? (b - i0) : kNb);
  const int cols = (int)((b - j0) < kNb ? (b - j0) : kNb);
  f32x16_t acc[2][2];
  float* C = S + i0 * b + j0;
  // C = C - Lp_i B (column block k is overwritten: it starts from zero)
  if (j == k) gemm_zero(acc);
  else gemm_load_c(acc, C, b, rows, cols);
  const float* A = P + i0 * kNb;  // Lp_i, k-contig, ld kNb
  if (j <= k) {
    // B[kk][jj] = S[k0+kk][j0+jj]  (X row k for j < k, X_kk for j == k)
    gemm_tile_f32<true, false>(A, kNb, rows, S + k0 * b + j0, b, cols, nbk, acc, smem, true);
  } else {
    // B[kk][jj] = Lp_j[jj][kk]
    gemm_tile_f32<true, true>(A, kNb, rows, P + j0 * kNb, kNb, cols, nbk, acc, smem, true);
  }
  gemm_foreach(acc, [&](int r, int c, float v) {
    if (r < rows && c < cols) C[(int64_t)r * b + c] = v;
  });
}

// U[a][c] = S[b-1-a][b-1-c] for c >= a, 0 below the diagonal (a flat reversal).
__global__ void reverse_kernel(const float* __restrict__ S, float* __restrict__ U, int64_t b) {
  const int64_t n = b * b;
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < n;
       x += (int64_t)gridDim.x * blockDim.x) {
    const int64_t a = x / b, c = x - a * b;
    U[x] = (c >= a) ? S[n - 1 - x] : 0.f;
  }
}

}  // namespace

hipError_t launch_chol_inv_inplace(float* S, int64_t b, float* P, DevState* st, hipStream_t s) {
  const int nblk = (int)cdiv(b, kNb);
  for (int k = 0; k < nblk; ++k) {
    const int64_t k0 = (int64_t)k * kNb;
    const int nbk = (int)((b - k0) < kNb ? (b - k0) : kNb);
    hipLaunchKernelGGL(diag_factor_kernel, dim3(1), dim3(256), 0, s, S, b, k0, nbk, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nrow = nblk - k - 1;
    if (nrow + k > 0) {
      hipLaunchKernelGGL(panel_kernel, dim3(nrow + k), dim3(256), 0, s, S, b, k, nbk, nrow, P);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (nrow > 0) {
      // tiles: sum_{i=k+1}^{nblk-1} (i+1)
      const int64_t ntiles = (int64_t)(nblk + k + 2) * nrow / 2;
      hipLaunchKernelGGL(trailing_kernel, dim3((unsigned)ntiles), dim3(256), 0, s, S, b, k, nbk,
                         nblk, P);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

hipError_t launch_reverse(const float* S, float* U, int64_t b, hipStream_t s) {
  const int64_t n = b * b;
  int64_t blocks = cdiv(n, 256);
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(reverse_kernel, dim3((unsigned)blocks), dim3(256), 0, s, S, U, b);
  return hipGetLastError();
}

}  // namespace th
