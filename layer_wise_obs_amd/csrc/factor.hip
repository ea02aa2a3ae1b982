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
//   step k:  (1) one workgroup factors the diagonal block (fp64 in LDS):
//                L_kk and X_kk = L_kk^-1, written back as X_kk;
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
constexpr int kDP = kNb + 1;  // fp64 LDS pitch

// (1) Diagonal block: Cholesky and lower-triangular inverse in fp64.
__global__ __launch_bounds__(1024) void diag_factor_kernel(float* __restrict__ S, int64_t b,
                                                           int64_t k0, int nbk, DevState* st) {
  extern __shared__ double L[];  // nbk x kDP
  __shared__ double colv[kNb];
  const int tid = threadIdx.x, nth = blockDim.x;
  for (int e = tid; e < nbk * nbk; e += nth) {
    const int i = e / nbk, j = e % nbk;
    L[i * kDP + j] = (j <= i) ? (double)S[(k0 + i) * b + k0 + j] : 0.0;
  }
  __syncthreads();
  // Right-looking Cholesky.
  for (int j = 0; j < nbk; ++j) {
    if (tid == 0) {
      double d = L[j * kDP + j];
      if (!(d > 0.0) || !isfinite(d)) {
        st->not_spd = 1;
        d = 1.0;
      }
      L[j * kDP + j] = sqrt(d);
    }
    __syncthreads();
    const double inv = 1.0 / L[j * kDP + j];
    for (int i = j + 1 + tid; i < nbk; i += nth) L[i * kDP + j] *= inv;
    __syncthreads();
    const int m = nbk - j - 1;
    for (int e = tid; e < m * m; e += nth) {
      const int i = j + 1 + e / m, c = j + 1 + e % m;
      if (c <= i) L[i * kDP + c] -= L[i * kDP + j] * L[c * kDP + j];
    }
    __syncthreads();
  }
  // In-place inverse of the lower factor, last column first:
  // X_jj = 1/L_jj;  X[j+1:, j] = -X_jj * X[j+1:, j+1:] L[j+1:, j].
  for (int j = nbk - 1; j >= 0; --j) {
    const double xjj = 1.0 / L[j * kDP + j];
    // y_i = sum_{m=j+1..i} X[i][m] L[m][j]; 8 threads per row
    const int rows = nbk - j - 1;
    double y = 0.0;
    const int i = j + 1 + tid / 8, part = tid % 8;
    if (tid / 8 < rows) {
      for (int m = j + 1 + part; m <= i; m += 8) y += L[i * kDP + m] * L[m * kDP + j];
    }
    y += __shfl_xor(y, 1);
    y += __shfl_xor(y, 2);
    y += __shfl_xor(y, 4);
    __syncthreads();
    if (tid / 8 < rows && part == 0) colv[i] = -xjj * y;
    __syncthreads();
    if (tid / 8 < rows && part == 0) L[i * kDP + j] = colv[i];
    if (tid == 0) L[j * kDP + j] = xjj;
    __syncthreads();
  }
  for (int e = tid; e < nbk * nbk; e += nth) {
    const int i = e / nbk, j = e % nbk;
    S[(k0 + i) * b + k0 + j] = (j <= i) ? (float)L[i * kDP + j] : 0.f;
  }
}

// (2) Panel: blockIdx.x < nrow -> Lp for block row k+1+blockIdx.x;
//            otherwise column tile (blockIdx.x - nrow) of row k: S[k,j] = X_kk S[k,j].
__global__ __launch_bounds__(256) void panel_kernel(float* __restrict__ S, int64_t b, int k,
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
__global__ __launch_bounds__(256) void trailing_kernel(float* __restrict__ S, int64_t b, int k,
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
  gemm_zero(acc);
  const float* A = P + i0 * kNb;  // Lp_i, k-contig, ld kNb
  if (j <= k) {
    // B[kk][jj] = S[k0+kk][j0+jj]  (X row k for j < k, X_kk for j == k)
    gemm_tile_f32<true, false>(A, kNb, rows, S + k0 * b + j0, b, cols, nbk, acc, smem);
  } else {
    // B[kk][jj] = Lp_j[jj][kk]
    gemm_tile_f32<true, true>(A, kNb, rows, P + j0 * kNb, kNb, cols, nbk, acc, smem);
  }
  const bool overwrite = (j == k);
  gemm_foreach(acc, [&](int r, int c, float v) {
    if (r < rows && c < cols) {
      float* dst = S + (i0 + r) * b + j0 + c;
      *dst = overwrite ? -v : (*dst - v);
    }
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
    const size_t lds = (size_t)nbk * kDP * sizeof(double);
    if (k == 0) {
      hipError_t a = hipFuncSetAttribute((const void*)diag_factor_kernel,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (a != hipSuccess) return a;
    }
    hipLaunchKernelGGL(diag_factor_kernel, dim3(1), dim3(1024), lds, s, S, b, k0, nbk, st);
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
