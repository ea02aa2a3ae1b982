// Per-block slices of the inverse Hessian, prepared once per layer from U.
//
// With H^-1 = U^T U (U upper) and F = [j0, b) the active columns of block
// J = [j0, j0+B), the inverse of the active Hessian is A_F = (H_F)^-1 =
// U_FF^T U_FF, so its rows J are A_F[J, F] = U_JJ^T U[J, F] and its diagonal is
// [A_F]_qq = sum_{i=j0..q} U_iq^2. "Pruning LLMs with Thanos", section
// "Contribution one: solve a selected set directly": R = rows Q of the inverse
// Hessian, R-hat = its principal submatrix on Q -- both are slices of A_F[J, F].
//
//   save_diag_blocks : Ublk[J] = U_JJ, UblkT[J] = U_JJ^T       (B x B, zero padded)
//   transform_rows   : R[J, F] = U_JJ^T U[J, F] in place      (split-bf16 MFMA)
//   colnorm partial  : per block row J, sum over its rows i <= q of U_iq^2 (fp64)
//   colnorm scan     : D[J][q] = 1/[A_F]_qq for q in F        (OBS score weight over F)
//   block_inverses   : N[J] = (A_F[J,J])^-1 = V_JJ V_JJ^T, V_JJ = U_JJ^-1
//                      (used when a row selects more than half of a block)
#include "gemm_f32.h"
#include "gemm_x3.h"

namespace th {

namespace {

// Ublk[J] = U_JJ and UblkT[J] = U_JJ^T (upper / lower triangular, zero padded).
// Block (x, y): block jlo + x, 32 x 32 sub-tile y of it, transposed through LDS so
// that both copies are written a row at a time.
__global__ __launch_bounds__(256) void save_diag_blocks_kernel(const float* __restrict__ U,
                                                               int64_t b, int64_t B,
                                                               float* __restrict__ Ublk,
                                                               float* __restrict__ UblkT, int jlo) {
  __shared__ float tile[32][33];
  const int64_t blk = jlo + (int64_t)blockIdx.x;
  const int64_t j0 = blk * B;
  const int64_t Bb = (b - j0) < B ? (b - j0) : B;
  const int nsub = (int)cdiv(B, 32);
  const int64_t a0 = (int64_t)(blockIdx.y / nsub) * 32, c0 = (int64_t)(blockIdx.y % nsub) * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  float* dst = Ublk + blk * B * B;
  float* dstT = UblkT + blk * B * B;
  for (int r = ty; r < 32; r += 8) {
    const int64_t a = a0 + r, c = c0 + tx;
    const float v = (a < Bb && c < Bb && c >= a) ? U[(j0 + a) * b + j0 + c] : 0.f;
    if (a < B && c < B) dst[a * B + c] = v;
    tile[r][tx] = v;
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int64_t c = c0 + r, a = a0 + tx;  // dstT[c][a] = U_JJ[a][c]
    if (a < B && c < B) dstT[c * B + a] = tile[tx][r];
  }
}

// One workgroup per (block J, 128-wide column tile of F): the product on the bf16
// matrix cores with split fp32 operands (errors of the order of fp32 accumulation).
__global__ __launch_bounds__(256, 2) void transform_rows_kernel(float* __restrict__ R, int64_t b,
                                                             int64_t B, int nblk,
                                                             const float* __restrict__ UblkT,
                                                             int jlo) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kX3LdsBytes];
  int rem = blockIdx.x, blk = jlo;
  int64_t ntile = 0;
  for (;;) {
    const int64_t j0 = (int64_t)blk * B;
    ntile = cdiv(b - j0, 128);
    if (rem < ntile) break;
    rem -= (int)ntile;
    ++blk;
    if (blk >= nblk) return;
  }
  const int64_t j0 = (int64_t)blk * B;
  const int Bb = (int)((b - j0) < B ? (b - j0) : B);
  const int64_t col0 = j0 + (int64_t)rem * 128;
  const int cols = (int)((b - col0) < 128 ? (b - col0) : 128);
  f32x16_t acc[2][2];
  gemm_zero(acc);
  // A[i][kk] = U_JJ[kk][i] = UblkT[i][kk] (k contiguous), B[kk][jj] = U[j0+kk][col0+jj]
  gemm_tile_x3<false>(UblkT + (int64_t)blk * B * B, B, Bb, R + j0 * b + col0, b, cols, Bb, acc,
                      smem);
  gemm_foreach(acc, [&](int r, int c, float v) {
    if (r < Bb && c < cols) R[(j0 + r) * b + col0 + c] = v;
  });
}

// The column sums in two coalesced passes: P[r][q] = sum over rows i of block r
// with i <= q of U_iq^2 (one workgroup per block row and 256 columns), then per
// column a suffix sum over the blocks, stored as its reciprocal:
// D[r][q] = 1 / sum_{r' >= r} P[r'][q], q >= r B.
__global__ void colnorm_partial_kernel(const float* __restrict__ U, int64_t b, int64_t B,
                                       double* __restrict__ P, int jlo) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t r = jlo + (int64_t)blockIdx.y;
  if (q >= b) return;
  const int64_t j0 = r * B;
  const int64_t j1 = (j0 + B) < b ? (j0 + B) : b;
  double s = 0.0;
  for (int64_t i = j0; i < j1; ++i) {
    const double u = (i <= q) ? (double)U[i * b + q] : 0.0;
    s += u * u;
  }
  P[r * b + q] = s;
}

__global__ void colnorm_scan_kernel(const double* __restrict__ P, int64_t b, int64_t B, int nblk,
                                    float* __restrict__ D) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= b) return;
  double s = 0.0;
  for (int r = nblk - 1; r >= 0; --r) {
    s += P[(int64_t)r * b + q];
    if (q >= (int64_t)r * B) D[(int64_t)r * b + q] = __fdiv_rn(1.0f, (float)s);
  }
}

// N = (U_JJ^T U_JJ)^-1 = V V^T with V = U_JJ^-1 (upper), in fp64.
__global__ __launch_bounds__(1024) void block_inverse_kernel(const float* __restrict__ Ublk,
                                                             int64_t b, int64_t B,
                                                             float* __restrict__ Nblk, int jlo) {
  extern __shared__ double V[];  // B x (B+1)
  const int64_t P = B + 1;
  const int64_t blk = jlo + (int64_t)blockIdx.x;
  const int64_t j0 = blk * B;
  const int Bb = (int)((b - j0) < B ? (b - j0) : B);
  const float* Ub = Ublk + blk * B * B;
  const int tid = threadIdx.x, nth = blockDim.x;
  for (int64_t e = tid; e < (int64_t)Bb * Bb; e += nth) {
    const int a = (int)(e / Bb), c = (int)(e % Bb);
    V[a * P + c] = (c >= a) ? (double)Ub[a * B + c] : 0.0;
  }
  __syncthreads();
  // In-place upper-triangular inverse, first column first:
  // V_jj = 1/U_jj;  V[0:j, j] = -V_jj * V[0:j, 0:j] U[0:j, j].
  __shared__ double colv[kMaxBlock];
  for (int j = 0; j < Bb; ++j) {
    const double vjj = 1.0 / V[j * P + j];
    const int i = tid / 8, part = tid % 8;
    double y = 0.0;
    if (i < j) {
      for (int m = i + part; m < j; m += 8) y += V[i * P + m] * V[m * P + j];
    }
    y += __shfl_xor(y, 1);
    y += __shfl_xor(y, 2);
    y += __shfl_xor(y, 4);
    __syncthreads();
    if (i < j && part == 0) colv[i] = -vjj * y;
    __syncthreads();
    if (i < j && part == 0) V[i * P + j] = colv[i];
    if (tid == 0) V[j * P + j] = vjj;
    __syncthreads();
  }
  float* Nb = Nblk + blk * B * B;
  for (int64_t e = tid; e < B * B; e += nth) {
    const int a = (int)(e / B), c = (int)(e % B);
    double s = 0.0;
    if (a < Bb && c < Bb) {
      const int from = a > c ? a : c;
      for (int m = from; m < Bb; ++m) s += V[a * P + m] * V[c * P + m];
    }
    Nb[e] = (float)s;
  }
}

}  // namespace

hipError_t launch_save_diag_blocks(const float* U, int64_t b, int64_t B, float* Ublk, float* UblkT,
                                   int jlo, int jhi, hipStream_t s) {
  if (jhi <= jlo) return hipSuccess;
  const unsigned nsub = (unsigned)cdiv(B, 32);
  hipLaunchKernelGGL(save_diag_blocks_kernel, dim3(jhi - jlo, nsub * nsub), dim3(256), 0, s, U, b,
                     B, Ublk, UblkT, jlo);
  return hipGetLastError();
}

hipError_t launch_transform_rows(float* R, int64_t b, int64_t B, const float* UblkT, int jlo,
                                 int jhi, hipStream_t s) {
  if (jhi <= jlo) return hipSuccess;
  int64_t total = 0;
  for (int k = jlo; k < jhi; ++k) total += cdiv(b - (int64_t)k * B, 128);
  hipLaunchKernelGGL(transform_rows_kernel, dim3((unsigned)total), dim3(256), 0, s, R, b, B, jhi,
                     UblkT, jlo);
  return hipGetLastError();
}

hipError_t launch_colnorm_partial(const float* U, int64_t b, int64_t B, double* Dpart, int jlo,
                                  int jhi, hipStream_t s) {
  if (jhi <= jlo) return hipSuccess;
  hipLaunchKernelGGL(colnorm_partial_kernel, dim3((unsigned)cdiv(b, 256), (unsigned)(jhi - jlo)),
                     dim3(256), 0, s, U, b, B, Dpart, jlo);
  return hipGetLastError();
}

hipError_t launch_colnorm_scan(const double* Dpart, int64_t b, int64_t B, float* D, hipStream_t s) {
  hipLaunchKernelGGL(colnorm_scan_kernel, dim3((unsigned)cdiv(b, 256)), dim3(256), 0, s, Dpart, b,
                     B, (int)cdiv(b, B), D);
  return hipGetLastError();
}

hipError_t launch_block_inverses(const float* Ublk, int64_t b, int64_t B, float* Nblk, int jlo,
                                 int jhi, hipStream_t s) {
  if (jhi <= jlo) return hipSuccess;
  const size_t lds = (size_t)B * (B + 1) * sizeof(double);
  hipError_t a = hipFuncSetAttribute((const void*)block_inverse_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (a != hipSuccess) return a;
  hipLaunchKernelGGL(block_inverse_kernel, dim3(jhi - jlo), dim3(1024), lds, s, Ublk, b, B, Nblk,
                     jlo);
  return hipGetLastError();
}

}  // namespace th
