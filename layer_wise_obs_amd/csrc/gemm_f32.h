// 128x128 fp32 output tile on the CDNA4 fp32 matrix cores
// (v_mfma_f32_32x32x2_f32), 256 threads = 4 waves, each wave owning a 64x64
// quadrant as 2x2 MFMA blocks of 32x32. K is staged through LDS in steps of 32
// with the next step's global loads in flight during the current step's MFMAs.
//
// Operand layouts are compile-time:
//   A_KC: A[i][k] = A[i*lda + k]   (k contiguous)   else A[k*lda + i]
//   B_KC: B[k][j] = B[j*ldb + k]   (k contiguous)   else B[k*ldb + j]
// Pointers point at the tile origin; a_rows / b_cols / K bound the valid
// region, everything outside reads as zero. With negA the tile computes
// acc -= A*B (A is negated on its way into LDS), so an accumulator preloaded
// with C (gemm_load_c) yields C - A*B without a read in the epilogue.
//
// Accumulator layout of one 32x32 block (lane l, register r):
//   row = 8*(r/4) + 4*(l/32) + (r%4), col = l%32.
#pragma once

#include "common.h"

namespace th {

// threadIdx.x through an empty asm: index math derived from it cannot be shared
// with (and kept alive from) an earlier use, e.g. the C-tile addresses of the
// load before the K loop and of the stores after it.
__device__ __forceinline__ int opaque_tid() {
  int t = threadIdx.x;
  __asm__ volatile("" : "+v"(t));
  return t;
}

constexpr int kGemmBK = 32;
constexpr int kGemmLdsPitch = 132;  // floats per staged k-row (128 + 4)
constexpr int kGemmLdsFloats = 2 * kGemmBK * kGemmLdsPitch;

// 16 values of one thread's share of a 128 x 32 operand tile.
template <bool KC>
__device__ __forceinline__ void gemm_load_part(const float* __restrict__ P, int64_t ld, int nvalid,
                                               int K, int kb, int tid, float (&r)[16]) {
  if (KC) {  // thread: row i, 16 consecutive k
    const int i = tid >> 1, k0 = kb + (tid & 1) * 16;
    const float* src = P + (int64_t)i * ld + k0;
    if (i < nvalid && k0 + 16 <= K && ((((uintptr_t)src) & 15) == 0)) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4_t v = *(const f32x4_t*)(src + 4 * q);
        r[4 * q] = v[0]; r[4 * q + 1] = v[1]; r[4 * q + 2] = v[2]; r[4 * q + 3] = v[3];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) r[e] = (i < nvalid && k0 + e < K) ? src[e] : 0.f;
    }
  } else {  // thread: k row, 16 consecutive i
    const int k = kb + (tid >> 3), i0 = (tid & 7) * 16;
    const float* src = P + (int64_t)k * ld + i0;
    if (k < K && i0 + 16 <= nvalid && ((((uintptr_t)src) & 15) == 0)) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4_t v = *(const f32x4_t*)(src + 4 * q);
        r[4 * q] = v[0]; r[4 * q + 1] = v[1]; r[4 * q + 2] = v[2]; r[4 * q + 3] = v[3];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) r[e] = (k < K && i0 + e < nvalid) ? src[e] : 0.f;
    }
  }
}

template <bool KC>
__device__ __forceinline__ void gemm_store_part(float* __restrict__ sm, int tid, const float (&r)[16],
                                                float sign) {
  if (KC) {
    const int i = tid >> 1, k0 = (tid & 1) * 16;
#pragma unroll
    for (int e = 0; e < 16; ++e) sm[(k0 + e) * kGemmLdsPitch + i] = sign * r[e];
  } else {
    const int k = tid >> 3, i0 = (tid & 7) * 16;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *(f32x4_t*)(sm + k * kGemmLdsPitch + i0 + 4 * q) =
          f32x4_t{sign * r[4 * q], sign * r[4 * q + 1], sign * r[4 * q + 2], sign * r[4 * q + 3]};
  }
}

__device__ __forceinline__ void gemm_zero(f32x16_t (&acc)[2][2]) {
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][c][r] = 0.f;
}

// Visit every accumulator element with its tile-local (row, col).
template <class F>
__device__ __forceinline__ void gemm_foreach(const f32x16_t (&acc)[2][2], F&& f) {
  const int tid = opaque_tid();
  const int lane = tid & 63, wave = tid >> 6;
  const int wi = (wave >> 1) * 64, wj = (wave & 1) * 64;
#pragma unroll
  for (int ti = 0; ti < 2; ++ti)
#pragma unroll
    for (int tj = 0; tj < 2; ++tj)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wi + ti * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = wj + tj * 32 + (lane & 31);
        f(row, col, acc[ti][tj][r]);
      }
}

// acc = C (row-major, ldc) on the valid rows x cols, 0 elsewhere.
__device__ __forceinline__ void gemm_load_c(f32x16_t (&acc)[2][2], const float* __restrict__ C,
                                            int64_t ldc, int rows, int cols) {
  const int tid = opaque_tid();
  const int lane = tid & 63, wave = tid >> 6;
  const int wi = (wave >> 1) * 64, wj = (wave & 1) * 64;
#pragma unroll
  for (int ti = 0; ti < 2; ++ti)
#pragma unroll
    for (int tj = 0; tj < 2; ++tj)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wi + ti * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = wj + tj * 32 + (lane & 31);
        acc[ti][tj][r] = (row < rows && col < cols) ? C[(int64_t)row * ldc + col] : 0.f;
      }
}

// acc += (negA ? -A : A) (128 x K) * B (K x 128). All 256 threads must call it.
template <bool A_KC, bool B_KC>
__device__ __forceinline__ void gemm_tile_f32(const float* __restrict__ A, int64_t lda, int a_rows,
                                              const float* __restrict__ B, int64_t ldb, int b_cols,
                                              int K, f32x16_t (&acc)[2][2], float* smem,
                                              bool negA = false) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wi = (wave >> 1) * 64, wj = (wave & 1) * 64;
  float* sA = smem;
  float* sB = smem + kGemmBK * kGemmLdsPitch;
  const float sign = negA ? -1.f : 1.f;
  float ra[16], rb[16];
  gemm_load_part<A_KC>(A, lda, a_rows, K, 0, tid, ra);
  gemm_load_part<B_KC>(B, ldb, b_cols, K, 0, tid, rb);
  const int lr = lane & 31, lk = lane >> 5;
  for (int kb = 0; kb < K; kb += kGemmBK) {
    __syncthreads();
    gemm_store_part<A_KC>(sA, tid, ra, sign);
    gemm_store_part<B_KC>(sB, tid, rb, 1.f);
    __syncthreads();
    if (kb + kGemmBK < K) {
      gemm_load_part<A_KC>(A, lda, a_rows, K, kb + kGemmBK, tid, ra);
      gemm_load_part<B_KC>(B, ldb, b_cols, K, kb + kGemmBK, tid, rb);
    }
    const int kmax = (K - kb) < kGemmBK ? (K - kb) : kGemmBK;
    if (kmax == kGemmBK) {
#pragma unroll
      for (int kk = 0; kk < kGemmBK; kk += 2) {
        const float* pa = sA + (kk + lk) * kGemmLdsPitch + wi + lr;
        const float* pb = sB + (kk + lk) * kGemmLdsPitch + wj + lr;
        const float a0 = pa[0], a1 = pa[32];
        const float b0 = pb[0], b1 = pb[32];
        acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
        acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
        acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
        acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
      }
    } else {
      for (int kk = 0; kk < kmax; kk += 2) {  // zero-padded rows past K
        const float* pa = sA + (kk + lk) * kGemmLdsPitch + wi + lr;
        const float* pb = sB + (kk + lk) * kGemmLdsPitch + wj + lr;
        const float a0 = pa[0], a1 = pa[32];
        const float b0 = pb[0], b1 = pb[32];
        acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
        acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
        acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
        acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
      }
    }
  }
}

}  // namespace th

namespace th {

// ---- 64x64 variant: 256 threads = 4 waves, each wave one 32x32 MFMA block.
// For short GEMMs with few output tiles (block-local updates, panels), where
// more and smaller workgroups finish sooner than a few 128x128 ones.
constexpr int kG64Pitch = 68;  // floats per staged k-row (64 + 4)
constexpr int kG64LdsFloats = 2 * kGemmBK * kG64Pitch;

template <bool KC>
__device__ __forceinline__ void g64_load_part(const float* __restrict__ P, int64_t ld, int nvalid,
                                              int K, int kb, int tid, float (&r)[8]) {
  if (KC) {  // thread: row i, 8 consecutive k
    const int i = tid >> 2, k0 = kb + (tid & 3) * 8;
    const float* src = P + (int64_t)i * ld + k0;
    if (i < nvalid && k0 + 8 <= K && ((((uintptr_t)src) & 15) == 0)) {
      const f32x4_t v0 = *(const f32x4_t*)src, v1 = *(const f32x4_t*)(src + 4);
      r[0] = v0[0]; r[1] = v0[1]; r[2] = v0[2]; r[3] = v0[3];
      r[4] = v1[0]; r[5] = v1[1]; r[6] = v1[2]; r[7] = v1[3];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] = (i < nvalid && k0 + e < K) ? src[e] : 0.f;
    }
  } else {  // thread: k row, 8 consecutive i
    const int k = kb + (tid >> 3), i0 = (tid & 7) * 8;
    const float* src = P + (int64_t)k * ld + i0;
    if (k < K && i0 + 8 <= nvalid && ((((uintptr_t)src) & 15) == 0)) {
      const f32x4_t v0 = *(const f32x4_t*)src, v1 = *(const f32x4_t*)(src + 4);
      r[0] = v0[0]; r[1] = v0[1]; r[2] = v0[2]; r[3] = v0[3];
      r[4] = v1[0]; r[5] = v1[1]; r[6] = v1[2]; r[7] = v1[3];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] = (k < K && i0 + e < nvalid) ? src[e] : 0.f;
    }
  }
}

template <bool KC>
__device__ __forceinline__ void g64_store_part(float* __restrict__ sm, int tid, const float (&r)[8],
                                               float sign) {
  if (KC) {
    const int i = tid >> 2, k0 = (tid & 3) * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) sm[(k0 + e) * kG64Pitch + i] = sign * r[e];
  } else {
    const int k = tid >> 3, i0 = (tid & 7) * 8;
    *(f32x4_t*)(sm + k * kG64Pitch + i0) = f32x4_t{sign * r[0], sign * r[1], sign * r[2], sign * r[3]};
    *(f32x4_t*)(sm + k * kG64Pitch + i0 + 4) =
        f32x4_t{sign * r[4], sign * r[5], sign * r[6], sign * r[7]};
  }
}

// Visit every accumulator element of the 64x64 tile with its tile-local (row, col).
template <class F>
__device__ __forceinline__ void g64_foreach(const f32x16_t& acc, F&& f) {
  const int tid = opaque_tid();
  const int lane = tid & 63, wave = tid >> 6;
  const int wi = (wave >> 1) * 32, wj = (wave & 1) * 32;
#pragma unroll
  for (int r = 0; r < 16; ++r)
    f(wi + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3), wj + (lane & 31), acc[r]);
}

__device__ __forceinline__ void g64_load_c(f32x16_t& acc, const float* __restrict__ C, int64_t ldc,
                                           int rows, int cols) {
  const int tid = opaque_tid();
  const int lane = tid & 63, wave = tid >> 6;
  const int wi = (wave >> 1) * 32, wj = (wave & 1) * 32;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = wi + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    const int col = wj + (lane & 31);
    acc[r] = (row < rows && col < cols) ? C[(int64_t)row * ldc + col] : 0.f;
  }
}

// acc += (negA ? -A : A) (64 x K) * B (K x 64). All 256 threads must call it.
template <bool A_KC, bool B_KC>
__device__ __forceinline__ void g64_tile_f32(const float* __restrict__ A, int64_t lda, int a_rows,
                                             const float* __restrict__ B, int64_t ldb, int b_cols,
                                             int K, f32x16_t& acc, float* smem,
                                             bool negA = false) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wi = (wave >> 1) * 32, wj = (wave & 1) * 32;
  float* sA = smem;
  float* sB = smem + kGemmBK * kG64Pitch;
  const float sign = negA ? -1.f : 1.f;
  float ra[8], rb[8];
  g64_load_part<A_KC>(A, lda, a_rows, K, 0, tid, ra);
  g64_load_part<B_KC>(B, ldb, b_cols, K, 0, tid, rb);
  const int lr = lane & 31, lk = lane >> 5;
  for (int kb = 0; kb < K; kb += kGemmBK) {
    __syncthreads();
    g64_store_part<A_KC>(sA, tid, ra, sign);
    g64_store_part<B_KC>(sB, tid, rb, 1.f);
    __syncthreads();
    if (kb + kGemmBK < K) {
      g64_load_part<A_KC>(A, lda, a_rows, K, kb + kGemmBK, tid, ra);
      g64_load_part<B_KC>(B, ldb, b_cols, K, kb + kGemmBK, tid, rb);
    }
    const int kmax = (K - kb) < kGemmBK ? (K - kb) : kGemmBK;
    if (kmax == kGemmBK) {
#pragma unroll
      for (int kk = 0; kk < kGemmBK; kk += 2)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(sA[(kk + lk) * kG64Pitch + wi + lr],
                                                   sB[(kk + lk) * kG64Pitch + wj + lr], acc, 0, 0, 0);
    } else {
      for (int kk = 0; kk < kmax; kk += 2)  // zero-padded rows past K
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(sA[(kk + lk) * kG64Pitch + wi + lr],
                                                   sB[(kk + lk) * kG64Pitch + wj + lr], acc, 0, 0, 0);
    }
  }
}

}  // namespace th
