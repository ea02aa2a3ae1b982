// 128x128 fp32 output tile computed on the bf16 matrix cores with three-way
// split operands (same tile, waves and accumulator layout as gemm_tile_f32).
//
// Every fp32 operand x is split into three bf16 numbers, x = h + m + l + e with
// h = bf16(x), m = bf16(x - h), l = bf16(x - h - m) (round to nearest even; the
// differences are exact in fp32), so |e| <= 2^-24 |x|. Of the nine products of
// a = ah + am + al and b = bh + bm + bl the six with weight >= 2^-16 are kept
// (ah bh, ah bm, am bh, am bm, ah bl, al bh); each is exact in fp32 and is
// accumulated in fp32 by v_mfma_f32_32x32x16_bf16. The dropped terms are below
// 2^-24 |a||b| each, so a dot product carries errors of the same order as fp32
// FMA accumulation, at six bf16 MFMAs (6 x 32 cycles per 32x32x16 block) instead
// of eight fp32 ones (8 x 64 cycles).
//
// Operands are split once, when a K step of 32 is staged in LDS, into three
// bf16 planes, laid out so that every LDS access below is free of bank conflicts
// (64 banks of 4 bytes; a 16-byte access serves 16 lanes per cycle, an 8-byte
// access 32):
//   k-contiguous operands (A always; B when B_KC): one 64-byte row of 32 k per
//     output row, its four 16-byte units XOR-swizzled by (row >> 2) & 3; MFMA
//     fragments are 16-byte reads;
//   B with k as the row index (B_KC false): rows of 128 values (256 bytes) with
//     16-byte pieces XOR-swizzled by 4 (k & 3) + (k & 1), fragments by
//     ds_read_b64_tr_b16.
#pragma once

#include "gemm_f32.h"

namespace th {

constexpr int kX3KRow = 64;                            // bytes per row of a k-contiguous plane
constexpr int kX3NRow = 256;                           // bytes per k row of an n-contiguous plane
constexpr int kX3Plane = 128 * kX3KRow;                // bytes of a plane (either layout)
static_assert(kX3Plane == 32 * kX3NRow, "both plane layouts hold 128 x 32 values");
constexpr int kX3LdsBytes = 6 * kX3Plane;              // A: 3 planes, B: 3 planes

// Byte offset of 16-byte unit u (k = 8u .. 8u+7) of row r in a k-contiguous plane.
__device__ __forceinline__ int x3_kc_off(int r, int u) {
  return r * kX3KRow + ((u ^ ((r >> 2) & 3)) << 4);
}
// Byte offset of piece fg (values 8 fg .. 8 fg + 7) of k row k in an n-contiguous plane.
__device__ __forceinline__ int x3_n_off(int k, int fg) {
  return k * kX3NRow + ((fg ^ ((k & 3) << 2) ^ (k & 1)) << 4);
}

typedef short x3_v4i16 __attribute__((ext_vector_type(4)));
typedef short x3_v8i16 __attribute__((ext_vector_type(8)));

typedef float x3_f2 __attribute__((ext_vector_type(2)));
typedef __bf16 x3_b2 __attribute__((ext_vector_type(2)));

// bf16 pair (round to nearest even, one v_cvt_pk_bf16_f32) and its exact fp32 value.
__device__ __forceinline__ unsigned x3_round2(x3_f2 v, x3_f2& back) {
  const unsigned p = __builtin_bit_cast(unsigned, __builtin_convertvector(v, x3_b2));
  back = x3_f2{__builtin_bit_cast(float, p << 16), __builtin_bit_cast(float, p & 0xffff0000u)};
  return p;
}

// Two values split at once: x = h + m + l (+ |e| <= 2^-24 |x|), each part bf16;
// h, m and l are packed pairs (element 0 in the low half).
__device__ __forceinline__ void x3_split2(x3_f2 x, unsigned& h, unsigned& m, unsigned& l) {
  x3_f2 back;
  h = x3_round2(x, back);
  const x3_f2 r1 = x - back;
  m = x3_round2(r1, back);
  const x3_f2 r2 = r1 - back;
  l = __builtin_bit_cast(unsigned, __builtin_convertvector(r2, x3_b2));
}

// Store one thread's 16 staged values, split into the three planes.
// KC: the thread holds row i = tid/2, k = 16*(tid%2) .. +15 (gemm_load_part<true>).
// !KC: the thread holds k row tid/8, values i = 16*(tid%8) .. +15.
template <bool KC>
__device__ __forceinline__ void x3_store_part(unsigned char* planes, int tid, const float (&r)[16],
                                              float sign) {
  unsigned part[3][8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
    x3_split2(x3_f2{sign * r[2 * e], sign * r[2 * e + 1]}, part[0][e], part[1][e], part[2][e]);
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    const unsigned* v = part[p];
    const u32x4_t w0 = {v[0], v[1], v[2], v[3]};
    const u32x4_t w1 = {v[4], v[5], v[6], v[7]};
    unsigned char* base = planes + p * kX3Plane;
    if (KC) {
      const int i = tid >> 1, u0 = (tid & 1) * 2;
      *(u32x4_t*)(base + x3_kc_off(i, u0)) = w0;
      *(u32x4_t*)(base + x3_kc_off(i, u0 + 1)) = w1;
    } else {
      const int k = tid >> 3, fg0 = (tid & 7) * 2;  // 8-value pieces fg0, fg0+1
      *(u32x4_t*)(base + x3_n_off(k, fg0)) = w0;
      *(u32x4_t*)(base + x3_n_off(k, fg0 + 1)) = w1;
    }
  }
}

// Fragment of 32 rows (r0 .. r0+31) x 16 k (k0 .. k0+15) of a k-contiguous plane:
// lane l holds row r0 + l%32, k0 + 8*(l/32) .. +7.
__device__ __forceinline__ bf16x8_t x3_frag_kc(const unsigned char* plane, int r0, int k0,
                                               int lane) {
  const int r = r0 + (lane & 31);
  const unsigned char* p = plane + x3_kc_off(r, (k0 >> 3) + (lane >> 5));
  return __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)p);
}

// The same fragment from an n-contiguous plane (k rows of 128 values): each
// ds_read_b64_tr_b16 transposes, per 16-lane group, 4 k x 16 n -- slot s reads k
// row tb + s/4 at n = fb + 4*(s%4); lane s then holds n = fb + s for the 4 k.
__device__ __forceinline__ bf16x8_t x3_frag_tr(const unsigned char* plane, int n0, int k0,
                                               int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int fb = n0 + ((g & 1) << 4) + ((s & 3) << 2);
  const int tb = k0 + ((g >> 1) << 3) + (s >> 2);
  const int fg = fb >> 3, within = (fb & 7) << 1;
  const x3_v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) x3_v4i16*)(plane + x3_n_off(tb, fg) + within));
  const x3_v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) x3_v4i16*)(plane + x3_n_off(tb + 4, fg) + within));
  const x3_v8i16 r = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, r);
}

// acc += (negA ? -A : A) (128 x K) * B (K x 128), A k-contiguous (A[i][k] =
// A[i*lda + k]); B[k][j] = B[j*ldb + k] if B_KC else B[k*ldb + j]. smem: at least
// kX3LdsBytes, 16-byte aligned. All 256 threads must call it.
template <bool B_KC>
__device__ __forceinline__ void gemm_tile_x3(const float* __restrict__ A, int64_t lda, int a_rows,
                                             const float* __restrict__ B, int64_t ldb, int b_cols,
                                             int K, f32x16_t (&acc)[2][2], unsigned char* smem,
                                             bool negA = false) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wi = (wave >> 1) * 64, wj = (wave & 1) * 64;
  unsigned char* sA = smem;
  unsigned char* sB = smem + 3 * kX3Plane;
  const float sign = negA ? -1.f : 1.f;
  float ra[16], rb[16];
  gemm_load_part<true>(A, lda, a_rows, K, 0, tid, ra);
  gemm_load_part<B_KC>(B, ldb, b_cols, K, 0, tid, rb);
  for (int kb = 0; kb < K; kb += kGemmBK) {
    __syncthreads();
    x3_store_part<true>(sA, tid, ra, sign);
    x3_store_part<B_KC>(sB, tid, rb, 1.f);
    __syncthreads();
    if (kb + kGemmBK < K) {
      gemm_load_part<true>(A, lda, a_rows, K, kb + kGemmBK, tid, ra);
      gemm_load_part<B_KC>(B, ldb, b_cols, K, kb + kGemmBK, tid, rb);
    }
    // zero-padded k past K contribute nothing, so both 16-k halves always run
#pragma unroll
    for (int ks = 0; ks < kGemmBK; ks += 16) {
      bf16x8_t fa[2][3], fb[2][3];
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          fa[t][p] = x3_frag_kc(sA + p * kX3Plane, wi + 32 * t, ks, lane);
          fb[t][p] = B_KC ? x3_frag_kc(sB + p * kX3Plane, wj + 32 * t, ks, lane)
                          : x3_frag_tr(sB + p * kX3Plane, wj + 32 * t, ks, lane);
        }
#pragma unroll
      for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int tj = 0; tj < 2; ++tj) {
          f32x16_t c = acc[ti][tj];
          // smallest terms first
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ti][2], fb[tj][0], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ti][0], fb[tj][2], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ti][1], fb[tj][1], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ti][1], fb[tj][0], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ti][0], fb[tj][1], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ti][0], fb[tj][0], c, 0, 0, 0);
          acc[ti][tj] = c;
        }
    }
  }
}

}  // namespace th
