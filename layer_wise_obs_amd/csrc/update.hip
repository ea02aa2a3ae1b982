// Compensation update, dtype conversions and the reconstruction error.
//
// Update ("Pruning LLMs with Thanos", sections "Contribution one" and "The scaling
// problem, and what SparseGPT changes": only still-active columns receive
// compensation): W[:, F] -= Z [A_F]_{J,F}, a rank-B update (128 x 128 tiles on
// the bf16 matrix cores with three-way split fp32 operands, gemm_x3.h; 64 x 64
// tiles on the fp32 matrix cores for launches with few tiles), after which the
// pruned entries of block J are set to exactly zero.
// The kernel takes any column range and any K, so the host code can split one
// block's update into the columns it needs now and a deferred part that is
// applied for several blocks at once (K = several blocks).
//
// Error ("The layer-reconstruction lens"): E = ||(W - What) X||_F^2 =
// sum_k D_k G D_k^T, computed as T = D G per 128x128 tile (fp32 MFMA) with the
// tile's sum of T .* D in fp64; partial sums are reduced in a fixed order.
#include "gemm_x3.h"

namespace th {

namespace {

// First radix digit of the selection keys of the next block (unstructured): the
// update writes every weight of the next active region, so it histograms the top
// 11 bits of their 64-bit keys (the score bits >> 21: the flat index does not
// reach that digit) exactly as the first selection pass would, into an LDS
// histogram that is added to the global one at the end (integer counts, so the
// result is that of the pass). hist_zero / hist_add / hist_flush are no-ops
// without HIST.
template <bool HIST>
struct NextDigit {
  unsigned int* sh;
  __device__ __forceinline__ void zero() {
    if constexpr (HIST)
      for (int i = threadIdx.x; i < kSelBins; i += blockDim.x) sh[i] = 0u;
  }
  __device__ __forceinline__ void add(float w, float g) {
    if constexpr (HIST) atomicAdd(&sh[__float_as_uint(score_of(w, g)) >> 21], 1u);
  }
  // hist: kSelCopies histograms of kSelBins; this workgroup adds to copy i % kSelCopies
  __device__ __forceinline__ void flush(unsigned int* __restrict__ hist) {
    if constexpr (HIST) {
      __syncthreads();
      unsigned int* gh = hist + (blockIdx.x % kSelCopies) * kSelBins;
      for (int i = threadIdx.x; i < kSelBins; i += blockDim.x)
        if (sh[i]) atomicAdd(&gh[i], sh[i]);
    }
  }
};

// W[row0:, col0:] -= Z[rows, 0:K] R[r0:r0+K, cols]; zero the pruned entries of
// columns [mask_j0, mask_jend); with HIST, the first key digit of columns >= hist_j0.
// Tiles t = blockIdx.x + i gridDim.x: with HIST the grid is a few workgroups per
// compute unit, so that each one adds its histogram to the global one once, after
// all its tiles (the global atomics of one flush per tile met on the same bins).
template <bool HIST>
__global__ __launch_bounds__(256, 2) void update_kernel(float* __restrict__ W, int64_t c, int64_t b,
                                                     int64_t r0, int K, int64_t ldz,
                                                     int64_t col_begin, int64_t col_end,
                                                     int ncol_tiles, int64_t ntiles,
                                                     const float* __restrict__ Z,
                                                     const float* __restrict__ R,
                                                     const uint8_t* __restrict__ mask,
                                                     int64_t mask_j0, int64_t mask_jend,
                                                     const float* __restrict__ gn, int64_t hist_j0,
                                                     unsigned int* __restrict__ hist) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kX3LdsBytes];
  NextDigit<HIST> nd;
  if constexpr (HIST) {
    __shared__ unsigned int sh[kSelBins];
    nd.sh = sh;
  }
  nd.zero();
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
  // every wave is done with the previous tile's operands before they are restaged
  if (t != (int64_t)blockIdx.x) __syncthreads();
  const int64_t row0 = (t / ncol_tiles) * 128;
  const int64_t col0 = col_begin + (t % ncol_tiles) * 128;
  const int rows = (int)((c - row0) < 128 ? (c - row0) : 128);
  const int cols = (int)((col_end - col0) < 128 ? (col_end - col0) : 128);
  // score weights of this lane's two columns (wave column 64 (wave & 1), then +32),
  // loaded before the GEMM so that their latency hides behind it
  float gv[2] = {0.f, 0.f};
  if constexpr (HIST) {
    const int cl = (int)((threadIdx.x >> 6) & 1) * 64 + (int)(threadIdx.x & 31);
#pragma unroll
    for (int tj = 0; tj < 2; ++tj)
      if (cl + 32 * tj < cols && col0 + cl + 32 * tj >= hist_j0) gv[tj] = gn[col0 + cl + 32 * tj];
  }
  f32x16_t acc[2][2];
  float* C = W + row0 * b + col0;
  gemm_load_c(acc, C, b, rows, cols);  // W tile, then W - Z R
  gemm_tile_x3<false>(Z + row0 * ldz, ldz, rows, R + r0 * b + col0, b, cols, K, acc, smem,
                             true);
  const bool masked = col0 < mask_jend && col0 + 128 > mask_j0;
  gemm_foreach(acc, [&](int r, int cc, float v) {
    if (r < rows && cc < cols) {
      const int64_t row = row0 + r, col = col0 + cc;
      if (masked && col >= mask_j0 && col < mask_jend && mask[row * b + col]) v = 0.f;
      W[row * b + col] = v;
      if (HIST && col >= hist_j0) nd.add(v, gv[(cc >> 5) & 1]);
    }
  });
  }
  nd.flush(hist);
}

// The same update on 64 x 64 tiles, for launches with few 128 x 128 tiles.
template <bool HIST>
__global__ __launch_bounds__(256, 2) void update64_kernel(float* __restrict__ W, int64_t c,
                                                       int64_t b, int64_t r0, int K, int64_t ldz,
                                                       int64_t col_begin, int64_t col_end,
                                                       int ncol_tiles, const float* __restrict__ Z,
                                                       const float* __restrict__ R,
                                                       const uint8_t* __restrict__ mask,
                                                       int64_t mask_j0, int64_t mask_jend,
                                                       const float* __restrict__ gn,
                                                       int64_t hist_j0,
                                                       unsigned int* __restrict__ hist) {
  __shared__ __attribute__((aligned(16))) float smem[kG64LdsFloats];
  NextDigit<HIST> nd;
  if constexpr (HIST) {
    __shared__ unsigned int sh[kSelBins];
    nd.sh = sh;
  }
  nd.zero();
  const int64_t row0 = (int64_t)(blockIdx.x / ncol_tiles) * 64;
  const int64_t col0 = col_begin + (int64_t)(blockIdx.x % ncol_tiles) * 64;
  const int rows = (int)((c - row0) < 64 ? (c - row0) : 64);
  const int cols = (int)((col_end - col0) < 64 ? (col_end - col0) : 64);
  f32x16_t acc;
  float* C = W + row0 * b + col0;
  g64_load_c(acc, C, b, rows, cols);
  g64_tile_f32<true, false>(Z + row0 * ldz, ldz, rows, R + r0 * b + col0, b, cols, K, acc, smem,
                            true);
  const bool masked = col0 < mask_jend && col0 + 64 > mask_j0;
  // score weight of this lane's column (wave column 32 (wave & 1)), loaded before
  // the stores so that no load waits inside the loop below
  float gv = 0.f;
  if constexpr (HIST) {
    const int cl = (int)((threadIdx.x >> 6) & 1) * 32 + (int)(threadIdx.x & 31);
    if (cl < cols && col0 + cl >= hist_j0) gv = gn[col0 + cl];
  }
  g64_foreach(acc, [&](int r, int cc, float v) {
    if (r < rows && cc < cols) {
      const int64_t row = row0 + r, col = col0 + cc;
      if (masked && col >= mask_j0 && col < mask_jend && mask[row * b + col]) v = 0.f;
      W[row * b + col] = v;
      if (HIST && col >= hist_j0) nd.add(v, gv);
    }
  });
  nd.flush(hist);
}

__global__ void to_f32_kernel(const void* __restrict__ src, int dt, int64_t n,
                              float* __restrict__ dst, DevState* st) {
  int bad = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const float v = (dt == TH_BF16) ? bf16_to_f32(((const unsigned short*)src)[i])
                                    : ((const float*)src)[i];
    if (!isfinite(v)) bad = 1;
    dst[i] = v;
  }
  if (bad && st) st->nonfinite = 1;
}

// Clears memory with vector stores (16 bytes per thread and step; a byte tail):
// used instead of a runtime memset so that every step of a layer call is a kernel.
__global__ void zero_kernel(uint4* __restrict__ p16, int64_t n16, unsigned char* __restrict__ tail,
                            int ntail) {
  const uint4 z = make_uint4(0u, 0u, 0u, 0u);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * blockDim.x)
    p16[i] = z;
  if (blockIdx.x == 0 && (int)threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

__global__ void from_f32_kernel(const float* __restrict__ src, int64_t n, int dt,
                                void* __restrict__ dst) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    if (dt == TH_BF16) ((unsigned short*)dst)[i] = f32_to_bf16_rne(src[i]);
    else ((float*)dst)[i] = src[i];
  }
}

__global__ void diff_kernel(const void* __restrict__ A, const void* __restrict__ B, int dt,
                            int64_t n, float* __restrict__ D) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    float a, bb;
    if (dt == TH_BF16) {
      a = bf16_to_f32(((const unsigned short*)A)[i]);
      bb = bf16_to_f32(((const unsigned short*)B)[i]);
    } else {
      a = ((const float*)A)[i];
      bb = ((const float*)B)[i];
    }
    D[i] = a - bb;
  }
}

// partial[tile] = sum over the tile of (D G) .* D   (G full symmetric, b x b)
__global__ __launch_bounds__(256, 2) void quadform_kernel(const float* __restrict__ D, int64_t c,
                                                       int64_t b, int ncol_tiles,
                                                       const float* __restrict__ G,
                                                       double* __restrict__ partials) {
  __shared__ __attribute__((aligned(16))) float smem[kGemmLdsFloats];
  __shared__ double red[256];
  const int64_t row0 = (int64_t)(blockIdx.x / ncol_tiles) * 128;
  const int64_t col0 = (int64_t)(blockIdx.x % ncol_tiles) * 128;
  const int rows = (int)((c - row0) < 128 ? (c - row0) : 128);
  const int cols = (int)((b - col0) < 128 ? (b - col0) : 128);
  f32x16_t acc[2][2];
  gemm_zero(acc);
  gemm_tile_f32<true, false>(D + row0 * b, b, rows, G + col0, b, cols, (int)b, acc, smem);
  double s = 0.0;
  gemm_foreach(acc, [&](int r, int cc, float v) {
    if (r < rows && cc < cols) s += (double)v * (double)D[(row0 + r) * b + col0 + cc];
  });
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) partials[blockIdx.x] = red[0];
}

__global__ void sum_kernel(const double* __restrict__ p, int64_t n, double* __restrict__ out) {
  __shared__ double red[256];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) s += p[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = red[0];
}

unsigned ew_grid(int64_t n) {
  int64_t g = cdiv(n, 256 * 4);
  if (g > 16384) g = 16384;
  if (g < 1) g = 1;
  return (unsigned)g;
}

}  // namespace

bool update_large_tiles(int64_t c, int64_t col0, int64_t col_end) {
  // under ~4 tiles per CU the 64 x 64 tiles finish sooner
  return cdiv(col_end - col0, 128) * cdiv(c, 128) >= 1024;
}

hipError_t launch_update(float* W, int64_t c, int64_t b, int64_t r0, int64_t K, int64_t ldz,
                         int64_t col0, int64_t col_end, const float* Z, const float* R,
                         const uint8_t* mask, int64_t mask_j0, int64_t mask_w, hipStream_t s,
                         const float* gn, int64_t hist_j0, unsigned int* hist) {
  if (col_end <= col0 || K <= 0) return hipSuccess;
  if (hist && !gn) return hipErrorInvalidValue;
  const int nct = (int)cdiv(col_end - col0, 128);
  const int nrt = (int)cdiv(c, 128);
  if (!update_large_tiles(c, col0, col_end)) {
    const int nct64 = (int)cdiv(col_end - col0, 64);
    const int nrt64 = (int)cdiv(c, 64);
    if (hist)
      hipLaunchKernelGGL(update64_kernel<true>, dim3((unsigned)(nct64 * nrt64)), dim3(256), 0, s, W,
                         c, b, r0, (int)K, ldz, col0, col_end, nct64, Z, R, mask, mask_j0,
                         mask_j0 + mask_w, gn, hist_j0, hist);
    else
      hipLaunchKernelGGL(update64_kernel<false>, dim3((unsigned)(nct64 * nrt64)), dim3(256), 0, s, W,
                         c, b, r0, (int)K, ldz, col0, col_end, nct64, Z, R, mask, mask_j0,
                         mask_j0 + mask_w, gn, hist_j0, hist);
    return hipGetLastError();
  }
  const int64_t ntiles = (int64_t)nct * nrt;
  if (hist) {
    // two workgroups per compute unit fit (LDS), 256 compute units
    const int64_t grid = ntiles < 512 ? ntiles : 512;
    hipLaunchKernelGGL(update_kernel<true>, dim3((unsigned)grid), dim3(256), 0, s, W, c, b, r0,
                       (int)K, ldz, col0, col_end, nct, ntiles, Z, R, mask, mask_j0,
                       mask_j0 + mask_w, gn, hist_j0, hist);
  } else {
    hipLaunchKernelGGL(update_kernel<false>, dim3((unsigned)ntiles), dim3(256), 0, s, W, c, b, r0,
                       (int)K, ldz, col0, col_end, nct, ntiles, Z, R, mask, mask_j0,
                       mask_j0 + mask_w, gn, hist_j0, hist);
  }
  return hipGetLastError();
}

hipError_t launch_to_f32(const void* src, th_dtype dt, int64_t count, float* dst, DevState* st,
                         hipStream_t s) {
  hipLaunchKernelGGL(to_f32_kernel, dim3(ew_grid(count)), dim3(256), 0, s, src, (int)dt, count,
                     dst, st);
  return hipGetLastError();
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  if ((uintptr_t)p & 15) return hipErrorInvalidValue;  // callers pass 256-byte aligned buffers
  const int64_t n16 = (int64_t)(bytes / 16);
  const int ntail = (int)(bytes % 16);
  hipLaunchKernelGGL(zero_kernel, dim3(ew_grid(n16 > 0 ? n16 : 1)), dim3(256), 0, s, (uint4*)p, n16,
                     (unsigned char*)p + n16 * 16, ntail);
  return hipGetLastError();
}

hipError_t launch_from_f32(const float* src, int64_t count, th_dtype dt, void* dst,
                           hipStream_t s) {
  hipLaunchKernelGGL(from_f32_kernel, dim3(ew_grid(count)), dim3(256), 0, s, src, count, (int)dt,
                     dst);
  return hipGetLastError();
}

hipError_t launch_diff_f32(const void* W, const void* What, th_dtype dt, int64_t count, float* D,
                           hipStream_t s) {
  hipLaunchKernelGGL(diff_kernel, dim3(ew_grid(count)), dim3(256), 0, s, W, What, (int)dt, count,
                     D);
  return hipGetLastError();
}

hipError_t launch_quadform(const float* D, int64_t c, int64_t b, const float* G, double* partials,
                           int64_t* nparts, hipStream_t s) {
  const int nct = (int)cdiv(b, 128);
  const int nrt = (int)cdiv(c, 128);
  *nparts = (int64_t)nct * nrt;
  hipLaunchKernelGGL(quadform_kernel, dim3((unsigned)(nct * nrt)), dim3(256), 0, s, D, c, b, nct,
                     G, partials);
  return hipGetLastError();
}

hipError_t launch_sum_partials(const double* partials, int64_t n, double* out, hipStream_t s) {
  hipLaunchKernelGGL(sum_kernel, dim3(1), dim3(256), 0, s, partials, n, out);
  return hipGetLastError();
}

}  // namespace th
