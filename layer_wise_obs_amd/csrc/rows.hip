// Rows kept dense (the alpha variant) and the gather / scatter around the layer
// step on the other rows.
//
// "Pruning LLMs with Thanos", section "What the experiments show": the alpha
// variant keeps a fraction alpha of the rows as outliers. Read here as the
// round-half-even(alpha c) rows of largest output energy s_k = sum_q W_kq^2 G_qq
// (fp64 sums, ranked by their fp32 value, ties to the higher row index); the
// other rows form a layer of their own (rows are independent given H, "The
// layer-reconstruction lens"), which the unchanged layer step prunes.
//
// The c - r rows that are pruned are found as the c - r smallest keys
// (fp32 energy bits << 32 | row) by the radix select of the global budget; a
// one-workgroup scan then numbers them, and the gather / scatter kernels move
// rows between the caller's layout and the compact one.
#include "common.h"

namespace th {

namespace {

constexpr int kRowWaves = 4;

// s_k = fp32(sum_q W_kq^2 g_q), fp64 sums; one wave per row.
__global__ __launch_bounds__(kRowWaves * 64) void row_energy_kernel(const void* __restrict__ W,
                                                                    int wdt, int64_t c, int64_t b,
                                                                    const float* __restrict__ g,
                                                                    float* __restrict__ s) {
  const int lane = threadIdx.x & 63;
  const int64_t k = (int64_t)blockIdx.x * kRowWaves + (threadIdx.x >> 6);
  if (k >= c) return;
  double acc = 0.0;
  for (int64_t q = lane; q < b; q += 64) {
    const float w = wdt == TH_BF16 ? bf16_to_f32(((const unsigned short*)W)[k * b + q])
                                   : ((const float*)W)[k * b + q];
    acc += (double)w * (double)w * (double)g[q];
  }
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (lane == 0) s[k] = (float)acc;
}

// idx[k] = position of row k among the pruned rows (key < tbound of the selection
// state), -1 if dense; rowmap[j] = k for the j-th pruned row; a non-finite energy
// raises the layer state's flag. One workgroup of 1024 threads, each owning a
// contiguous run of rows.
__global__ __launch_bounds__(1024) void row_index_kernel(const float* __restrict__ s, int64_t c,
                                                         const DevState* __restrict__ st,
                                                         int32_t* __restrict__ idx,
                                                         int32_t* __restrict__ rowmap,
                                                         uint8_t* __restrict__ dense_out,
                                                         DevState* layer) {
  __shared__ int part[1024];
  const int t = threadIdx.x;
  const unsigned long long tb = st->tbound;
  const int64_t per = cdiv(c, 1024);
  const int64_t r0 = t * per, r1 = (r0 + per < c) ? r0 + per : c;
  int cnt = 0;
  for (int64_t k = r0; k < r1; ++k) cnt += make_key(s[k], (unsigned int)k) < tb;
  part[t] = cnt;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive scan
    const int v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int pos = part[t] - cnt;
  for (int64_t k = r0; k < r1; ++k) {
    if (!isfinite(s[k])) layer->nonfinite = 1;
    const bool pruned = make_key(s[k], (unsigned int)k) < tb;
    idx[k] = pruned ? pos : -1;
    if (pruned) rowmap[pos++] = (int32_t)k;
    if (dense_out) dense_out[k] = pruned ? 0 : 1;
  }
}

// Wf[j, :] = fp32(W[rowmap[j], :]); non-finite values raise the state flag.
__global__ void gather_rows_kernel(const void* __restrict__ W, int wdt, int64_t b,
                                   const int32_t* __restrict__ rowmap, int64_t cp,
                                   float* __restrict__ Wf, DevState* st) {
  const int64_t n = cp * b;
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < n;
       x += (int64_t)gridDim.x * blockDim.x) {
    const int64_t j = x / b, q = x - j * b;
    const int64_t src = (int64_t)rowmap[j] * b + q;
    const float v = wdt == TH_BF16 ? bf16_to_f32(((const unsigned short*)W)[src])
                                   : ((const float*)W)[src];
    if (!isfinite(v)) st->nonfinite = 1;
    Wf[x] = v;
  }
}

// Back to the caller's layout: pruned rows from the compact result (W in its
// dtype, optional fp32 copy and mask), dense rows unchanged with a zero mask.
__global__ void scatter_rows_kernel(void* __restrict__ W, int wdt, int64_t c, int64_t b,
                                    const int32_t* __restrict__ idx, const float* __restrict__ Wf,
                                    const uint8_t* __restrict__ mc, float* __restrict__ Wout,
                                    uint8_t* __restrict__ mask) {
  const int64_t n = c * b;
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < n;
       x += (int64_t)gridDim.x * blockDim.x) {
    const int64_t k = x / b, q = x - k * b;
    const int32_t j = idx[k];
    if (j < 0) {
      if (Wout) Wout[x] = wdt == TH_BF16 ? bf16_to_f32(((const unsigned short*)W)[x])
                                         : ((const float*)W)[x];
      if (mask) mask[x] = 0;
    } else {
      const int64_t y = (int64_t)j * b + q;
      const float v = Wf[y];
      if (wdt == TH_BF16) ((unsigned short*)W)[x] = f32_to_bf16_rne(v);
      else ((float*)W)[x] = v;
      if (Wout) Wout[x] = v;
      if (mask) mask[x] = mc[y];
    }
  }
}

unsigned ew_blocks(int64_t n) {
  int64_t g = cdiv(n, 256);
  if (g > 8192) g = 8192;
  return (unsigned)(g < 1 ? 1 : g);
}

}  // namespace

hipError_t launch_row_energy(const void* W, th_dtype wdt, int64_t c, int64_t b, const float* g,
                             float* s, hipStream_t st) {
  hipLaunchKernelGGL(row_energy_kernel, dim3((unsigned)cdiv(c, kRowWaves)), dim3(kRowWaves * 64), 0,
                     st, W, (int)wdt, c, b, g, s);
  return hipGetLastError();
}

hipError_t launch_row_index(const float* s, int64_t c, const DevState* sel, int32_t* idx,
                            int32_t* rowmap, uint8_t* dense_out, DevState* layer,
                            hipStream_t st) {
  hipLaunchKernelGGL(row_index_kernel, dim3(1), dim3(1024), 0, st, s, c, sel, idx, rowmap,
                     dense_out, layer);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* W, th_dtype wdt, int64_t b, const int32_t* rowmap,
                              int64_t cp, float* Wf, DevState* dst, hipStream_t st) {
  hipLaunchKernelGGL(gather_rows_kernel, dim3(ew_blocks(cp * b)), dim3(256), 0, st, W, (int)wdt, b,
                     rowmap, cp, Wf, dst);
  return hipGetLastError();
}

hipError_t launch_scatter_rows(void* W, th_dtype wdt, int64_t c, int64_t b, const int32_t* idx,
                               const float* Wf, const uint8_t* mc, float* Wout, uint8_t* mask,
                               hipStream_t st) {
  hipLaunchKernelGGL(scatter_rows_kernel, dim3(ew_blocks(c * b)), dim3(256), 0, st, W, (int)wdt, c,
                     b, idx, Wf, mc, Wout, mask);
  return hipGetLastError();
}

}  // namespace th
