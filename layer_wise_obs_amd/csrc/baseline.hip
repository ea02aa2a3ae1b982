// Comparators the joint-compensation method is measured against: magnitude and
// Wanda pruning, which zero the lowest-scoring weights and leave every other
// weight unchanged.
//
// "Weight Pruning in Large Language Models ..." (explainer), section "Wanda:
// Pruning by Weights and Activations": score |W_kq| * ||X_q||_2, thresholds per
// output row (each row loses its lowest fraction), no update of the remaining
// weights; section "The Failure of Magnitude Pruning in Large Transformers": rank
// by |W_kq| and remove the smallest; section "N:M Semi-Structured Sparsity (2:4
// Pattern)": the group constraint is enforced within every group of m. "Pruning
// LLMs with Thanos", section "Why magnitude alone misses important weights": the
// squared Wanda score W_kq^2 G_qq (G = X X^T) has the same order.
//
// Keys: score_of(w, g) (w^2, then times g, each rounded in fp32) with g = G_qq
// (Wanda) or 1 (magnitude, the order of |w|), ties broken by the lower column.
#include "common.h"

namespace th {

namespace {

constexpr int kColsqThreads = 256;

__device__ __forceinline__ float load_elem(const void* p, int dt, int64_t i) {
  return dt == TH_BF16 ? bf16_to_f32(((const unsigned short*)p)[i]) : ((const float*)p)[i];
}

// part[y][q] = sum over tokens of split y of X_tq^2 (fp64), token-major X.
__global__ __launch_bounds__(kColsqThreads) void colsq_partial_kernel(const void* __restrict__ X,
                                                                     int xdt, int64_t n, int64_t b,
                                                                     int64_t ldx, int64_t tok_per,
                                                                     double* __restrict__ part) {
  const int64_t q = (int64_t)blockIdx.x * kColsqThreads + threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.y * tok_per;
  const int64_t t1 = (t0 + tok_per < n) ? t0 + tok_per : n;
  if (q >= b) return;
  double s = 0.0;
  for (int64_t t = t0; t < t1; ++t) {
    const double v = (double)load_elem(X, xdt, t * ldx + q);
    s += v * v;
  }
  part[(int64_t)blockIdx.y * b + q] = s;
}

// g[q] = fp32(sum_y part[y][q]), summed in split order.
__global__ void colsq_finish_kernel(const double* __restrict__ part, int splits, int64_t b,
                                    float* __restrict__ g) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= b) return;
  double s = 0.0;
  for (int y = 0; y < splits; ++y) s += part[(int64_t)y * b + q];
  g[q] = (float)s;
}

// One workgroup per row: prune the krow smallest (key, column) of the row.
// The key threshold T is found by a radix select over the 32-bit score (four
// 8-bit digits, LDS histograms); entries below T are pruned, and of the entries
// equal to T the lowest columns until krow are reached.
__global__ __launch_bounds__(256) void baseline_row_kernel(void* __restrict__ W, int wdt, int64_t b,
                                                           const float* __restrict__ g,
                                                           int64_t krow,
                                                           uint8_t* __restrict__ mask) {
  __shared__ unsigned hist[256];
  __shared__ unsigned sh_prefix, sh_remaining;
  __shared__ unsigned wcount[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const int64_t off = row * b;
  auto key = [&](int64_t q) -> unsigned {
    const float w = load_elem(W, wdt, off + q);
    return __float_as_uint(score_of(w, g ? g[q] : 1.f));
  };
  unsigned T = 0xffffffffu, need = 0;
  bool all = krow >= b, none = krow <= 0;
  if (!all && !none) {
    unsigned prefix = 0, remaining = (unsigned)krow;  // rank (1-based) still to place
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      const unsigned hmask = pass == 0 ? 0u : (0xffffffffu << (shift + 8));
      hist[tid] = 0;
      __syncthreads();
      for (int64_t q = tid; q < b; q += 256) {
        const unsigned s = key(q);
        if ((s & hmask) == (prefix & hmask)) atomicAdd(&hist[(s >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        unsigned cum = 0;
        int d = 0;
        for (; d < 255; ++d) {
          if (cum + hist[d] >= remaining) break;
          cum += hist[d];
        }
        sh_prefix = prefix | ((unsigned)d << shift);
        sh_remaining = remaining - cum;
      }
      __syncthreads();
      prefix = sh_prefix;
      remaining = sh_remaining;
      __syncthreads();
    }
    T = prefix;       // the krow-th smallest score
    need = remaining; // how many entries equal to T are pruned (lowest columns first)
  }
  unsigned carry = 0;
  for (int64_t base = 0; base < b; base += 256) {
    const int64_t q = base + tid;
    const bool valid = q < b;
    const unsigned s = valid ? key(q) : 0xffffffffu;
    const bool eq = valid && !all && !none && s == T;
    const unsigned long long bal = __ballot(eq);
    if (lane == 0) wcount[wave] = (unsigned)__popcll(bal);
    __syncthreads();
    unsigned before = carry;
    for (int w = 0; w < wave; ++w) before += wcount[w];
    const unsigned long long lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    const unsigned rank = before + (unsigned)__popcll(bal & lt);
    const bool prune = valid && (all || (!none && (s < T || (eq && rank < need))));
    if (valid) {
      if (prune) {
        if (wdt == TH_BF16) ((unsigned short*)W)[off + q] = 0;
        else ((float*)W)[off + q] = 0.f;
      }
      if (mask) mask[off + q] = prune ? 1 : 0;
    }
    carry += wcount[0] + wcount[1] + wcount[2] + wcount[3];
    __syncthreads();
  }
}

// One thread per (row, aligned group of m): prune the m-n smallest (key, column).
__global__ void baseline_nm_kernel(void* __restrict__ W, int wdt, int64_t c, int64_t b,
                                   const float* __restrict__ g, int n, int m,
                                   uint8_t* __restrict__ mask) {
  const int64_t ngroups = b / m;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= c * ngroups) return;
  const int64_t row = idx / ngroups, q0 = (idx - row * ngroups) * m;
  const int64_t off = row * b + q0;
  auto key = [&](int t) -> unsigned {
    return __float_as_uint(score_of(load_elem(W, wdt, off + t), g ? g[q0 + t] : 1.f));
  };
  // ranks first (the group is rewritten only after every key of it is read)
  unsigned pm[4] = {0u, 0u, 0u, 0u};  // prune bits for up to 128 members
  for (int t = 0; t < m; ++t) {
    const unsigned kt = key(t);
    int rank = 0;
    for (int u = 0; u < m; ++u) {
      const unsigned ku = key(u);
      rank += (ku < kt) || (ku == kt && u < t);
    }
    if (rank < m - n) pm[t >> 5] |= 1u << (t & 31);
  }
  for (int t = 0; t < m; ++t) {
    const bool prune = (pm[t >> 5] >> (t & 31)) & 1u;
    if (prune) {
      if (wdt == TH_BF16) ((unsigned short*)W)[off + t] = 0;
      else ((float*)W)[off + t] = 0.f;
    }
    if (mask) mask[off + t] = prune ? 1 : 0;
  }
}

}  // namespace

int colsq_splits(int64_t n) {
  int64_t s = cdiv(n, 2048);
  if (s > 128) s = 128;
  if (s < 1) s = 1;
  return (int)s;
}

hipError_t launch_column_sq_norms(const void* X, th_dtype xdt, int64_t n, int64_t b, int64_t ldx,
                                  double* part, float* g, hipStream_t s) {
  const int splits = colsq_splits(n);
  const int64_t tok_per = cdiv(n, splits);
  hipLaunchKernelGGL(colsq_partial_kernel, dim3((unsigned)cdiv(b, kColsqThreads), splits),
                     dim3(kColsqThreads), 0, s, X, (int)xdt, n, b, ldx, tok_per, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(colsq_finish_kernel, dim3((unsigned)cdiv(b, 256)), dim3(256), 0, s, part,
                     splits, b, g);
  return hipGetLastError();
}

hipError_t launch_baseline_rows(void* W, th_dtype wdt, int64_t c, int64_t b, const float* g,
                                int64_t krow, uint8_t* mask, hipStream_t s) {
  hipLaunchKernelGGL(baseline_row_kernel, dim3((unsigned)c), dim3(256), 0, s, W, (int)wdt, b, g,
                     krow, mask);
  return hipGetLastError();
}

hipError_t launch_baseline_nm(void* W, th_dtype wdt, int64_t c, int64_t b, const float* g, int n,
                              int m, uint8_t* mask, hipStream_t s) {
  const int64_t total = c * (b / m);
  hipLaunchKernelGGL(baseline_nm_kernel, dim3((unsigned)cdiv(total, 256)), dim3(256), 0, s, W,
                     (int)wdt, c, b, g, n, m, mask);
  return hipGetLastError();
}

}  // namespace th
