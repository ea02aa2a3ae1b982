// Global residual-budget selection for unstructured sparsity.
//
// "Pruning LLMs with Thanos", section "Contribution two: keep the budget global
// and the execution local": for each block, r = (weights still to remove), the
// scores of the whole active region F are recomputed from the current weights,
// the r lowest form a provisional candidate set, and only its intersection with
// the current block is pruned.
//
// The r-th smallest key is found exactly by an MSD radix select over 64-bit keys
// (fp32 score bits << 32 | flat index k*b + q). Keys are unique, so the
// candidate set is exactly { key < tbound } and ties in the score go to the
// lower flat index. Each pass histograms one 11-bit digit (LDS histogram per
// workgroup, integer atomics into the global one, so counts are exact and
// order-independent); a one-workgroup pick kernel narrows the prefix (a kernel
// boundary orders the counts of all XCDs for it far more cheaply than a device-
// scope fence in every workgroup would). Budget, prefix and threshold stay on
// the device: the host launches a fixed number of passes and finished passes
// exit at once.
//
// Candidate list: the first pass whose prefix is not empty (the second digit)
// still reads every key, and also stores the keys that match its prefix -- the
// bucket of the first digit, a few percent of the region -- in a segment of its
// workgroup (an LDS counter gives each key its slot; no global atomics). The later
// passes of the block read only those segments: every key they count matches a
// longer prefix, so it is in the list. A segment that would overflow makes the
// list unusable and the later passes read W again, as without a list.
#include "common.h"

namespace th {

namespace {

// Digits: shifts 53, 42, 31, 20, 9 (11 bits each) then 0 (9 bits).
__device__ __forceinline__ void digit_of(int shift, int& width) {
  width = (shift == 0) ? 9 : 11;
}

__global__ void select_init_kernel(DevState* st, long long add_budget, long long ncand) {
  for (int i = threadIdx.x; i < kSelCopies * kSelBins; i += blockDim.x) (&st->hist[0][0])[i] = 0u;
  if (threadIdx.x == 0) {
    const long long budget = st->budget + add_budget;
    st->budget = budget;
    const long long r = budget - st->pruned;
    st->rrem = r;
    st->prefix = 0ull;
    st->shift = 53;
    st->cand_state = 0;
    st->cand_over = 0;
    if (r <= 0) {
      st->done = 1;
      st->tbound = 0ull;
    } else if (r >= ncand) {
      st->done = 1;
      st->tbound = ~0ull;
    } else {
      st->done = 0;
      st->tbound = 0ull;
    }
  }
}

// Narrow the prefix by the digit whose bucket holds the rrem-th smallest key
// (one workgroup of 256 threads, 8 bins each), then clear the histogram for the
// next pass. An inclusive scan of the per-thread sums (within each wave by lane
// shuffles, then over the four wave totals) finds the one thread whose bins hold
// rank rrem (exclusive sum < rrem <= inclusive sum); that thread walks its 8
// bins. Integer counts throughout, so the result does not depend on order.
__global__ __launch_bounds__(256) void select_pick_kernel(DevState* st) {
  if (st->done) return;
  // the pass just counted was the one that builds the candidate list
  const bool built = st->cand_state == 0 && st->shift < 53;
  __shared__ unsigned long long wsum[4];
  __shared__ int found;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int per = kSelBins / 256;  // 8 bins per thread
  static_assert(per == 8, "two 16-byte loads per copy");
  // this thread's 8 bins summed over the copies: two 16-byte loads per copy, all
  // in flight at once
  u32x4_t a[kSelCopies], c[kSelCopies];
#pragma unroll
  for (int cp = 0; cp < kSelCopies; ++cp) {
    const u32x4_t* src = (const u32x4_t*)&st->hist[cp][tid * per];
    a[cp] = src[0];
    c[cp] = src[1];
  }
  unsigned int h[per];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = 0u;
    h[4 + e] = 0u;
#pragma unroll
    for (int cp = 0; cp < kSelCopies; ++cp) {
      h[e] += a[cp][e];
      h[4 + e] += c[cp][e];
    }
  }
  unsigned long long local = 0;
#pragma unroll
  for (int e = 0; e < per; ++e) local += h[e];
  // inclusive scan inside the wave
  unsigned long long incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned long long v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wsum[wave] = incl;
  if (tid == 0) found = 0;
  __syncthreads();
  for (int w = 0; w < wave; ++w) incl += wsum[w];
  const long long r = st->rrem;
  const long long excl = (long long)incl - (long long)local;
  if (excl < r && r <= (long long)incl) {
    long long cum = excl;
    int d = tid * per + per - 1;
    long long inb = h[per - 1];
#pragma unroll
    for (int e = per - 1; e >= 0; --e) {  // the first bin (from the left) that reaches r
      long long before = excl;
#pragma unroll
      for (int t = 0; t < e; ++t) before += h[t];
      if (before < r && before + (long long)h[e] >= r) {
        d = tid * per + e;
        cum = before;
        inb = h[e];
      }
    }
    const int shift = st->shift;
    const long long rnew = r - cum;
    st->prefix |= ((unsigned long long)d) << shift;
    st->rrem = rnew;
    if (inb == rnew || shift == 0) {
      // every key of the bucket is within the r smallest (shift == 0: inb == 1)
      st->tbound = st->prefix + (1ull << shift);
      st->done = 1;
    } else {
      st->shift = (shift >= 20) ? shift - 11 : 0;
    }
    found = 1;
  }
  if (tid == 0 && built) st->cand_state = st->cand_over ? 2 : 1;
  __syncthreads();
  if (tid == 0 && !found) {  // cannot happen when the histogram is consistent
    st->tbound = st->prefix;
    st->done = 1;
  }
  const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int cp = 0; cp < kSelCopies; ++cp) {
    u32x4_t* dst = (u32x4_t*)&st->hist[cp][tid * per];
    dst[0] = z;
    dst[1] = z;
  }
}

// Histogram of the current digit over the keys of rows k = blockIdx.x + m gridDim.x,
// columns 0..f-1 (keyf(k, q)).
template <class KeyF>
__device__ __forceinline__ void pass_body(DevState* st, int64_t rows, int64_t f, KeyF&& keyf) {
  __shared__ unsigned int sh[kSelBins];
  const int shift = st->shift;
  int width;
  digit_of(shift, width);
  const int top = shift + width;
  const unsigned long long prefix = st->prefix;
  for (int i = threadIdx.x; i < kSelBins; i += blockDim.x) sh[i] = 0u;
  __syncthreads();
  const unsigned long long dmask = (1ull << width) - 1ull;
  for (int64_t k = blockIdx.x; k < rows; k += gridDim.x) {
    for (int64_t q = threadIdx.x; q < f; q += blockDim.x) {
      const unsigned long long key = keyf(k, q);
      const bool match = (top >= 64) || ((key >> top) == (prefix >> top));
      if (match) atomicAdd(&sh[(key >> shift) & dmask], 1u);
    }
  }
  __syncthreads();
  unsigned int* gh = st->hist[blockIdx.x % kSelCopies];
  for (int i = threadIdx.x; i < kSelBins; i += blockDim.x)
    if (sh[i]) atomicAdd(&gh[i], sh[i]);
}

// Keys recomputed from the current weights: S = W^2 * g with g the per-column
// score weight (1/[A_F]_qq for OBS, G_qq for Wanda). The pass streams W[:, j0:j1)
// once, so it is bound by the loads: with 16-byte aligned rows each thread reads
// four columns of W and g per 16-byte load, four loads in flight (the histogram
// atomics are not the limit: without them a pass is only ~7% faster).
__global__ __launch_bounds__(256) void select_pass_kernel(const float* __restrict__ W, int64_t c,
                                                          int64_t b, int64_t j0, int64_t j1,
                                                          const float* __restrict__ g,
                                                          DevState* st,
                                                          unsigned long long* __restrict__ cand,
                                                          unsigned int* __restrict__ cand_n,
                                                          int64_t quota) {
  if (st->done) return;
  __shared__ unsigned int sh[kSelBins];
  __shared__ unsigned int slot;
  const int shift = st->shift;
  int width;
  digit_of(shift, width);
  const int top = shift + width;
  const unsigned long long prefix = st->prefix;
  const int cstate = st->cand_state;
  for (int i = threadIdx.x; i < kSelBins; i += blockDim.x) sh[i] = 0u;
  if (threadIdx.x == 0) slot = 0u;
  __syncthreads();
  const unsigned long long dmask = (1ull << width) - 1ull;
  auto flush = [&]() {
    __syncthreads();
    unsigned int* gh = st->hist[blockIdx.x % kSelCopies];
    for (int i = threadIdx.x; i < kSelBins; i += blockDim.x)
      if (sh[i]) atomicAdd(&gh[i], sh[i]);
  };
  if (cstate == 1) {  // the keys of the list (gridDim.x segments: this pass's grid)
    const unsigned long long* seg = cand + (int64_t)blockIdx.x * quota;
    const unsigned int n = cand_n[blockIdx.x];
    for (unsigned int i = threadIdx.x; i < n; i += blockDim.x) {
      const unsigned long long key = seg[i];
      if ((key >> top) == (prefix >> top)) atomicAdd(&sh[(key >> shift) & dmask], 1u);
    }
    flush();
    return;
  }
  const bool build = cstate == 0 && shift < 53 && cand != nullptr;
  if (cstate == 0 && shift < 53 && cand == nullptr && blockIdx.x == 0 && threadIdx.x == 0)
    st->cand_over = 1;  // no list buffer: the later passes read W
  unsigned long long* seg = build ? cand + (int64_t)blockIdx.x * quota : nullptr;
  auto count = [&](float w, float gq, int64_t flat) {
    const unsigned long long key = make_key(score_of(w, gq), (unsigned int)flat);
    const bool match = (top >= 64) || ((key >> top) == (prefix >> top));
    if (match) {
      atomicAdd(&sh[(key >> shift) & dmask], 1u);
      if (build) {
        const unsigned int at = atomicAdd(&slot, 1u);
        if (at < (unsigned long long)quota) seg[at] = key;
      }
    }
  };
  const int64_t f = j1 - j0;
  const bool vec = ((b & 3) == 0) && ((j0 & 3) == 0) && ((((uintptr_t)W | (uintptr_t)g) & 15) == 0);
  const int64_t f4 = vec ? (f >> 2) : 0;
  for (int64_t k = blockIdx.x; k < c; k += gridDim.x) {
    const float* wr = W + k * b + j0;
    const float* gr = g + j0;
    const int64_t base = k * b + j0;
#pragma unroll 4
    for (int64_t v = threadIdx.x; v < f4; v += blockDim.x) {
      const f32x4_t w4 = ((const f32x4_t*)wr)[v];
      const f32x4_t g4 = ((const f32x4_t*)gr)[v];
      const int64_t q = 4 * v;
      count(w4[0], g4[0], base + q);
      count(w4[1], g4[1], base + q + 1);
      count(w4[2], g4[2], base + q + 2);
      count(w4[3], g4[3], base + q + 3);
    }
    for (int64_t q = 4 * f4 + threadIdx.x; q < f; q += blockDim.x) count(wr[q], gr[q], base + q);
  }
  flush();
  if (build && threadIdx.x == 0) {
    const unsigned int n = slot;
    cand_n[blockIdx.x] = n < (unsigned long long)quota ? n : (unsigned int)quota;
    if (n > (unsigned long long)quota) st->cand_over = 1;
  }
}

// Keys from given scores [c, f] (parity entry point).
__global__ __launch_bounds__(256) void select_scores_pass_kernel(const float* __restrict__ S,
                                                                 int64_t c, int64_t f,
                                                                 int64_t b_full, int64_t j0,
                                                                 DevState* st) {
  if (st->done) return;
  pass_body(st, c, f, [&](int64_t k, int64_t q) {
    return make_key(S[k * f + q], (unsigned int)(k * b_full + j0 + q));
  });
}

}  // namespace

hipError_t launch_select_init(DevState* st, long long add_budget, long long ncand,
                              hipStream_t s) {
  hipLaunchKernelGGL(select_init_kernel, dim3(1), dim3(256), 0, s, st, add_budget, ncand);
  return hipGetLastError();
}

static unsigned pass_grid(int64_t rows) {
  int64_t g = rows < 1024 ? rows : 1024;
  return (unsigned)(g < 1 ? 1 : g);
}

int64_t select_segments(int64_t c) { return pass_grid(c); }

// One eighth of a segment's keys (a workgroup's rows times the layer's columns):
// the first digit's bucket at the threshold holds a few percent of them.
int64_t select_quota(int64_t c, int64_t b) {
  const int64_t rows = cdiv(c, (int64_t)pass_grid(c));
  const int64_t q = cdiv(rows * b, (int64_t)8);
  return q < 64 ? 64 : q;
}

hipError_t launch_select_pass(const float* W, int64_t c, int64_t b, int64_t j0, int64_t j1,
                              const float* g, DevState* st, hipStream_t s,
                              unsigned long long* cand, unsigned int* cand_n, int64_t quota) {
  if (cand && (!cand_n || quota <= 0)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(select_pass_kernel, dim3(pass_grid(c)), dim3(256), 0, s, W, c, b, j0, j1, g,
                     st, cand, cand_n, quota);
  return hipGetLastError();
}

hipError_t launch_select_scores_pass(const float* scores, int64_t c, int64_t f, int64_t b_full,
                                     int64_t j0, DevState* st, hipStream_t s) {
  hipLaunchKernelGGL(select_scores_pass_kernel, dim3(pass_grid(c)), dim3(256), 0, s, scores, c, f,
                     b_full, j0, st);
  return hipGetLastError();
}

hipError_t launch_select_pick(DevState* st, hipStream_t s) {
  hipLaunchKernelGGL(select_pick_kernel, dim3(1), dim3(256), 0, s, st);
  return hipGetLastError();
}

}  // namespace th
