// Column-sequential comparator: the synchronized column schedule of SparseGPT.
//
// "Pruning LLMs with Thanos", section "The scaling problem, and what SparseGPT
// changes": columns are handled left to right for every row at once, a finished
// column is frozen, compensation flows only into active columns, and the pruning
// decisions are refreshed block by block. The explainer's section "SparseGPT:
// Second-Order Reconstruction at Scale": pruning w_kq subtracts
// (w_kq / [H^-1]_qq) * [H^-1]_{q, q+1:} from the rest of row k, with H^-1 the
// inverse over the columns still active. With H^-1 = U^T U (U upper), the inverse
// over columns q.. is U_{q:,q:}^T U_{q:,q:}, so its row q is U_qq * U_{q, q:} and the
// update is e_kq * U_{q, q:} with e_kq = w_kq / U_qq.
//
// Per block J the error row e_k (zero for kept weights) is a short recurrence over
// the block's pruned columns in order (each pruned column sees the updates of the
// ones before it). One wave owns a row at a time with the block's 128 weights in
// two registers per lane and U_JJ in LDS; kept weights are not written back here.
// Because U is upper triangular, one GEMM W[:, J..] -= E U[J, J..] then gives the
// kept weights of the block exactly the compensation the recurrence applied, and
// the columns after the block the whole block's compensation (the update kernel,
// which also writes the exact zeros).
//
// Scores: the OBS cost of deleting w_kq when column q is processed,
// w_kq^2 / [inv(H_{q:})]_qq = w_kq^2 / U_qq^2, from the weights at the start of
// the block. Unstructured: the block's round-half-even(p * c * |J|) lowest keys
// (score, flat index) by the radix select, an equal quota per block; N:M: the m-n
// lowest (score, column) of every aligned group.
#include "common.h"

namespace th {

namespace {

constexpr int kWaves = 8;

// g[q] = 1 / U_qq^2, the score weight of column q.
__global__ void sgpt_gdiag_kernel(const float* __restrict__ U, int64_t b, float* __restrict__ g) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= b) return;
  const float u = U[q * b + q];
  g[q] = __fdiv_rn(1.0f, __fmul_rn(u, u));
}

struct SgptArgs {
  const float* W;   // working weights, c x b (block-start values)
  int64_t c, b, j0;
  int Bb;           // block width
  int n, m;         // N:M (mode 0)
  const float* U;   // b x b, upper, zero below the diagonal
  const float* g;   // 1 / U_qq^2
  float* E;         // c rows, pitch lde: this block's errors
  int64_t lde;
  uint8_t* mask;    // c x b
  DevState* st;
  unsigned long long* blk_count;
};

template <int MODE>  // 0: N:M groups, 1: keys below the block's threshold
__global__ __launch_bounds__(kWaves * 64, 2) void sgpt_errors_kernel(SgptArgs a) {
  __shared__ float sU[kMaxBlock * kMaxBlock];  // U_JJ, zero below the diagonal and past Bb
  __shared__ float sg[kMaxBlock];
  __shared__ float sbuf[kWaves][kMaxBlock];
  __shared__ unsigned long long scount[kWaves];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Bb = a.Bb;
  const int64_t b = a.b, j0 = a.j0;
  for (int idx = tid; idx < kMaxBlock * kMaxBlock; idx += kWaves * 64) {
    const int r = idx >> 7, q = idx & (kMaxBlock - 1);
    sU[idx] = (r < Bb && q < Bb && q >= r) ? a.U[(j0 + r) * b + j0 + q] : 0.f;
  }
  for (int q = tid; q < kMaxBlock; q += kWaves * 64) sg[q] = q < Bb ? a.g[j0 + q] : 0.f;
  __syncthreads();
  const unsigned long long tbound = (MODE == 1) ? a.st->tbound : 0ull;
  unsigned long long count = 0;

  for (int64_t k = (int64_t)blockIdx.x * kWaves + wave; k < a.c; k += (int64_t)gridDim.x * kWaves) {
    const int e0 = lane, e1 = lane + 64;
    const bool v0 = e0 < Bb, v1 = e1 < Bb;
    const float* wrow = a.W + k * b + j0;
    float w0 = v0 ? wrow[e0] : 0.f;
    float w1 = v1 ? wrow[e1] : 0.f;
    bool s0, s1;
    if (MODE == 0) {
      if (v0) sbuf[wave][e0] = score_of(w0, sg[e0]);
      if (v1) sbuf[wave][e1] = score_of(w1, sg[e1]);
      wave_sync();
      s0 = v0 && nm_pruned(sbuf[wave], e0, a.n, a.m);
      s1 = v1 && nm_pruned(sbuf[wave], e1, a.n, a.m);
    } else {
      s0 = v0 && make_key(score_of(w0, sg[e0]), (unsigned int)(k * b + j0 + e0)) < tbound;
      s1 = v1 && make_key(score_of(w1, sg[e1]), (unsigned int)(k * b + j0 + e1)) < tbound;
    }
    const unsigned long long m0 = __ballot(s0), m1 = __ballot(s1);
    // the recurrence over the pruned columns, in column order (wave-uniform loops)
    float err0 = 0.f, err1 = 0.f;
    for (unsigned long long mm = m0; mm; mm &= mm - 1) {
      const int q = __builtin_ctzll(mm);
      const float e = bcast(w0, q) / sU[q * kMaxBlock + q];
      err0 = (lane == q) ? e : err0;
      w0 = fmaf(-e, sU[q * kMaxBlock + lane], w0);
      w1 = fmaf(-e, sU[q * kMaxBlock + 64 + lane], w1);
    }
    for (unsigned long long mm = m1; mm; mm &= mm - 1) {
      const int q = __builtin_ctzll(mm);  // column 64 + q; columns below 64 are not touched
      const float e = bcast(w1, q) / sU[(64 + q) * kMaxBlock + 64 + q];
      err1 = (lane == q) ? e : err1;
      w1 = fmaf(-e, sU[(64 + q) * kMaxBlock + 64 + lane], w1);
    }
    float* erow = a.E + k * a.lde;
    if (v0) erow[e0] = err0;
    if (v1) erow[e1] = err1;
    uint8_t* mrow = a.mask + k * b + j0;
    if (v0) mrow[e0] = s0 ? 1 : 0;
    if (v1) mrow[e1] = s1 ? 1 : 0;
    count += (unsigned long long)(__popcll(m0) + __popcll(m1));
    wave_sync();  // sbuf is rewritten for the next row
  }
  // one pair of atomics per workgroup
  if (lane == 0) scount[wave] = count;
  __syncthreads();
  if (tid == 0) {
    unsigned long long tot = 0;
    for (int w = 0; w < kWaves; ++w) tot += scount[w];
    if (tot) {
      atomicAdd((unsigned long long*)&a.st->pruned, tot);
      atomicAdd(a.blk_count, tot);
    }
  }
}

unsigned errors_grid(int64_t c) {
  int64_t g = cdiv(c, kWaves);
  if (g > 512) g = 512;
  return (unsigned)g;
}

}  // namespace

hipError_t launch_sgpt_gdiag(const float* U, int64_t b, float* g, hipStream_t s) {
  hipLaunchKernelGGL(sgpt_gdiag_kernel, dim3((unsigned)cdiv(b, 256)), dim3(256), 0, s, U, b, g);
  return hipGetLastError();
}

hipError_t launch_sgpt_errors(const float* W, int64_t c, int64_t b, int64_t j0, int64_t B, int n,
                              int m, int unstructured, const float* U, const float* g, float* E,
                              int64_t lde, uint8_t* mask, DevState* st,
                              unsigned long long* blk_count, hipStream_t s) {
  SgptArgs a;
  a.W = W; a.c = c; a.b = b; a.j0 = j0;
  a.Bb = (int)((b - j0) < B ? (b - j0) : B);
  a.n = n; a.m = m; a.U = U; a.g = g; a.E = E; a.lde = lde;
  a.mask = mask; a.st = st; a.blk_count = blk_count;
  if (unstructured)
    hipLaunchKernelGGL((sgpt_errors_kernel<1>), dim3(errors_grid(c)), dim3(kWaves * 64), 0, s, a);
  else
    hipLaunchKernelGGL((sgpt_errors_kernel<0>), dim3(errors_grid(c)), dim3(kWaves * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace th
