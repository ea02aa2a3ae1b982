// Mask selection inside a block and the per-row joint solve.
//
// "Pruning LLMs with Thanos", section "Contribution one: solve a selected set
// directly": for row k with selected set Q (s entries) and u = W[k, Q], the
// update is delta = -u Rhat^-1 R with Rhat = [A_F]_{Q,Q} and R = [A_F]_{Q,F}.
// Each wave owns one row at a time and computes the coefficients z = u Rhat^-1
// (scattered into Z[k, J], zero outside Q); the update kernel then applies
// W[:, F] -= Z [A_F]_{J,F} on the matrix cores.
//
// Solving: lane a holds row a of the system in 64 registers (fully unrolled) and
// the right-hand side in one more; Gauss-Jordan elimination without pivoting
// (the systems are symmetric positive definite). The pivot row of step j is
// column j of the still-symmetric trailing block, so broadcasting it costs one
// LDS store per lane. Rows with s < 64 are padded with identity rows and zero
// right-hand sides, which contribute nothing ("Making irregular row masks
// batchable").
//
// Route A (s <= 64): the system is Rhat = M[Q,Q] with M = [A_F]_{J,J} in LDS.
// Route B (s > 64, only when B > 64): with N = M^-1 and P = J \ Q (p = B - s < 64
// entries), Rhat^-1 = N_QQ - N_QP N_PP^-1 N_PQ, so one p x p system suffices:
//   N_PP x = N_PQ u^T,  v = [v_Q = u, v_P = -x],  z_Q = (v N)_Q.
//
// Masks: N:M ("The compression target: linear layers"; the explainer's "N:M
// Semi-Structured Sparsity (2:4 Pattern)"): in every aligned group of m entries
// the m-n lowest (score, column) are pruned. Unstructured: the entries of the
// block whose key (score bits, flat index) lies below the global threshold.
#include "common.h"

namespace th {

namespace {

constexpr int kWaves = 8;
// M (or N) in LDS, 128 x 128 with an XOR swizzle: entry (r, q) sits at
// r * 128 + (q ^ (r & 31)), so the per-lane row gathers of the solve (one
// column, 64 different rows) hit distinct banks without padding the pitch.
__device__ __forceinline__ int mat_idx(int r, int q) { return r * kMaxBlock + (q ^ (r & 31)); }

// Gauss-Jordan on 64 registers per lane: rows = lanes, all 64 steps (rows and
// columns past the system size hold the identity and a zero right-hand side, so
// their steps change nothing). Returns x_lane = rhs_lane / pivot_lane. The pivot
// row of step j equals column j of the (still symmetric) trailing block, i.e.
// lane c's register j. Entries c < kLdsFrom are broadcast with v_readlane (a
// VALU op each); for c >= kLdsFrom every lane stores its register j into a
// per-wave LDS row and the entries are read back as wave-uniform 128-bit loads,
// which moves part of the broadcast work from the VALU to the LDS pipe. The
// pivot reciprocal is rcp plus one Newton step. Each step's pivot goes straight
// into its lane of a VGPR (v_writelane), and `lane` arrives through an opaque
// move inside the caller's row loop: otherwise the compiler keeps all 64 pivots
// and hoists all 64 lane masks as SGPRs for the whole loop and spills them.
// The elimination runs at the fp32 VALU rate (a wave64 FMA takes four cycles of
// a 16-lane SIMD): about 20 us of a 2:4 block's 37 us at c = 4096.
constexpr int kLdsFrom = 32;

__device__ __forceinline__ float gauss_jordan64(float (&reg)[64], float rhs, float* row, int lane) {
  float piv = 1.f;
  static_for<0, 64>([&](auto J) __attribute__((always_inline)) {
    constexpr int j = J;
    if constexpr (j + 1 < 64) row[lane] = reg[j];
    const float p = bcast(reg[j], j);
    const float rj = bcast(rhs, j);
    float pinv = __builtin_amdgcn_rcpf(p);
    pinv = pinv * fmaf(-p, pinv, 2.f);
    const float f = (lane == j) ? 0.f : reg[j] * pinv;
    // lane j's pivot, written straight into lane j (no select chain kept alive)
    __asm__ volatile("v_writelane_b32 %0, %1, %2" : "+v"(piv) : "s"(p), "n"(j));
    rhs = fmaf(-f, rj, rhs);
    static_for<j + 1, 64>([&](auto C) __attribute__((always_inline)) {
      constexpr int c = C;
      const float v = (c >= kLdsFrom) ? row[c] : bcast(reg[j], c);
      reg[c] = fmaf(-f, v, reg[c]);
    });
  });
  return rhs / piv;
}

struct SolveArgs {
  const float* W;      // working weights, c x b
  int64_t c, b, j0;
  int Bb, B;           // block width, N row pitch
  int64_t ldz;         // Z row pitch
  int n, m;            // N:M (mode 0)
  const float* R;      // transformed rows: R[J, F] = [A_F]_{J,F}
  const float* Nblk;   // this block's N (route B), B x B
  const float* g;      // g_q source: mode 0 Wanda: gW; mode 1: D row (OBS) or gW
  int g_mode;          // 0: 1/M_qq (OBS, N:M), 2: g[q] given (OBS unstructured, Wanda)
  float* Z;            // c rows, pitch ldz: this block's coefficients
  uint8_t* mask;       // c x b
  DevState* st;
  unsigned long long* blk_count;
};

template <int MODE, int ROUTE>
__global__ __launch_bounds__(kWaves * 64, 4) void solve_kernel(SolveArgs a) {
  __shared__ float sM[kMaxBlock * kMaxBlock];
  __shared__ float sg[kMaxBlock];
  __shared__ float sbuf[kWaves][kMaxBlock];
  __shared__ float su[kWaves][kMaxBlock];
  __shared__ int sQ[kWaves][kMaxBlock];
  // sP (route B's complement list) is read only by the gather before the
  // elimination, which then reuses the same words as its LDS pivot row.
  __shared__ __attribute__((aligned(16))) int sP[kWaves][64];
  __shared__ unsigned long long scount[kWaves];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Bb = a.Bb;
  const int64_t b = a.b, j0 = a.j0;
  {  // M (or N): all 32 loads of a thread in flight at once, addresses clamped
    const float* src = (ROUTE == 0) ? a.R + j0 * b + j0 : a.Nblk;
    const int64_t ld = (ROUTE == 0) ? b : a.B;
    constexpr int kPer = kMaxBlock * kMaxBlock / (kWaves * 64);
    float v[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int idx = e * kWaves * 64 + tid, r = idx >> 7, q = idx & (kMaxBlock - 1);
      const int rr = r < Bb ? r : Bb - 1, qq = q < Bb ? q : Bb - 1;
      v[e] = src[rr * ld + qq];
    }
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int idx = e * kWaves * 64 + tid, r = idx >> 7, q = idx & (kMaxBlock - 1);
      if (r < Bb && q < Bb) sM[mat_idx(r, q)] = v[e];
    }
  }
  for (int q = tid; q < Bb; q += blockDim.x) {
    float gq;
    if (a.g_mode == 0) gq = __fdiv_rn(1.0f, a.R[(j0 + q) * b + j0 + q]);
    else gq = a.g[j0 + q];
    sg[q] = gq;
  }
  __syncthreads();
  const unsigned long long tbound = (MODE == 1) ? a.st->tbound : 0ull;
  const unsigned long long lt = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  unsigned long long count = 0;

  for (int64_t k = (int64_t)blockIdx.x * kWaves + wave; k < a.c; k += (int64_t)gridDim.x * kWaves) {
    const int e0 = lane, e1 = lane + 64;
    const bool v0 = e0 < Bb, v1 = e1 < Bb;
    const float* wrow = a.W + k * b + j0;
    const float w0 = v0 ? wrow[e0] : 0.f;
    const float w1 = v1 ? wrow[e1] : 0.f;
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
    const int s = __popcll(m0) + __popcll(m1);
    if (MODE == 1) {
      if (ROUTE == 0 && s > 64) continue;
      if (ROUTE == 1 && s <= 64) continue;
    }
    uint8_t* mrow = a.mask + k * b + j0;
    if (v0) mrow[e0] = s0 ? 1 : 0;
    if (v1) mrow[e1] = s1 ? 1 : 0;
    float* zrow = a.Z + k * a.ldz;
    if (v0 && !s0) zrow[e0] = 0.f;
    if (v1 && !s1) zrow[e1] = 0.f;
    const int pos0 = __popcll(m0 & lt), pos1 = __popcll(m0) + __popcll(m1 & lt);
    if (s0) { sQ[wave][pos0] = e0; su[wave][pos0] = w0; }
    if (s1) { sQ[wave][pos1] = e1; su[wave][pos1] = w1; }
    if (ROUTE == 1) {
      const unsigned long long n0 = __ballot(v0 && !s0), n1 = __ballot(v1 && !s1);
      const int pp0 = __popcll(n0 & lt), pp1 = __popcll(n0) + __popcll(n1 & lt);
      if (v0 && !s0) sP[wave][pp0] = e0;
      if (v1 && !s1) sP[wave][pp1] = e1;
    }
    wave_sync();
    if (s > 0) {
      // The lane index through an opaque move: the per-step lane masks are then
      // formed inside the row loop (one compare each) instead of being hoisted out
      // of it as 64-bit SGPR masks that spill.
      int olane;
      __asm__ volatile("v_mov_b32 %0, %1" : "=v"(olane) : "v"(lane));
      float reg[64];
      if (ROUTE == 0) {
        const bool act = lane < s;
        const int qa = act ? sQ[wave][lane] : 0;
#pragma unroll
        for (int c = 0; c < 64; ++c) {  // branch-free, so all 64 reads are in flight
          const bool in = (c < s) && act;
          const int qc = (c < s) ? sQ[wave][c] : 0;
          const float v = sM[mat_idx(qa, qc)];
          reg[c] = in ? v : ((c == olane) ? 1.f : 0.f);
        }
        const float u = act ? su[wave][lane] : 0.f;
        wave_sync();  // the gather's reads are done before the pivot row is written
        const float z = gauss_jordan64(reg, u, (float*)sP[wave], olane);
        if (act) zrow[qa] = z;
      } else {
        const int p = Bb - s;
        const bool act = lane < p;
        const int pb = act ? sP[wave][lane] : 0;
#pragma unroll
        for (int c = 0; c < 64; ++c) {
          const bool in = (c < p) && act;
          const int pc = (c < p) ? sP[wave][c] : 0;
          const float v = sM[mat_idx(pb, pc)];
          reg[c] = in ? v : ((c == olane) ? 1.f : 0.f);
        }
        float y = 0.f;
        if (act) {
          for (int t = 0; t < s; ++t) y = fmaf(su[wave][t], sM[mat_idx(sQ[wave][t], pb)], y);
        }
        wave_sync();  // the gather's reads of sP are done before it becomes the pivot row
        const float x = gauss_jordan64(reg, y, (float*)sP[wave], olane);
        // v = [u on Q, -x on P], then z_q = (v N)_q for q in Q
        if (act) sbuf[wave][pb] = -x;
        if (s0) sbuf[wave][e0] = w0;
        if (s1) sbuf[wave][e1] = w1;
        wave_sync();
        float z0 = 0.f, z1 = 0.f;
        for (int t = 0; t < Bb; ++t) {
          const float vt = sbuf[wave][t];
          if (v0) z0 = fmaf(vt, sM[mat_idx(t, e0)], z0);
          if (v1) z1 = fmaf(vt, sM[mat_idx(t, e1)], z1);
        }
        if (s0) zrow[e0] = z0;
        if (s1) zrow[e1] = z1;
      }
    }
    count += (unsigned long long)s;
    wave_sync();
  }
  // one pair of atomics per workgroup (same-address atomics serialise in L2)
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

// Parity entry: N:M selection on given scores, one wave per row.
__global__ __launch_bounds__(256) void debug_select_nm_kernel(const float* __restrict__ S,
                                                              int64_t c, int64_t blk, int n,
                                                              int m, uint8_t* __restrict__ mask) {
  __shared__ float sc[4][kMaxBlock * 8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t k = (int64_t)blockIdx.x * 4 + wave;
  if (k >= c) return;
  for (int64_t e = lane; e < blk; e += 64) sc[wave][e] = S[k * blk + e];
  wave_sync();
  for (int64_t e = lane; e < blk; e += 64) mask[k * blk + e] = nm_pruned(sc[wave], (int)e, n, m) ? 1 : 0;
}

// Parity entry: block mask and per-row counts from given scores and the threshold.
__global__ void debug_mask_kernel(const float* __restrict__ S, int64_t c, int64_t f,
                                  int64_t b_full, int64_t j0, int64_t blk, const DevState* st,
                                  uint8_t* __restrict__ mask, int32_t* __restrict__ s_k) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= c) return;
  const unsigned long long tb = st->tbound;
  int cnt = 0;
  for (int64_t q = 0; q < blk; ++q) {
    const bool sel = make_key(S[k * f + q], (unsigned int)(k * b_full + j0 + q)) < tb;
    mask[k * blk + q] = sel ? 1 : 0;
    cnt += sel;
  }
  if (s_k) s_k[k] = cnt;
}

unsigned solve_grid(int64_t c) {
  int64_t g = cdiv(c, kWaves);
  if (g > 512) g = 512;
  return (unsigned)g;
}

}  // namespace

hipError_t launch_solve_nm(const float* W, int64_t c, int64_t b, int64_t j0, int64_t B, int n,
                           int m, const float* R, const float* gW, const float* Nblk, float* Z,
                           int64_t ldz, uint8_t* mask, DevState* st, unsigned long long* blk_count,
                           hipStream_t s) {
  SolveArgs a;
  a.W = W; a.c = c; a.b = b; a.j0 = j0;
  a.Bb = (int)((b - j0) < B ? (b - j0) : B);
  a.B = (int)B; a.n = n; a.m = m; a.R = R; a.Nblk = Nblk;
  a.g = gW; a.g_mode = gW ? 2 : 0;
  a.Z = Z; a.ldz = ldz; a.mask = mask; a.st = st; a.blk_count = blk_count;
  const int sel = a.Bb / m * (m - n);
  if (sel <= 64)
    hipLaunchKernelGGL((solve_kernel<0, 0>), dim3(solve_grid(c)), dim3(kWaves * 64), 0, s, a);
  else
    hipLaunchKernelGGL((solve_kernel<0, 1>), dim3(solve_grid(c)), dim3(kWaves * 64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_solve_unstructured(const float* W, int64_t c, int64_t b, int64_t j0, int64_t B,
                                     const float* R, const float* Nblk, const float* g,
                                     float* Z, uint8_t* mask, DevState* st,
                                     unsigned long long* blk_count, hipStream_t s) {
  SolveArgs a;
  a.W = W; a.c = c; a.b = b; a.j0 = j0;
  a.Bb = (int)((b - j0) < B ? (b - j0) : B);
  a.B = (int)B; a.n = 0; a.m = 1; a.R = R; a.Nblk = Nblk;
  a.g = g; a.g_mode = 2;  // per-column score weight given (1/[A_F]_qq or G_qq)
  a.Z = Z; a.ldz = B; a.mask = mask; a.st = st; a.blk_count = blk_count;
  hipLaunchKernelGGL((solve_kernel<1, 0>), dim3(solve_grid(c)), dim3(kWaves * 64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.Bb <= 64) return e;
  hipLaunchKernelGGL((solve_kernel<1, 1>), dim3(solve_grid(c)), dim3(kWaves * 64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_debug_select_nm(const float* scores, int64_t c, int64_t blk, int n, int m,
                                  uint8_t* mask, hipStream_t s) {
  hipLaunchKernelGGL(debug_select_nm_kernel, dim3((unsigned)cdiv(c, 4)), dim3(256), 0, s, scores,
                     c, blk, n, m, mask);
  return hipGetLastError();
}

hipError_t launch_debug_mask_from_scores(const float* scores, int64_t c, int64_t f,
                                         int64_t b_full, int64_t j0, int64_t blk,
                                         const DevState* st, uint8_t* mask, int32_t* s_k,
                                         hipStream_t s) {
  hipLaunchKernelGGL(debug_mask_kernel, dim3((unsigned)cdiv(c, 256)), dim3(256), 0, s, scores, c,
                     f, b_full, j0, blk, st, mask, s_k);
  return hipGetLastError();
}

}  // namespace th
