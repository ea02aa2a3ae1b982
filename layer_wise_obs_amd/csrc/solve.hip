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
// Unstructured rows take either route, so that launch holds both M and N in LDS
// (one workgroup per compute unit) and picks the route per row: one launch per
// block instead of one per route, each of which paid the loads and the row scan.
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
// Largest inner dimension of the folded group product (seven earlier blocks of 128).
constexpr int kLocalMaxK = 7 * kMaxBlock;

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

// ROUTE: 0 route A, 1 route B, 2 the route of each row (M and N both in LDS).
template <int MODE, int ROUTE, int NW = kWaves>
__global__ __launch_bounds__(NW * 64, NW == 16 ? 4 : (ROUTE == 2 ? 2 : 4)) void solve_kernel(SolveArgs a) {
  __shared__ float sM[kMaxBlock * kMaxBlock];
  __shared__ float sN2[ROUTE == 2 ? kMaxBlock * kMaxBlock : 1];
  __shared__ float sg[kMaxBlock];
  __shared__ float sbuf[NW][kMaxBlock];
  __shared__ float su[NW][kMaxBlock];
  __shared__ int sQ[NW][kMaxBlock];
  // sP (route B's complement list) is read only by the gather before the
  // elimination, which then reuses the same words as its LDS pivot row.
  __shared__ __attribute__((aligned(16))) int sP[NW][64];
  __shared__ unsigned long long scount[NW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Bb = a.Bb;
  const int64_t b = a.b, j0 = a.j0;
  // route B's matrix: N, in sM (route B alone) or in sN2 (both routes)
  float* const sN = (ROUTE == 2) ? sN2 : sM;
  // M (or N): all 32 loads of a thread in flight at once, addresses clamped
  auto load_mat = [&](const float* src, int64_t ld, float* dst) {
    constexpr int kPer = kMaxBlock * kMaxBlock / (NW * 64);
    float v[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int idx = e * NW * 64 + tid, r = idx >> 7, q = idx & (kMaxBlock - 1);
      const int rr = r < Bb ? r : Bb - 1, qq = q < Bb ? q : Bb - 1;
      v[e] = src[rr * ld + qq];
    }
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int idx = e * NW * 64 + tid, r = idx >> 7, q = idx & (kMaxBlock - 1);
      if (r < Bb && q < Bb) dst[mat_idx(r, q)] = v[e];
    }
  };
  if (ROUTE != 1) load_mat(a.R + j0 * b + j0, b, sM);
  if (ROUTE != 0) load_mat(a.Nblk, a.B, sN);
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

  for (int64_t k = (int64_t)blockIdx.x * NW + wave; k < a.c; k += (int64_t)gridDim.x * NW) {
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
    const bool rb = (ROUTE == 1) || (ROUTE == 2 && s > 64);  // this row takes route B (uniform)
    uint8_t* mrow = a.mask + k * b + j0;
    if (v0) mrow[e0] = s0 ? 1 : 0;
    if (v1) mrow[e1] = s1 ? 1 : 0;
    float* zrow = a.Z + k * a.ldz;
    if (v0 && !s0) zrow[e0] = 0.f;
    if (v1 && !s1) zrow[e1] = 0.f;
    const int pos0 = __popcll(m0 & lt), pos1 = __popcll(m0) + __popcll(m1 & lt);
    if (s0) { sQ[wave][pos0] = e0; su[wave][pos0] = w0; }
    if (s1) { sQ[wave][pos1] = e1; su[wave][pos1] = w1; }
    if (rb) {
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
      if (!rb) {
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
          const float v = sN[mat_idx(pb, pc)];
          reg[c] = in ? v : ((c == olane) ? 1.f : 0.f);
        }
        float y = 0.f;
        if (act) {
          for (int t = 0; t < s; ++t) y = fmaf(su[wave][t], sN[mat_idx(sQ[wave][t], pb)], y);
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
          if (v0) z0 = fmaf(vt, sN[mat_idx(t, e0)], z0);
          if (v1) z1 = fmaf(vt, sN[mat_idx(t, e1)], z1);
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
    for (int w = 0; w < NW; ++w) tot += scount[w];
    if (tot) {
      atomicAdd((unsigned long long*)&a.st->pruned, tot);
      atomicAdd(a.blk_count, tot);
    }
  }
}

// N:M, route A (s <= 64), with the block-local compensation of the block's group
// folded into the solve. Under N:M no budget couples the rows, so each row's
// blocks can be taken left-looking: before scoring block J, a workgroup
// subtracts from its rows' W[k, J] the compensation of the earlier blocks
// of the same group -- their coefficients (Z, columns 0 .. Kp of the group's
// rows) times their slices R[J_i, J] -- and after the solve it writes the block's
// final weights: W[k, q] - (z M)[q] on the kept columns, exact zeros on the
// pruned ones ("Pruning LLMs with Thanos", section "Contribution one: solve a
// selected set directly"). The columns past the group are updated once per group,
// by the far-column update, from the same Z. This replaces one update launch per
// block; the arithmetic is the same products summed in another order.
//
// A workgroup takes kLocalRows rows (one wave each). The group's product runs on
// the fp32 matrix cores (v_mfma_f32_16x16x4f32: the 16 rows of the batch times
// 16-column pieces of R[r0:j0, J]): the batch's coefficients are staged in LDS
// first (the space of M, which is loaded after the product), R is read from global
// memory in 256-byte row pieces, three chunks ahead, and the eight parts of the
// inner index meet in LDS, added in a fixed order.
constexpr int kLocalRows = 16;

__global__ __launch_bounds__(kLocalRows * 64, 4) void solve_nm_local_kernel(
    SolveArgs a, float* Ww, int64_t r0, int Kp, void* Wout, int out_bf16, int64_t pf_r0,
    int pf_rows, int64_t pf_col0, int pf_cols) {
  constexpr int kW = kLocalRows;
  __shared__ __attribute__((aligned(16))) float sM[kMaxBlock * kMaxBlock];
  __shared__ float sg[kMaxBlock];
  __shared__ float sbuf[kW][kMaxBlock];
  __shared__ float su[kW][kMaxBlock];
  __shared__ int sQ[kW][kMaxBlock];
  __shared__ __attribute__((aligned(16))) int sP[kW][64];
  __shared__ unsigned long long scount[kW];
  static_assert(kW * kLocalMaxK <= kMaxBlock * kMaxBlock, "staged coefficients fit in M's space");
  static_assert(kW / 2 * kW * kMaxBlock <= kMaxBlock * kMaxBlock, "partial sums fit in M's space");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Bb = a.Bb;
  const int64_t b = a.b, j0 = a.j0, c = a.c, ldz = a.ldz;
  const float* Zg = a.Z - Kp;  // the group's first coefficient column
  for (int q = tid; q < Bb; q += blockDim.x) {
    float gq;
    if (a.g_mode == 0) gq = __fdiv_rn(1.0f, a.R[(j0 + q) * b + j0 + q]);
    else gq = a.g[j0 + q];
    sg[q] = gq;
  }
  const unsigned long long lt = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  unsigned long long count = 0;

  // What the next block of the group reads of R (rows pf_r0 .. +pf_rows, columns
  // pf_col0 .. +pf_cols: its M and the slab of its group product) is pulled into
  // L2 now: workgroup w runs on XCD w % 8, and each of the nx workgroups of an
  // XCD reads every nx-th row (32 rows per workgroup, 16 bytes per thread). The
  // values are consumed by an empty asm at the end; since the load counter
  // completes in order, the first wait for this block's own loads also covers
  // these, whose latency thus overlaps that of the block's first loads.
  f32x4_t pf = {0.f, 0.f, 0.f, 0.f};
  {
    const int nx = (int)((gridDim.x + 7) / 8), widx = (int)(blockIdx.x / 8);
    const int seg = tid & 31, row = widx + nx * (tid >> 5);
    if (row < pf_rows && 4 * seg < pf_cols)
      pf = *(const f32x4_t*)(a.R + (pf_r0 + row) * a.b + pf_col0 + 4 * seg);
  }

  const int64_t kb = (int64_t)blockIdx.x * kW;
  const int64_t k = kb + wave;
  const bool rowv = k < c;
  const int e0 = lane, e1 = lane + 64;
  const bool v0 = e0 < Bb, v1 = e1 < Bb;
  float* wrow = Ww + (rowv ? k : 0) * b + j0;
  float w0 = (rowv && v0) ? wrow[e0] : 0.f;
  float w1 = (rowv && v1) ? wrow[e1] : 0.f;
  if (Kp > 0) {
    float* const sZ = sM;  // sZ[kk * kW + r]
    {  // all loads of a thread in flight at once (Kp <= kLocalMaxK)
      constexpr int kH = (kLocalMaxK + kW * 64 - 1) / (kW * 64);
      float zv[kW][kH];
#pragma unroll
      for (int r = 0; r < kW; ++r) {
        const int64_t row = (kb + r) < c ? (kb + r) : (c - 1);
#pragma unroll
        for (int h = 0; h < kH; ++h) {
          const int kk = tid + h * kW * 64;
          zv[r][h] = kk < Kp ? Zg[row * ldz + kk] : 0.f;
        }
      }
#pragma unroll
      for (int r = 0; r < kW; ++r) {
#pragma unroll
        for (int h = 0; h < kH; ++h) {
          const int kk = tid + h * kW * 64;
          if (kk < Kp) sZ[kk * kW + r] = zv[r][h];
        }
      }
    }
    __syncthreads();
    // Wave w takes columns 64 (w % 2) .. +63 and eighth w / 2 of the inner index.
    // Per step of 4 inner indices a lane reads four adjacent columns of one row of R
    // (16 bytes; a row of 16 lanes covers 256 contiguous bytes) and feeds four MFMAs:
    //   A[i][kk] = Z[row i][kk]            (lane: i = lane % 16, kk = step + lane / 16)
    //   B_e[kk][j] = R[r0 + kk][j0 + c0 + 4 j + e], e = 0..3 (lane: kk as A, j = lane % 16)
    const int wv = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform, in scalar registers
    const int ch = wv & 1, ks = wv >> 1;
    constexpr int kSplit = kW / 2;
    const int kbeg = ks * Kp / kSplit, kend = (ks + 1) * Kp / kSplit;
    const int li = lane & 15, lk = lane >> 4;
    const int c0 = ch * 64 + 4 * li;  // a multiple of 4; Bb is too on this path
    const float* Rc = a.R + r0 * b + j0 + (c0 < Bb ? c0 : Bb - 4);
    f32x4_t acc[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // R in chunks of kU steps, three chunks in flight. Loads and LDS reads past the
    // range are clamped into it (no branch around a load) and their coefficient is
    // multiplied by zero: R and Z are finite, so those products add exact zeros.
    constexpr int kU = 4, kC = 4 * kU;
    float4 ra[kU], rb[kU], rc[kU];
    auto load_chunk = [&](int kk0, float4 (&dst)[kU]) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int kk = kk0 + 4 * u + lk;
        dst[u] = *(const float4*)(Rc + (int64_t)(kk < kend ? kk : kend - 1) * b);
      }
    };
    auto mfma_chunk = [&](int kk0, const float4 (&src)[kU]) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int kk = kk0 + 4 * u + lk;
        const float zi = sZ[(kk < kend ? kk : kend - 1) * kW + li] * (kk < kend ? 1.f : 0.f);
        acc[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(zi, src[u].x, acc[0], 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(zi, src[u].y, acc[1], 0, 0, 0);
        acc[2] = __builtin_amdgcn_mfma_f32_16x16x4f32(zi, src[u].z, acc[2], 0, 0, 0);
        acc[3] = __builtin_amdgcn_mfma_f32_16x16x4f32(zi, src[u].w, acc[3], 0, 0, 0);
      }
    };
    if (kend > kbeg) {  // wave-uniform
      load_chunk(kbeg, ra);
      load_chunk(kbeg + kC, rb);
      load_chunk(kbeg + 2 * kC, rc);
    }
    for (int kk0 = kbeg; kk0 < kend; kk0 += 3 * kC) {
      mfma_chunk(kk0, ra);
      if (kk0 + 3 * kC < kend) load_chunk(kk0 + 3 * kC, ra);
      if (kk0 + kC < kend) {
        mfma_chunk(kk0 + kC, rb);
        if (kk0 + 4 * kC < kend) load_chunk(kk0 + 4 * kC, rb);
      }
      if (kk0 + 2 * kC < kend) {
        mfma_chunk(kk0 + 2 * kC, rc);
        if (kk0 + 5 * kC < kend) load_chunk(kk0 + 5 * kC, rc);
      }
    }
    __syncthreads();  // every wave is done with the staged coefficients
    // D_e[i][j] in register r of lane l: i = 4 (l / 16) + r, j = l % 16 -> column c0 + e
    float* const part = sM;  // part[eighth][row][column]
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float* pr = part + (ks * kW + 4 * lk + r) * kMaxBlock + c0;
      *(float4*)pr = float4{acc[0][r], acc[1][r], acc[2][r], acc[3][r]};
    }
    __syncthreads();
    const float* p0 = part + wave * kMaxBlock;
    constexpr int kPart = kW * kMaxBlock;
    float s0 = 0.f, s1 = 0.f;  // the eighths in a fixed order
#pragma unroll
    for (int e = 0; e < kSplit; ++e) {
      s0 += p0[e * kPart + e0];
      s1 += p0[e * kPart + e1];
    }
    if (v0) w0 -= s0;
    if (v1) w1 -= s1;
    __syncthreads();  // the partial sums are read before M overwrites them
  }
  {  // M = [A_F]_{J,J}: all 16 loads of a thread in flight at once, addresses clamped
    constexpr int kPer = kMaxBlock * kMaxBlock / (kW * 64);
    const float* src = a.R + j0 * b + j0;
    float v[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int idx = e * kW * 64 + tid, r = idx >> 7, q = idx & (kMaxBlock - 1);
      const int rr = r < Bb ? r : Bb - 1, qq = q < Bb ? q : Bb - 1;
      v[e] = src[rr * b + qq];
    }
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int idx = e * kW * 64 + tid, r = idx >> 7, q = idx & (kMaxBlock - 1);
      if (r < Bb && q < Bb) sM[mat_idx(r, q)] = v[e];
    }
  }
  __syncthreads();
  if (rowv) {
    if (v0) sbuf[wave][e0] = score_of(w0, sg[e0]);
    if (v1) sbuf[wave][e1] = score_of(w1, sg[e1]);
    wave_sync();
    const bool s0 = v0 && nm_pruned(sbuf[wave], e0, a.n, a.m);
    const bool s1 = v1 && nm_pruned(sbuf[wave], e1, a.n, a.m);
    const unsigned long long m0 = __ballot(s0), m1 = __ballot(s1);
    const int s = __popcll(m0) + __popcll(m1);
    uint8_t* mrow = a.mask + k * b + j0;
    if (v0) mrow[e0] = s0 ? 1 : 0;
    if (v1) mrow[e1] = s1 ? 1 : 0;
    float* zrow = a.Z + k * ldz;
    if (v0 && !s0) zrow[e0] = 0.f;
    if (v1 && !s1) zrow[e1] = 0.f;
    const int pos0 = __popcll(m0 & lt), pos1 = __popcll(m0) + __popcll(m1 & lt);
    if (s0) { sQ[wave][pos0] = e0; su[wave][pos0] = w0; }
    if (s1) { sQ[wave][pos1] = e1; su[wave][pos1] = w1; }
    wave_sync();
    float d0 = 0.f, d1 = 0.f;
    if (s > 0) {
      int olane;
      __asm__ volatile("v_mov_b32 %0, %1" : "=v"(olane) : "v"(lane));
      float reg[64];
      const bool act = lane < s;
      const int qa = act ? sQ[wave][lane] : 0;
#pragma unroll
      for (int cc = 0; cc < 64; ++cc) {
        const bool in = (cc < s) && act;
        const int qc = (cc < s) ? sQ[wave][cc] : 0;
        const float v = sM[mat_idx(qa, qc)];
        reg[cc] = in ? v : ((cc == olane) ? 1.f : 0.f);
      }
      const float u = act ? su[wave][lane] : 0.f;
      wave_sync();
      const float z = gauss_jordan64(reg, u, (float*)sP[wave], olane);
      if (act) zrow[qa] = z;
      // the block's own compensation: d_e = sum over the selected t of z_t M[Q_t, e],
      // unrolled over all 64 lanes (lanes past s hold z = 0 and Q = 0, so they add
      // exact zeros) so that the reads of M are independent of each other
      const float za = act ? z : 0.f;
      static_for<0, 64>([&](auto T) __attribute__((always_inline)) {
        constexpr int t = T;
        const float zt = bcast(za, t);
        const int qt = __builtin_amdgcn_readlane(qa, t);
        // mat_idx(qt, e1) = mat_idx(qt, e0) + 64 (the swizzle changes the low 5 bits only)
        const int i0 = mat_idx(qt, e0);
        d0 = fmaf(zt, sM[i0], d0);
        d1 = fmaf(zt, sM[i0 + 64], d1);
      });
    }
    const float f0 = s0 ? 0.f : w0 - d0, f1 = s1 ? 0.f : w1 - d1;
    if (v0) wrow[e0] = f0;
    if (v1) wrow[e1] = f1;
    if (Wout) {  // the block's columns are final: the output dtype's copy too
      if (out_bf16) {
        unsigned short* o = (unsigned short*)Wout + k * b + j0;
        if (v0) o[e0] = f32_to_bf16_rne(f0);
        if (v1) o[e1] = f32_to_bf16_rne(f1);
      } else {
        float* o = (float*)Wout + k * b + j0;
        if (v0) o[e0] = f0;
        if (v1) o[e1] = f1;
      }
    }
    count = (unsigned long long)s;
  }
  if (lane == 0) scount[wave] = count;
  __asm__ volatile("" ::"v"(pf[0]), "v"(pf[1]), "v"(pf[2]), "v"(pf[3]));
  __syncthreads();
  if (tid == 0) {
    unsigned long long tot = 0;
    for (int w = 0; w < kW; ++w) tot += scount[w];
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

bool solve_nm_local_applies(int64_t b, int64_t B, int n, int m) {
  // route A in every block; widths that are multiples of 4 for the 16-byte reads of R
  return B / m * (m - n) <= 64 && b % 4 == 0 && B % 4 == 0;
}

hipError_t launch_solve_nm_local(float* W, int64_t c, int64_t b, int64_t j0, int64_t B, int n,
                                 int m, const float* R, const float* gW, float* Z, int64_t ldz,
                                 int64_t r0, uint8_t* mask, DevState* st,
                                 unsigned long long* blk_count, void* Wout, th_dtype wdt,
                                 int64_t group_end, hipStream_t s) {
  SolveArgs a;
  a.W = W; a.c = c; a.b = b; a.j0 = j0;
  a.Bb = (int)((b - j0) < B ? (b - j0) : B);
  a.B = (int)B; a.n = n; a.m = m; a.R = R; a.Nblk = nullptr;
  a.g = gW; a.g_mode = gW ? 2 : 0;
  a.Z = Z; a.ldz = ldz; a.mask = mask; a.st = st; a.blk_count = blk_count;
  if (!solve_nm_local_applies(b, B, n, m) || j0 < r0 || j0 - r0 > kLocalMaxK)
    return hipErrorInvalidValue;
  if (c == 0) return hipSuccess;
  // one batch of kLocalRows rows per workgroup
  const int64_t g = cdiv(c, kLocalRows);
  if (g > 0x7fffffff) return hipErrorInvalidValue;
  // the next block, if it belongs to the same group (rows r0 .. its end, its columns)
  const int64_t jn = j0 + a.Bb;
  const int64_t bn = jn < group_end ? ((b - jn) < B ? (b - jn) : B) : 0;
  const int pf_rows = bn > 0 ? (int)(jn + bn - r0) : 0;
  hipLaunchKernelGGL(solve_nm_local_kernel, dim3((unsigned)g), dim3(kLocalRows * 64), 0, s, a, W,
                     r0, (int)(j0 - r0), Wout, wdt == TH_BF16 ? 1 : 0, r0, pf_rows, jn, (int)bn);
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
  if (a.Bb <= 64)
    hipLaunchKernelGGL((solve_kernel<1, 0>), dim3(solve_grid(c)), dim3(kWaves * 64), 0, s, a);
  else
    // one workgroup per compute unit fits (M and N take 128 KB of LDS), of 16 waves
    // (four per SIMD: the eliminations of four rows share each SIMD): a grid of 256
    // runs in one round, each wave taking its rows in turn
    hipLaunchKernelGGL((solve_kernel<1, 2, 16>), dim3((unsigned)(cdiv(c, 16) < 256 ? cdiv(c, 16) : 256)),
                       dim3(16 * 64), 0, s, a);
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
