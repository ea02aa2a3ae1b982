// Hessian accumulation H += 2 X^T X (lower triangle) and its damping.
//
// "Weight Pruning in Large Language Models ..." (explainer), section "SparseGPT:
// Second-Order Reconstruction at Scale": H = 2XX^T + lambda*I. "Pruning LLMs with
// Thanos", section "One deletion with compensation: the OBS view": G = XX^T is the
// Gram matrix, lambda*I is added for numerical stability.
//
// bf16 path: 256x256 output tiles of the lower triangle, 512 threads (8 waves as
// 2 x 4, each wave 128x64 = 4x2 blocks of v_mfma_f32_32x32x16_bf16; two waves per
// SIMD so one wave's loads, transposes and LDS traffic overlap the other's MFMAs).
// Tokens are the contraction dimension; X^T arrives token-major, so every thread
// loads an 8-token x 8-feature brick (eight 16-byte loads) of one panel,
// transposes them in registers with v_perm_b32 and stores 8 feature rows of 8
// tokens (16 bytes each) into LDS, where the MFMA operands are read as 16-byte
// K-contiguous vectors. The LDS row pitch of 72 bf16 (36 dwords) makes both the
// stores and the operand reads bank-conflict free. Two LDS stages (144 KB) give one
// barrier per 64 tokens; inside a stage the operand fragments are double-buffered
// in registers and the next stage's transpose-store is split into four parts
// interleaved with the four k-substeps of MFMAs. The loop body is branch-free
// (clamped loads, stores into the idle buffer), so the compiler can interleave
// LDS traffic, VALU transposes and MFMAs of one wave, and the two waves of a
// SIMD no longer alternate between an MFMA phase and a store phase.
#include "common.h"

namespace th {

namespace {

constexpr int kTile = 256;
constexpr int kBK = 64;
constexpr int kPitch = 72;  // bf16 elements per LDS feature row (64 tokens + 8 pad)
constexpr int kThreads = 512;

// 8 tokens x 8 features starting at (tok0, f0). b is a multiple of 8, so a
// feature group is either fully inside or fully outside. Addresses are clamped
// instead of branched on (loads stay branch-free and in bounds); the returned
// bit mask marks the valid rows, and zeroing happens in transpose_store, so
// nothing waits for the loads until the data is stored to LDS.
__device__ __forceinline__ unsigned load_brick(const unsigned short* __restrict__ X, int64_t ldx,
                                               int64_t t_valid, int64_t b, int64_t tok0,
                                               int64_t f0, u32x4_t (&v)[8]) {
  const bool fok = f0 < b;
  const int64_t fc = fok ? f0 : 0;
  unsigned ok = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t t = tok0 + i;
    const int64_t tc = (t < t_valid) ? t : (t_valid - 1);
    v[i] = *(const u32x4_t*)(X + tc * ldx + fc);
    ok |= (fok && t < t_valid) ? (1u << i) : 0u;
  }
  return ok;
}

// Part d (0..3) of transpose_store: features 2d and 2d+1 of the brick.
__device__ __forceinline__ void transpose_store_part(unsigned short* __restrict__ s, int frow0,
                                                     int oct, const u32x4_t (&v)[8], unsigned ok,
                                                     int d) {
  u32x4_t lo, hi;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const unsigned a = ((ok >> (2 * p)) & 1u) ? v[2 * p][d] : 0u;
    const unsigned c = ((ok >> (2 * p + 1)) & 1u) ? v[2 * p + 1][d] : 0u;
    lo[p] = __builtin_amdgcn_perm(c, a, 0x05040100u);
    hi[p] = __builtin_amdgcn_perm(c, a, 0x07060302u);
  }
  *(u32x4_t*)(s + (frow0 + 2 * d) * kPitch + oct * 8) = lo;
  *(u32x4_t*)(s + (frow0 + 2 * d + 1) * kPitch + oct * 8) = hi;
}

// 8 tokens x 8 features (v[token].dword[f/2]) -> 8 features x 8 tokens; rows
// whose bit is clear in `ok` are stored as zeros.
__device__ __forceinline__ void transpose_store(unsigned short* __restrict__ s, int frow0, int oct,
                                                const u32x4_t (&v)[8], unsigned ok) {
  u32x4_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = ((ok >> i) & 1u) ? v[i] : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    u32x4_t lo, hi;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      lo[p] = __builtin_amdgcn_perm(w[2 * p + 1][d], w[2 * p][d], 0x05040100u);
      hi[p] = __builtin_amdgcn_perm(w[2 * p + 1][d], w[2 * p][d], 0x07060302u);
    }
    *(u32x4_t*)(s + (frow0 + 2 * d) * kPitch + oct * 8) = lo;
    *(u32x4_t*)(s + (frow0 + 2 * d + 1) * kPitch + oct * 8) = hi;
  }
}

// Tile order for L2 reuse: the lower triangle of nt x nt tiles is walked in
// super-tiles of 4 tile rows x 8 tile columns (row-major inside each), super-
// tiles row by row. Returns tile (ti, tj) of position lin.
constexpr int kSupR = 4, kSupC = 8;
__device__ __forceinline__ void tile_of(int lin, int nt, int& ti, int& tj) {
  for (int sr = 0; sr * kSupR < nt; ++sr) {
    const int r0 = sr * kSupR, r1 = min(nt, r0 + kSupR);
    for (int sc = 0; sc * kSupC <= r1 - 1; ++sc) {
      const int c0 = sc * kSupC, c1 = c0 + kSupC;
      int cnt = 0;  // tiles (r, c) with r0 <= r < r1, c0 <= c < c1, c <= r
      for (int r = r0; r < r1; ++r) cnt += max(0, min(c1, r + 1) - c0);
      if (lin < cnt) {
        for (int r = r0; r < r1; ++r) {
          const int w = max(0, min(c1, r + 1) - c0);
          if (lin < w) {
            ti = r;
            tj = c0 + lin;
            return;
          }
          lin -= w;
        }
      }
      lin -= cnt;
    }
  }
  ti = tj = 0;  // not reached for lin < nt(nt+1)/2
}

__global__ __launch_bounds__(kThreads) void syrk_bf16_kernel(
    float* __restrict__ H, const unsigned short* __restrict__ X, int64_t t, int64_t b, int64_t ldx,
    int ntile_rows, int ntiles, int per_xcd, int splits, int64_t tok_per_split,
    float* __restrict__ partials) {
  // XCD-aware order: consecutive workgroup ids go to different XCDs, so each XCD
  // gets a contiguous run of the super-tile order below; the ~32 tiles an XCD
  // runs at once then share 4 row panels and 8 column panels in its L2.
  const int wg = blockIdx.x;
  const int lin = (wg % 8) * per_xcd + wg / 8;
  const int split = blockIdx.y;
  if (lin >= ntiles) return;
  int ti, tj;
  tile_of(lin, ntile_rows, ti, tj);
  const bool diag = (ti == tj);
  const int64_t I0 = (int64_t)ti * kTile, J0 = (int64_t)tj * kTile;

  // two pipeline stages x (A panel, B panel), each 256 features x 64 tokens
  __shared__ __attribute__((aligned(16))) unsigned short smem[2 * 2 * kTile * kPitch];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int part = tid >> 8;             // 0: A panel, 1: B panel
  const int q = tid & 255;
  const int oct = q & 7, fgrp = q >> 3;  // 8 token octets x 32 feature groups
  const int64_t fbase = (part == 0 ? I0 : J0) + fgrp * 8;

  const int64_t k_begin = (int64_t)split * tok_per_split;
  const int64_t k_end = (k_begin + tok_per_split < t) ? k_begin + tok_per_split : t;
  const int nk = (int)cdiv(k_end - k_begin, kBK);

  f32x16_t acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][c][r] = 0.f;

  const int wrow = wave >> 2, wcol = wave & 3;
  const int lr = lane & 31, lk = lane >> 5;

  auto sbuf = [&](int stage, int panel) { return smem + (stage * 2 + panel) * (kTile * kPitch); };
  u32x4_t v[8];
  unsigned ok = 0;
  ok = load_brick(X, ldx, k_end, b, k_begin + oct * 8, fbase, v);
  transpose_store(sbuf(0, part), fgrp * 8, oct, v, ok);
  ok = load_brick(X, ldx, k_end, b, k_begin + kBK + oct * 8, fbase, v);
  __syncthreads();
  for (int it = 0; it < nk; ++it) {
    const int cur = it & 1;
    const unsigned short* sA = sbuf(cur, 0);
    const unsigned short* sB = diag ? sA : sbuf(cur, 1);
    // Every thread loads and stores every iteration (branch-free loop body): on
    // diagonal tiles the second half of the threads fills the unused B buffer,
    // and past the last stage the clamped loads and stores land in the buffer
    // that is no longer read.
    unsigned short* snext = sbuf(cur ^ 1, part);
    // Operand fragments are double-buffered in registers: the reads for
    // k-substep ks+1 are issued before the MFMAs of ks, and a quarter of the
    // next stage's transpose-store follows each substep's MFMAs.
    bf16x8_t af[2][4], bfr[2][2];
#pragma unroll
    for (int a = 0; a < 4; ++a)
      af[0][a] = *(const bf16x8_t*)(sA + (wrow * 128 + a * 32 + lr) * kPitch + lk * 8);
#pragma unroll
    for (int c = 0; c < 2; ++c)
      bfr[0][c] = *(const bf16x8_t*)(sB + (wcol * 64 + c * 32 + lr) * kPitch + lk * 8);
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int cb = ks & 1, nb = cb ^ 1;
      if (ks + 1 < kBK / 16) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
          af[nb][a] = *(const bf16x8_t*)(sA + (wrow * 128 + a * 32 + lr) * kPitch + (ks + 1) * 16 +
                                         lk * 8);
#pragma unroll
        for (int c = 0; c < 2; ++c)
          bfr[nb][c] = *(const bf16x8_t*)(sB + (wcol * 64 + c * 32 + lr) * kPitch +
                                          (ks + 1) * 16 + lk * 8);
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 2; ++c)
          acc[a][c] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cb][a], bfr[cb][c], acc[a][c], 0, 0, 0);
      transpose_store_part(snext, fgrp * 8, oct, v, ok, ks);
    }
    ok = load_brick(X, ldx, k_end, b, k_begin + (int64_t)(it + 2) * kBK + oct * 8, fbase, v);
    __syncthreads();
  }

  if (splits == 1) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = I0 + wrow * 128 + a * 32 + 8 * (r >> 2) + 4 * lk + (r & 3);
          const int64_t col = J0 + wcol * 64 + c * 32 + lr;
          if (row < b && col < b && col <= row) H[row * b + col] += 2.0f * acc[a][c][r];
        }
  } else {
    float* dst = partials + ((int64_t)split * ntiles + lin) * (int64_t)(kTile * kTile);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wrow * 128 + a * 32 + 8 * (r >> 2) + 4 * lk + (r & 3);
          const int col = wcol * 64 + c * 32 + lr;
          dst[row * kTile + col] = acc[a][c][r];
        }
  }
}

// Fixed-order sum of the token splits: H += 2 * sum_s partial_s.
__global__ void syrk_reduce_kernel(float* __restrict__ H, const float* __restrict__ partials,
                                   int64_t b, int ntiles, int splits) {
  const int lin = blockIdx.x;
  int ti, tj;
  tile_of(lin, (int)cdiv(b, kTile), ti, tj);
  const int64_t I0 = (int64_t)ti * kTile, J0 = (int64_t)tj * kTile;
  for (int e = threadIdx.x; e < kTile * kTile; e += blockDim.x) {
    const int r = e / kTile, c = e % kTile;
    const int64_t row = I0 + r, col = J0 + c;
    if (row >= b || col >= b || col > row) continue;
    float s = 0.f;
    for (int sp = 0; sp < splits; ++sp)
      s += partials[((int64_t)sp * ntiles + lin) * (int64_t)(kTile * kTile) + e];
    H[row * b + col] += 2.0f * s;
  }
}

// fp32 inputs (small layers): 32x32 tiles of the lower triangle, one thread per entry.
__global__ __launch_bounds__(256) void syrk_f32_kernel(float* __restrict__ H,
                                                       const float* __restrict__ X, int64_t t,
                                                       int64_t b, int64_t ldx) {
  __shared__ float sa[16][33], sb[16][33];
  const int64_t I0 = (int64_t)blockIdx.y * 32, J0 = (int64_t)blockIdx.x * 32;
  if (J0 > I0) return;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // ty 0..7
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int64_t k0 = 0; k0 < t; k0 += 16) {
    for (int e = threadIdx.x; e < 16 * 32; e += 256) {
      const int kk = e / 32, cc = e % 32;
      const int64_t tok = k0 + kk;
      sa[kk][cc] = (tok < t && I0 + cc < b) ? X[tok * ldx + I0 + cc] : 0.f;
      sb[kk][cc] = (tok < t && J0 + cc < b) ? X[tok * ldx + J0 + cc] : 0.f;
    }
    __syncthreads();
    for (int kk = 0; kk < 16; ++kk) {
      const float bj = sb[kk][tx];
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = fmaf(sa[kk][ty * 4 + r], bj, acc[r]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t row = I0 + ty * 4 + r, col = J0 + tx;
    if (row < b && col < b && col <= row) H[row * b + col] += 2.0f * acc[r];
  }
}

// lambda from the mean of diag(H). If H is an accumulated (undamped) 2G, the
// relative rule gives lambda = rel * mean(diag 2G). If H is already damped with
// a relative lambda, mean(diag H) = (1+rel) mean(diag 2G), which recovers it.
__global__ void lambda_kernel(const float* __restrict__ H, int64_t b, double lam, int rel,
                              int h_is_damped, DevState* st) {
  __shared__ double red[256];
  __shared__ int bad;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  double s = 0.0;
  int lbad = 0;
  for (int64_t q = threadIdx.x; q < b; q += blockDim.x) {
    const float d = H[q * b + q];
    if (!isfinite(d)) lbad = 1;
    s += (double)d;
  }
  red[threadIdx.x] = s;
  if (lbad) atomicOr(&bad, 1);
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double mean = red[0] / (double)b;
    double l;
    if (!rel) l = lam;
    else if (h_is_damped) l = lam / (1.0 + lam) * mean;
    else l = lam * mean;
    st->diag_mean = h_is_damped ? mean - l : mean;
    st->lambda = l;
    if (bad) st->nonfinite = 1;
  }
}

// Finalize: H_qq += lambda and mirror the lower triangle onto the upper one.
__global__ void damp_mirror_kernel(float* __restrict__ H, int64_t b, float lam) {
  __shared__ float tile[32][33];
  const int64_t I0 = (int64_t)blockIdx.y * 32, J0 = (int64_t)blockIdx.x * 32;
  if (J0 > I0) return;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int r = ty; r < 32; r += 8) {
    const int64_t row = I0 + r, col = J0 + tx;
    float v = 0.f;
    if (row < b && col < b) {
      v = H[row * b + col];
      if (row == col) {
        v += lam;
        H[row * b + col] = v;
      }
    }
    tile[r][tx] = v;
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int64_t row = J0 + r, col = I0 + tx;  // upper entry (row < col) mirrors (col,row)
    if (row < b && col < b && col > row) H[row * b + col] = tile[tx][r];
  }
}

// S = P H P restricted to its lower triangle, P the reversal permutation:
// S[i][j] = H[b-1-j][b-1-i] for j <= i (a lower entry of H), + lambda on the diagonal.
__global__ void flip_lower_kernel(const float* __restrict__ H, float* __restrict__ S, int64_t b,
                                  const DevState* st, int add_lambda) {
  __shared__ float tile[32][33];
  const int64_t I0 = (int64_t)blockIdx.y * 32, J0 = (int64_t)blockIdx.x * 32;
  if (J0 > I0) return;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  // Read H rows b-1-(J0+r), columns b-1-(I0+tx): a column-reversed, row-reversed block.
  for (int r = ty; r < 32; r += 8) {
    const int64_t hr = b - 1 - (J0 + r), hc = b - 1 - (I0 + tx);
    tile[r][tx] = (hr >= 0 && hc >= 0) ? H[hr * b + hc] : 0.f;
  }
  __syncthreads();
  const float lam = add_lambda ? (float)st->lambda : 0.f;
  for (int r = ty; r < 32; r += 8) {
    const int64_t i = I0 + r, j = J0 + tx;
    if (i < b && j < b && j <= i) {
      float v = tile[tx][r];  // = H[b-1-j][b-1-i]
      if (i == j) v += lam;
      S[i * b + j] = v;
    }
  }
}

// Wanda score factor g_q = G_qq = (H_qq - lambda)/2 for a damped H, H_qq/2 for 2G.
__global__ void wanda_diag_kernel(const float* __restrict__ H, int64_t b, const DevState* st,
                                  int h_is_damped, float* __restrict__ g) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= b) return;
  const double l = h_is_damped ? st->lambda : 0.0;
  g[q] = (float)(((double)H[q * b + q] - l) * 0.5);
}

}  // namespace

int syrk_bf16_splits(int64_t t, int64_t b) {
  const int64_t nt = cdiv(b, kTile);
  const int64_t ntiles = nt * (nt + 1) / 2;
  int64_t splits = 1;
  const int64_t target = 512;  // about two workgroups per CU
  if (ntiles < target) splits = cdiv(target, ntiles);
  const int64_t max_by_tokens = cdiv(t, 4 * kBK);  // keep >= 256 tokens per split
  if (splits > max_by_tokens) splits = max_by_tokens;
  if (splits < 1) splits = 1;
  if (splits > 16) splits = 16;
  return (int)splits;
}

hipError_t launch_syrk_bf16(float* H, const unsigned short* X, int64_t t, int64_t b, int64_t ldx,
                            float* partials, int splits, hipStream_t s) {
  if (t <= 0 || b <= 0) return hipSuccess;
  const int nt = (int)cdiv(b, kTile);
  const int ntiles = nt * (nt + 1) / 2;
  const int per_xcd = (int)cdiv(ntiles, 8);
  if (partials == nullptr) splits = 1;
  int64_t tps = cdiv(cdiv(t, splits), kBK) * kBK;
  splits = (int)cdiv(t, tps);
  dim3 grid(per_xcd * 8, splits);
  hipLaunchKernelGGL(syrk_bf16_kernel, grid, dim3(kThreads), 0, s, H, X, t, b, ldx, nt, ntiles,
                     per_xcd, splits, tps, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  hipLaunchKernelGGL(syrk_reduce_kernel, dim3(ntiles), dim3(256), 0, s, H, partials, b, ntiles,
                     splits);
  return hipGetLastError();
}

hipError_t launch_syrk_f32(float* H, const float* X, int64_t t, int64_t b, int64_t ldx,
                           hipStream_t s) {
  if (t <= 0 || b <= 0) return hipSuccess;
  const int nt = (int)cdiv(b, 32);
  hipLaunchKernelGGL(syrk_f32_kernel, dim3(nt, nt), dim3(256), 0, s, H, X, t, b, ldx);
  return hipGetLastError();
}

hipError_t launch_lambda(const float* H, int64_t b, double lam, int rel, int h_is_damped,
                         DevState* st, hipStream_t s) {
  hipLaunchKernelGGL(lambda_kernel, dim3(1), dim3(256), 0, s, H, b, lam, rel, h_is_damped, st);
  return hipGetLastError();
}

hipError_t launch_damp_mirror(float* H, int64_t b, float lam, hipStream_t s) {
  const int nt = (int)cdiv(b, 32);
  hipLaunchKernelGGL(damp_mirror_kernel, dim3(nt, nt), dim3(256), 0, s, H, b, lam);
  return hipGetLastError();
}

hipError_t launch_flip_lower(const float* H, float* S, int64_t b, const DevState* st,
                             int add_lambda, hipStream_t s) {
  const int nt = (int)cdiv(b, 32);
  hipLaunchKernelGGL(flip_lower_kernel, dim3(nt, nt), dim3(256), 0, s, H, S, b, st, add_lambda);
  return hipGetLastError();
}

hipError_t launch_wanda_diag(const float* H, int64_t b, const DevState* st, int h_is_damped,
                             float* gdiag, hipStream_t s) {
  hipLaunchKernelGGL(wanda_diag_kernel, dim3((unsigned)cdiv(b, 256)), dim3(256), 0, s, H, b, st,
                     h_is_damped, gdiag);
  return hipGetLastError();
}

}  // namespace th
