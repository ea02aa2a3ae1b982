// Input of down_proj from the (pruned) gate and up projections of a gated
// feed-forward: Y = silu(X W_gate^T) * (X W_up^T), X token-major [n, d], W [f, d],
// Y [n, f], all bf16; products exact in fp32 on the matrix cores, fp32 sums,
// silu(z) = z / (1 + e^-z) in fp32, the product rounded once to bf16.
//
// "Pruning LLMs with Thanos", section "The compression target: linear layers": a
// block's feed-forward projections are joined by a nonlinearity; gate_proj,
// up_proj and down_proj are LLaMA's gated feed-forward. Pruned layers are
// calibrated on the inputs their pruned predecessors produce ("The
// layer-reconstruction lens": each layer is reconstructed from its own inputs).
//
// One workgroup computes a 256-token x 128-feature tile of both products (4 waves
// as 2 x 2, each 128 x 64 of gate and of up: 16 v_mfma_f32_32x32x16_bf16
// accumulators in AGPRs), so the epilogue has g and u of every output at hand.
// The contraction dimension d is contiguous in both operands, so an MFMA operand
// (8 consecutive k of one row per lane) is one 16-byte LDS read. K stages of 32
// (64-byte rows, 32 KB per stage) are double-buffered and filled through
// registers; the 16-byte pieces of a row are XOR-swizzled by (row / 4) & 3 so
// that the operand reads (16 rows at one piece per 16 lanes) and the fills (4
// rows x 4 pieces) use all 64 banks. Tiles are walked in groups of 8 token tiles
// per feature-tile column, and each XCD takes a contiguous range of that order,
// so the 32 workgroups an XCD runs at once share their X and W slices in its L2.
#include "common.h"

namespace th {

namespace {

constexpr int kFM = 256;     // tokens per tile
constexpr int kFN = 128;     // features per tile
constexpr int kFK = 32;      // contraction per stage
constexpr int kFThreads = 256;
constexpr int kFGroup = 8;   // token tiles per group in the walk order
constexpr int kRow = kFK * 2;                 // bytes per staged row
constexpr int kABytes = kFM * kRow;           // 16 KB
constexpr int kBBytes = kFN * kRow;           // 8 KB per weight matrix
constexpr int kStage = kABytes + 2 * kBBytes; // 32 KB

__device__ __forceinline__ int sw_off(int r, int piece) {
  return r * kRow + ((piece ^ ((r >> 2) & 3)) << 4);
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + expf(-z)); }

// Tile (tm, tn) of walk position lin: groups of kFGroup token tiles, feature
// tiles column by column inside a group.
__device__ __forceinline__ void ffn_tile(int lin, int ntm, int ntn, int& tm, int& tn) {
  const int per_group = kFGroup * ntn;
  const int g = lin / per_group, in = lin - g * per_group;
  const int m0 = g * kFGroup;
  const int gs = min(kFGroup, ntm - m0);
  tm = m0 + in % gs;
  tn = in / gs;
}

__global__ __launch_bounds__(kFThreads) void gated_ffn_kernel(
    const unsigned short* __restrict__ X, const unsigned short* __restrict__ Wg,
    const unsigned short* __restrict__ Wu, unsigned short* __restrict__ Y, int64_t n, int64_t d,
    int64_t f, int ntm, int ntn, int per_xcd) {
  const int wg = blockIdx.x;
  const int lin = (wg % 8) * per_xcd + wg / 8;
  if (lin >= ntm * ntn) return;
  int tm, tn;
  ffn_tile(lin, ntm, ntn, tm, tn);
  const int64_t M0 = (int64_t)tm * kFM, N0 = (int64_t)tn * kFN;

  __shared__ __attribute__((aligned(1024))) unsigned char sm[2][kStage];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;  // wave tile: tokens wm*128.., features wn*64..

  // Fill assignment: thread tid moves piece (tid & 3) of rows (tid >> 2) + 64 i:
  // A rows i = 0..3, gate rows i = 0..1, up rows i = 0..1.
  const int prow = tid >> 2, piece = tid & 3;
  const unsigned short* srcA[4];
  const unsigned short* srcG[2];
  const unsigned short* srcU[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int64_t r = M0 + prow + 64 * i;
    r = r < n ? r : n - 1;
    srcA[i] = X + r * d + piece * 8;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    int64_t r = N0 + prow + 64 * i;
    r = r < f ? r : f - 1;
    srcG[i] = Wg + r * d + piece * 8;
    srcU[i] = Wu + r * d + piece * 8;
  }
  u32x4_t rA[4], rG[2], rU[2];
  const int nk = (int)cdiv(d, kFK);
  auto load = [&](int ks) {
    const int64_t k0 = (int64_t)ks * kFK;
    const bool in = k0 + piece * 8 < d;  // d % 8 == 0: a piece is wholly in or out
    const int64_t off = in ? k0 : 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rA[i] = *(const u32x4_t*)(srcA[i] + off);
      if (!in) rA[i] = u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      rG[i] = *(const u32x4_t*)(srcG[i] + off);
      rU[i] = *(const u32x4_t*)(srcU[i] + off);
      if (!in) {
        rG[i] = u32x4_t{0u, 0u, 0u, 0u};
        rU[i] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store = [&](unsigned char* st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *(u32x4_t*)(st + sw_off(prow + 64 * i, piece)) = rA[i];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      *(u32x4_t*)(st + kABytes + sw_off(prow + 64 * i, piece)) = rG[i];
      *(u32x4_t*)(st + kABytes + kBBytes + sw_off(prow + 64 * i, piece)) = rU[i];
    }
  };

  f32x16_t accG[4][2], accU[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        accG[i][j][e] = 0.f;
        accU[i][j][e] = 0.f;
      }

  load(0);
  store(sm[0]);
  __syncthreads();
  const int r32 = lane & 31, half = lane >> 5;
  for (int ks = 0; ks < nk; ++ks) {
    const unsigned char* cur = sm[ks & 1];
    if (ks + 1 < nk) load(ks + 1);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int pc = sub * 2 + half;  // piece of this lane's 8 k values
      bf16x8_t a[4], g[2], u[2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *(const bf16x8_t*)(cur + sw_off(wm * 128 + i * 32 + r32, pc));
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        g[j] = *(const bf16x8_t*)(cur + kABytes + sw_off(wn * 64 + j * 32 + r32, pc));
        u[j] = *(const bf16x8_t*)(cur + kABytes + kBBytes + sw_off(wn * 64 + j * 32 + r32, pc));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          accG[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], g[j], accG[i][j], 0, 0, 0);
          accU[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], u[j], accU[i][j], 0, 0, 0);
        }
    }
    if (ks + 1 < nk) {
      store(sm[(ks + 1) & 1]);  // the other buffer: its last reads ended at the barrier below
    }
    __syncthreads();
  }

  // Epilogue: lane holds feature column r32 of each 32 x 32 block and rows
  // 8 (e / 4) + 4 half + (e % 4).
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = N0 + wn * 64 + j * 32 + r32;
      if (col >= f) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = M0 + wm * 128 + i * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
        if (row < n) {
          const float y = silu_f32(accG[i][j][e]) * accU[i][j][e];
          Y[row * f + col] = f32_to_bf16_rne(y);
        }
      }
    }
}

}  // namespace

hipError_t launch_gated_ffn(const unsigned short* X, const unsigned short* Wg,
                            const unsigned short* Wu, unsigned short* Y, int64_t n, int64_t d,
                            int64_t f, hipStream_t s) {
  const int ntm = (int)cdiv(n, kFM), ntn = (int)cdiv(f, kFN);
  const int64_t ntiles = (int64_t)ntm * ntn;
  const int per_xcd = (int)cdiv(ntiles, 8);
  hipLaunchKernelGGL(gated_ffn_kernel, dim3((unsigned)(8 * per_xcd)), dim3(kFThreads), 0, s, X, Wg,
                     Wu, Y, n, d, f, ntm, ntn, per_xcd);
  return hipGetLastError();
}

}  // namespace th
