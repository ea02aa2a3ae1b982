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
// (64-byte rows: X 16 KB, W_gate and W_up 8 KB each) are filled by direct
// global->LDS loads, four stages deep with the loads three stages ahead, and the
// operand fragments are double-buffered across the two 16-wide substeps of a
// stage. The 16-byte pieces of a row are XOR-swizzled by (row / 4) & 3, so the
// operand reads (16 rows at one piece per 16 lanes) use all 64 banks; a load lane
// fetches whichever piece its fixed LDS slot holds. Tiles are walked in groups
// of 8 token tiles per feature-tile column, and each XCD takes a contiguous range
// of that order, so the 32 workgroups an XCD runs at once share their X and W
// slices in its L2.
#include "common.h"
#include "lds_dma.h"

namespace th {

namespace {

constexpr int kFM = 256;     // tokens per tile
constexpr int kFN = 128;     // features per tile
constexpr int kFK = 32;      // contraction per stage
constexpr int kFThreads = 256;
constexpr int kFStages = 4;
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

  __shared__ __attribute__((aligned(1024))) unsigned char sm0[kStage];
  __shared__ __attribute__((aligned(1024))) unsigned char sm1[kStage];
  __shared__ __attribute__((aligned(1024))) unsigned char sm2[kStage];
  __shared__ __attribute__((aligned(1024))) unsigned char sm3[kStage];
  auto buf = [&](auto S) -> unsigned char* {
    constexpr int s = decltype(S)::value;
    if constexpr (s == 0) return sm0;
    else if constexpr (s == 1) return sm1;
    else if constexpr (s == 2) return sm2;
    else return sm3;
  };
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;  // wave tile: tokens wm*128.., features wn*64..

  // Loader: a stage is 32 chunks of 1 KB (16 rows of 64 bytes): X chunks 0..15,
  // W_gate 16..23, W_up 24..31. Wave w loads X chunks w + 4m (m = 0..3) and gate
  // and up chunks w + 4m (m = 0, 1); with lds_dma_stage's slots (lds + 4096 i in
  // the order 0, 4, 1, 5, 2, 6, 3, 7 for i = 0..7) from base = stage + 1024 w, the
  // sources are ordered X0, G0, X1, G1, X2, U0, X3, U1. Lane l fills row
  // 16 chunk + l/4 at physical piece l%4, i.e. logical piece lp below.
  const int lrow = lane >> 2;
  const int64_t nk = cdiv(d, kFK);
  const unsigned short* src[8];
  int lp[8];
  {
    const int chunk[8] = {wave, 16 + wave, wave + 4, 16 + wave + 4, wave + 8, 24 + wave,
                          wave + 12, 24 + wave + 4};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = chunk[i];
      const int mat = c < 16 ? 0 : (c < 24 ? 1 : 2);
      const int row = (c - (mat == 0 ? 0 : (mat == 1 ? 16 : 24))) * 16 + lrow;
      lp[i] = (lane & 3) ^ ((row >> 2) & 3);
      int64_t r = (mat == 0 ? M0 : N0) + row;
      const int64_t lim = mat == 0 ? n : f;
      r = r < lim ? r : lim - 1;  // rows past the end feed outputs that are never stored
      const unsigned short* base = mat == 0 ? X : (mat == 1 ? Wg : Wu);
      src[i] = base + r * d + lp[i] * 8;
    }
  }
  auto issue_stage = [&](int64_t st, unsigned char* sbase) {
    const int64_t k0 = st * kFK;
    const void* g[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) g[i] = src[i] + ((k0 + lp[i] * 8 < d) ? k0 : 0);
    lds_dma_stage(g, sbase + wave * 1024);
  };
  // zero this wave's pieces of stage st that lie past d (its own loads have landed)
  auto zero_tail = [&](int64_t st, unsigned char* sbase) {
    const int64_t k0 = st * kFK;
    if (k0 + kFK <= d) return;
    constexpr int slot[8] = {0, 4, 1, 5, 2, 6, 3, 7};
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (k0 + lp[i] * 8 >= d)
        *(u32x4_t*)(sbase + wave * 1024 + slot[i] * 4096 + lane * 16) = u32x4_t{0u, 0u, 0u, 0u};
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
  const int r32 = lane & 31, half = lane >> 5;
  bf16x8_t a0[4], g0[2], u0[2], a1[4], g1[2], u1[2];
  auto read_frags = [&](const unsigned char* st, int sub, bf16x8_t (&a)[4], bf16x8_t (&g)[2],
                        bf16x8_t (&u)[2]) {
    const int pc = sub * 2 + half;  // piece of this lane's 8 k values
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *(const bf16x8_t*)(st + sw_off(wm * 128 + i * 32 + r32, pc));
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      g[j] = *(const bf16x8_t*)(st + kABytes + sw_off(wn * 64 + j * 32 + r32, pc));
      u[j] = *(const bf16x8_t*)(st + kABytes + kBBytes + sw_off(wn * 64 + j * 32 + r32, pc));
    }
  };
  auto mfmas = [&](const bf16x8_t (&a)[4], const bf16x8_t (&g)[2], const bf16x8_t (&u)[2]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        accG[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], g[j], accG[i][j], 0, 0, 0);
        accU[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], u[j], accU[i][j], 0, 0, 0);
      }
  };

  // prologue: stages 0, 1, 2 in flight; wait for stage 0
  issue_stage(0, sm0);
  issue_stage(1, sm1);
  issue_stage(2, sm2);
  __asm__ volatile("s_waitcnt vmcnt(16)" ::: "memory");
  zero_tail(0, sm0);
  __syncthreads();
  read_frags(sm0, 0, a0, g0, u0);
  for (int64_t it0 = 0; it0 < nk; it0 += kFStages) {
    static_for<0, kFStages>([&](auto U) __attribute__((always_inline)) {
      constexpr int uu = U;
      const int64_t it = it0 + uu;
      if (it < nk) {
        // buffer (uu+3)%4 was last read before the barrier of iteration it-1
        issue_stage(it + 3, buf(std::integral_constant<int, (uu + 3) % kFStages>{}));
        read_frags(buf(std::integral_constant<int, uu>{}), 1, a1, g1, u1);
        mfmas(a0, g0, u0);
        // stage it+1 complete for this wave (stages it+2, it+3 may still be in flight)
        __asm__ volatile("s_waitcnt vmcnt(16)" ::: "memory");
        unsigned char* nb = buf(std::integral_constant<int, (uu + 1) % kFStages>{});
        zero_tail(it + 1, nb);
        __syncthreads();
        read_frags(nb, 0, a0, g0, u0);
        mfmas(a1, g1, u1);
      }
    });
  }
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");

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
