// Hessian accumulation H += 2 X^T X (lower triangle) and its damping.
//
// "Weight Pruning in Large Language Models ..." (explainer), section "SparseGPT:
// Second-Order Reconstruction at Scale": H = 2XX^T + lambda*I. "Pruning LLMs with
// Thanos", section "One deletion with compensation: the OBS view": G = XX^T is the
// Gram matrix, lambda*I is added for numerical stability.
//
// bf16 path: 256x256 output tiles of the lower triangle, 256 threads (4 waves as
// 2 x 2, each wave 128x128 = 4x4 blocks of v_mfma_f32_32x32x16_bf16 with the
// accumulators in AGPRs). Tokens are the contraction dimension and X^T arrives
// token-major, so the tiles are staged in LDS as they are in memory (token rows
// of 256 features) with direct global->LDS loads (global_load_lds_dwordx4, no
// register staging), and the MFMA operands -- 8 consecutive tokens of one feature
// per lane -- are formed by the gfx950 transposing LDS read ds_read_b64_tr_b16.
// The 16-byte pieces of a token row are XOR-swizzled by (token & 3) so that those
// reads spread over all banks. Four LDS stages of 32 tokens (128 KB) keep the
// loads three stages ahead; operand fragments are double-buffered in registers
// across the 16-token substeps, so the reads for the next substep overlap the
// current substep's 16 MFMAs.
#include "common.h"
#include "lds_dma.h"

namespace th {

namespace {

constexpr int kTile = 256;
constexpr int kBK = 64;  // token granularity of the split ranges

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

constexpr int kDBK = 32;       // tokens per LDS stage
constexpr int kDStages = 4;    // LDS stages (loads run three stages ahead)
constexpr int kDThreads = 256; // 4 waves, 2 x 2, each 128 x 128
constexpr int kRowBytes = kTile * 2;                  // one token row of a panel
constexpr int kPanelBytes = kDBK * kRowBytes;         // 16 KB
constexpr int kStageBytes = 2 * kPanelBytes;          // A and B panels

// Byte offset of (token t, 8-feature piece fg) inside a panel: token-major rows of
// 512 bytes, pieces XOR-swizzled by (t & 3) so that the transposing operand reads
// of 8 tokens x 32 features spread over all banks.
__device__ __forceinline__ int piece_off(int t, int fg) { return t * kRowBytes + ((fg ^ ((t & 3) << 2)) << 4); }

typedef short v4i16_t __attribute__((ext_vector_type(4)));

// MFMA operand (32 features x 16 tokens, k-substep at token ks16) from a panel:
// lane L gets feature f0 + L%32, tokens ks16 + 8*(L/32) + 0..7. Each
// ds_read_b64_tr_b16 transposes, per 16-lane group, 4 tokens x 16 features: slot
// s reads token tb + s/4, features fb + 4*(s%4) .. +3; lane s then holds feature
// fb + s of the 4 tokens.
__device__ __forceinline__ bf16x8_t tr_frag(const unsigned char* panel, int f0, int ks16, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int fb = f0 + ((g & 1) << 4) + ((s & 3) << 2);  // first feature this slot reads
  const int tb = ks16 + ((g >> 1) << 3) + (s >> 2);
  const int fg = fb >> 3, within = (fb & 7) << 1;
  const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16_t*)(panel + piece_off(tb, fg) + within));
  const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16_t*)(panel + piece_off(tb + 4, fg) + within));
  typedef short v8i16_t __attribute__((ext_vector_type(8)));
  const v8i16_t r = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, r);
}

__global__ __launch_bounds__(kDThreads) void syrk_bf16_kernel(
    float* __restrict__ H, const unsigned short* __restrict__ X, int64_t t, int64_t b, int64_t ldx,
    int ntile_rows, int ntiles, int per_xcd, int splits, int64_t tok_per_split,
    float* __restrict__ partials) {
  const int wg = blockIdx.x;
  const int lin = (wg % 8) * per_xcd + wg / 8;
  const int split = blockIdx.y;
  if (lin >= ntiles) return;
  int ti, tj;
  tile_of(lin, ntile_rows, ti, tj);
  const bool diag = (ti == tj);
  const int64_t I0 = (int64_t)ti * kTile, J0 = (int64_t)tj * kTile;

  // One LDS array per stage: with the stage index a compile-time constant the
  // compiler can tell the buffers apart and does not make operand reads wait for
  // the direct-to-LDS loads that are in flight into the other buffers.
  __shared__ __attribute__((aligned(1024))) unsigned char sm0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char sm1[kStageBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char sm2[kStageBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char sm3[kStageBytes];
  auto buf = [&](auto S) -> unsigned char* {
    constexpr int s = decltype(S)::value;
    if constexpr (s == 0) return sm0;
    else if constexpr (s == 1) return sm1;
    else if constexpr (s == 2) return sm2;
    else return sm3;
  };
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t k_begin = (int64_t)split * tok_per_split;
  const int64_t k_end = (k_begin + tok_per_split < t) ? k_begin + tok_per_split : t;
  const int nk = (int)cdiv(k_end - k_begin, kDBK);

  // Loader: per stage and panel, 16 wave instructions of 1 KB (token rows 2i,
  // 2i+1); wave w issues i = w, w+4, w+8, w+12 for both panels. Lane l writes
  // bytes [16 l, 16 l + 16) of the chunk: row 2i + l/32, swizzled position l%32.
  const int lrow = lane >> 5, lpos = lane & 31;
  auto issue_stage = [&](int st, unsigned char* sbase) {
    const int64_t tok0 = k_begin + (int64_t)st * kDBK;
    const void* g[8];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int i = wave + 4 * m;
      const int tr = 2 * i + lrow;  // token row inside the stage
      const int fg = lpos ^ ((tr & 3) << 2);
      int64_t tok = tok0 + tr;
      tok = tok < k_end ? tok : k_end - 1;  // rows past the end are zeroed after the wait
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        int64_t f = (p == 0 ? I0 : J0) + fg * 8;
        f = f < b ? f : 0;  // features past b only feed outputs that are never stored
        g[2 * m + p] = X + tok * ldx + f;  // to sbase + p * kPanelBytes + i * 1024
      }
    }
    static_assert(kPanelBytes == 16384, "LDS offsets in lds_dma_stage");
    lds_dma_stage(g, sbase + wave * 1024);
  };
  // zero this wave's rows of stage st that lie past k_end (its own loads have landed)
  auto zero_tail = [&](int st, unsigned char* sbase) {
    const int64_t tok0 = k_begin + (int64_t)st * kDBK;
    if (tok0 + kDBK <= k_end) return;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int i = wave + 4 * m;
      const int tr = 2 * i + lrow;
      if (tok0 + tr >= k_end) {
#pragma unroll
        for (int p = 0; p < 2; ++p)
          *(u32x4_t*)(sbase + p * kPanelBytes + i * 1024 + lane * 16) = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][c][r] = 0.f;
  const int wrow = wave >> 1, wcol = wave & 1;
  const int lr = lane & 31, lk = lane >> 5;

  bf16x8_t af0[4], bf0[4], af1[4], bf1[4];
  auto read_frags = [&](const unsigned char* pA, int ks, bf16x8_t (&af)[4], bf16x8_t (&bf)[4]) {
    const unsigned char* pB = diag ? pA : pA + kPanelBytes;
#pragma unroll
    for (int a = 0; a < 4; ++a) af[a] = tr_frag(pA, wrow * 128 + a * 32, ks * 16, lane);
#pragma unroll
    for (int c = 0; c < 4; ++c) bf[c] = tr_frag(pB, wcol * 128 + c * 32, ks * 16, lane);
  };
  auto mfmas = [&](const bf16x8_t (&af)[4], const bf16x8_t (&bf)[4]) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bf[c], acc[a][c], 0, 0, 0);
  };

  // prologue: stages 0, 1, 2 in flight; wait for stage 0
  issue_stage(0, sm0);
  issue_stage(1, sm1);
  issue_stage(2, sm2);
  __asm__ volatile("s_waitcnt vmcnt(16)" ::: "memory");
  zero_tail(0, sm0);
  __syncthreads();
  read_frags(sm0, 0, af0, bf0);
  // Fragments are double-buffered across the two 16-token substeps of a stage:
  // the reads for the next substep (or the next stage's first, right after the
  // barrier) are in flight while the current substep's 16 MFMAs run. Unrolled by
  // the number of stages so that every buffer index is a constant.
  for (int it0 = 0; it0 < nk; it0 += kDStages) {
    static_for<0, kDStages>([&](auto U) __attribute__((always_inline)) {
      constexpr int u = U;
      const int it = it0 + u;
      if (it < nk) {
        // buffer (u+3)%4 was last read before the barrier of iteration it-1
        issue_stage(it + 3, buf(std::integral_constant<int, (u + 3) % kDStages>{}));
        read_frags(buf(std::integral_constant<int, u>{}), 1, af1, bf1);
        mfmas(af0, bf0);
        // stage it+1 complete for this wave (stages it+2, it+3 may still be in flight)
        __asm__ volatile("s_waitcnt vmcnt(16)" ::: "memory");
        unsigned char* nb = buf(std::integral_constant<int, (u + 1) % kDStages>{});
        zero_tail(it + 1, nb);
        __syncthreads();
        read_frags(nb, 0, af0, bf0);
        mfmas(af1, bf1);
      }
    });
  }
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  (void)lr;
  (void)lk;

  if (splits == 1) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = I0 + wrow * 128 + a * 32 + 8 * (r >> 2) + 4 * lk + (r & 3);
          const int64_t col = J0 + wcol * 128 + c * 32 + lr;
          if (row < b && col < b && col <= row) H[row * b + col] += 2.0f * acc[a][c][r];
        }
  } else {
    float* dst = partials + ((int64_t)split * ntiles + lin) * (int64_t)(kTile * kTile);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wrow * 128 + a * 32 + 8 * (r >> 2) + 4 * lk + (r & 3);
          const int col = wcol * 128 + c * 32 + lr;
          dst[row * kTile + col] = acc[a][c][r];
        }
  }
}

// ---------------------------------------------------------------- 384 x 256 tiles
// The same pipeline on 384 x 256 rectangles (384 rows of H, 256 columns): each
// wave owns 192 x 128 (6 x 4 accumulator blocks, 384 registers, AGPRs and VGPRs
// together), so a 32-token stage brings 40 KB into LDS for 1.5x the MFMA work of
// a 256 x 256 tile (32 KB): 17% fewer staged bytes per flop. A stage is five
// sub-panels of 128 features (three of the rows, two of the columns), each 32
// token rows of 256 bytes with the 16-byte pieces XOR-swizzled by (token & 3)
// like the square tiles' panels. Loads use the saddr form: a wave-uniform stage
// base plus per-lane offsets fixed for the whole tile.
constexpr int kRR = 384, kRC = 256;            // rows x columns of a rectangle
constexpr int kRSub = 128;                     // features per sub-panel
constexpr int kRSubRow = kRSub * 2;            // 256 bytes: one token row of a sub-panel
constexpr int kRSubBytes = kDBK * kRSubRow;    // 8 KB
constexpr int kRStageBytes = 5 * kRSubBytes;   // 40 KB
constexpr int kRStages = 4;
constexpr int kRLoads = kRStageBytes / 1024 / 4;  // 1 KB loads per wave per stage
static_assert(kRLoads == 10, "lds_dma10s");

// column tiles of strip r that hold an entry on or below the diagonal
__host__ __device__ __forceinline__ int rect_cols(int r, int64_t b) {
  const int64_t last = ((int64_t)kRR * (r + 1) < b ? (int64_t)kRR * (r + 1) : b) - 1;
  return (int)(last / kRC) + 1;
}

// Tile order: super-tiles of 4 strips x 8 column tiles, as for the squares.
__device__ __forceinline__ void rect_tile_of(int lin, int nstrips, int64_t b, int& ti, int& tj) {
  for (int sr = 0; sr * kSupR < nstrips; ++sr) {
    const int r0 = sr * kSupR, r1 = min(nstrips, r0 + kSupR);
    const int cmax = rect_cols(r1 - 1, b);
    for (int sc = 0; sc * kSupC < cmax; ++sc) {
      const int c0 = sc * kSupC, c1 = c0 + kSupC;
      int cnt = 0;
      for (int r = r0; r < r1; ++r) cnt += max(0, min(c1, rect_cols(r, b)) - c0);
      if (lin < cnt) {
        for (int r = r0; r < r1; ++r) {
          const int w = max(0, min(c1, rect_cols(r, b)) - c0);
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
  ti = tj = 0;  // not reached for lin < the tile count
}

// Offset of (token t, piece fg) inside a 128-feature sub-panel.
__device__ __forceinline__ int rpiece_off(int t, int fg) {
  return t * kRSubRow + ((fg ^ ((t & 3) << 2)) << 4);
}

// MFMA operand (32 features from f0 of a sub-panel x 16 tokens from ks16), lane
// layout as in tr_frag.
__device__ __forceinline__ bf16x8_t rtr_frag(const unsigned char* sub, int f0, int ks16, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int fb = f0 + ((g & 1) << 4) + ((s & 3) << 2);
  const int tb = ks16 + ((g >> 1) << 3) + (s >> 2);
  const int fg = fb >> 3, within = (fb & 7) << 1;
  const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16_t*)(sub + rpiece_off(tb, fg) + within));
  const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16_t*)(sub + rpiece_off(tb + 4, fg) + within));
  typedef short v8i16_t __attribute__((ext_vector_type(8)));
  const v8i16_t r = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, r);
}

// Work split: the first F = ntiles / P * P tiles run whole, in F rounds of P
// workgroups (P = the compute units); each of the T < P remaining tiles is cut
// into m pieces of consecutive 32-token stages, piece i of tile j being
// workgroup F P + i T + j, with m chosen so that the T m pieces fill whole rounds
// of P well. A whole tile is added to H at once; piece i T + j goes to slot
// i T + j of the workspace, in the accumulators' register order, and
// syrk_rect_fix_kernel adds the m pieces of each tile in order of i. Workgroups
// are numbered XCD-major (each XCD's concurrent workgroups take consecutive
// tiles, or consecutive tiles' pieces of the same stages).
struct RectSplit {
  int F, T, m;    // whole tiles, tiles cut in pieces, pieces per cut tile
  int nk;         // 32-token stages per tile
  int per_xcd;    // workgroups per XCD in the whole-tile and the piece parts
  int pper_xcd;
  int overwrite;  // H = 2 X^T X (every lower entry is written) instead of H +=
};
constexpr int kRTileElems = kRR * kRC;  // one slot: 98304 floats

__global__ __launch_bounds__(kDThreads, 1) void syrk_rect_kernel(
    float* __restrict__ H, const unsigned short* __restrict__ X, int64_t t, int64_t b, int64_t ldx,
    int nstrips, RectSplit sp, float* __restrict__ part) {
  const int wg = blockIdx.x;
  const int nk = sp.nk;
  int lin, s0 = 0, s1 = nk, slot = -1;
  if (wg < 8 * sp.per_xcd) {
    lin = (wg % 8) * sp.per_xcd + wg / 8;
    if (lin >= sp.F) return;
  } else {
    const int w = wg - 8 * sp.per_xcd;
    const int p = (w % 8) * sp.pper_xcd + w / 8;  // piece i T + j
    if (p >= sp.T * sp.m) return;
    const int i = p / sp.T, j = p % sp.T;
    lin = sp.F + j;
    s0 = (int)((int64_t)i * nk / sp.m);
    s1 = (int)((int64_t)(i + 1) * nk / sp.m);
    slot = p;
  }
  int ti, tj;
  rect_tile_of(lin, nstrips, b, ti, tj);
  const int64_t I0 = (int64_t)ti * kRR, J0 = (int64_t)tj * kRC;
  // the first piece of a cut tile records the tile for the fix-up kernel
  if (slot >= 0 && slot < sp.T && threadIdx.x == 0)
    reinterpret_cast<int*>(part + (int64_t)sp.T * sp.m * kRTileElems)[slot] = (ti << 16) | tj;

  __shared__ __attribute__((aligned(1024))) unsigned char sm0[kRStageBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char sm1[kRStageBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char sm2[kRStageBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char sm3[kRStageBytes];
  auto buf = [&](auto S) -> unsigned char* {
    constexpr int s = decltype(S)::value;
    if constexpr (s == 0) return sm0;
    else if constexpr (s == 1) return sm1;
    else if constexpr (s == 2) return sm2;
    else return sm3;
  };
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wrow = wave >> 1, wcol = wave & 1;
  const int lr = lane & 31, lk = lane >> 5;

  // Loader: chunk q (0..39) of a stage is sub-panel q/8, token rows 4(q%8) ..
  // 4(q%8)+3, at LDS offset 1024 q; wave w loads q = w + 4m, m = 2k + o
  // (k = 0..4, o = 0, 1): sub-panel k, token rows 4w + 16o + 0..3. Lane l writes
  // bytes [16 l, 16 l + 16) of its chunk: token row 4w + 16o + l/16, LDS piece
  // l%16, which holds the feature piece (l%16) ^ 4(row & 3) (row & 3 = (l/16) & 3
  // for both o). The per-lane offset vo[k] is that of o = 0; o = 1 is 16 token
  // rows further, a uniform step taken in the second base address.
  unsigned vo[5];
  {
    const int tr = 4 * wave + (lane >> 4);
    const int fg = (lane & 15) ^ ((tr & 3) << 2);
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      int64_t f = (k < 3 ? I0 + k * kRSub : J0 + (k - 3) * kRSub) + fg * 8;
      f = f < b ? f : 0;  // features past b only feed outputs that are never stored
      vo[k] = (unsigned)(((int64_t)tr * ldx + f) * 2);
    }
  }
  // t is a multiple of 32 (the caller adds the remaining tokens separately).
  // Stages past the piece are loaded too (at most three, never read) so that every
  // stage has the same number of loads for the vmcnt waits; past the end of the
  // tokens they re-read the last stage.
  auto issue_stage = [&](int st, unsigned char* sbase) {
    const int64_t tok0 = (int64_t)st * kDBK;
    const int64_t br = tok0 < t - kDBK ? tok0 : t - kDBK;
    lds_dma10s(vo, X + br * ldx, X + (br + 16) * ldx, sbase + wave * 1024);
  };

  f32x16_t acc[6][4];
#pragma unroll
  for (int a = 0; a < 6; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][c][r] = 0.f;

  bf16x8_t af0[6], bf0[4], af1[6], bf1[4];
  auto read_frags = [&](const unsigned char* sb, int ks, bf16x8_t (&af)[6], bf16x8_t (&bf)[4]) {
#pragma unroll
    for (int a = 0; a < 6; ++a) {
      const int fa = wrow * 192 + a * 32;
      af[a] = rtr_frag(sb + (fa >> 7) * kRSubBytes, fa & 127, ks * 16, lane);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
      bf[c] = rtr_frag(sb + (3 + wcol) * kRSubBytes, c * 32, ks * 16, lane);
  };
  // 256 accumulator registers are AGPRs: the compiler places the results of the
  // MFMA builtin there. The other 128 (rows a = 4, 5) are kept in VGPRs through
  // the VGPR form of the instruction written out (operands and accumulators as
  // "v"); their results are read only after the loop, behind explicit wait states.
  auto mfmas = [&](const bf16x8_t (&af)[6], const bf16x8_t (&bf)[4]) {
#pragma unroll
    for (int a = 0; a < 6; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (a < 4) {
          acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bf[c], acc[a][c], 0, 0, 0);
        } else {
          __asm__ volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                           : "+v"(acc[a][c])
                           : "v"(af[a]), "v"(bf[c]));
        }
      }
  };

  const int n = s1 - s0;
  issue_stage(s0, sm0);
  issue_stage(s0 + 1, sm1);
  issue_stage(s0 + 2, sm2);
  __asm__ volatile("s_waitcnt vmcnt(20)" ::: "memory");
  __syncthreads();
  read_frags(sm0, 0, af0, bf0);
  for (int l0 = 0; l0 < n; l0 += kRStages) {
    static_for<0, kRStages>([&](auto U) __attribute__((always_inline)) {
      constexpr int u = U;
      const int l = l0 + u;
      if (l < n) {
        issue_stage(s0 + l + 3, buf(std::integral_constant<int, (u + 3) % kRStages>{}));
        read_frags(buf(std::integral_constant<int, u>{}), 1, af1, bf1);
        mfmas(af0, bf0);
        __asm__ volatile("s_waitcnt vmcnt(20)" ::: "memory");
        unsigned char* nb = buf(std::integral_constant<int, (u + 1) % kRStages>{});
        __syncthreads();
        read_frags(nb, 0, af0, bf0);
        mfmas(af1, bf1);
      }
    });
  }
  // wait states between the last written-out MFMA and the first read of its result
  __asm__ volatile("s_waitcnt vmcnt(0)\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

  if (slot < 0) {
#pragma unroll
    for (int a = 0; a < 6; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = I0 + wrow * 192 + a * 32 + 8 * (r >> 2) + 4 * lk + (r & 3);
          const int64_t col = J0 + wcol * 128 + c * 32 + lr;
          if (row < b && col < b && col <= row)
            H[row * b + col] = 2.0f * acc[a][c][r] + (sp.overwrite ? 0.f : H[row * b + col]);
        }
  } else {
    float* dst = part + (int64_t)slot * kRTileElems;
#pragma unroll
    for (int a = 0; a < 6; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          dst[((wave * 6 + a) * 4 + c) * 1024 + r * 64 + lane] = acc[a][c][r];
  }
}

// H += 2 (sum of the m pieces in order) for each cut tile. Block (g, j): tile F + j,
// accumulator group g = (wave * 6 + a) * 4 + c (1024 floats, r * 64 + lane); each
// thread takes four consecutive lanes: four consecutive columns of one row.
__global__ __launch_bounds__(256) void syrk_rect_fix_kernel(float* __restrict__ H,
                                                            const float* __restrict__ part,
                                                            int64_t b, RectSplit sp) {
  const int j = blockIdx.y, g = blockIdx.x;
  // tile F + j, as its first piece recorded it (slot j's entry after the slots)
  const int tij = reinterpret_cast<const int*>(part + (int64_t)sp.T * sp.m * kRTileElems)[j];
  const int64_t I0 = (int64_t)(tij >> 16) * kRR, J0 = (int64_t)(tij & 0xffff) * kRC;
  const int wave = g / 24, a = (g / 4) % 6, c = g % 4;
  const int wrow = wave >> 1, wcol = wave & 1;
  const int e = threadIdx.x * 4;
  const int r = e >> 6, lane = e & 63;
  f32x4_t s = {0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < sp.m; ++i)
    s += *(const f32x4_t*)(part + ((int64_t)i * sp.T + j) * kRTileElems + g * 1024 + e);
  const int64_t row = I0 + wrow * 192 + a * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
  const int64_t col = J0 + wcol * 128 + c * 32 + (lane & 31);  // a multiple of 4; b % 8 == 0
  if (row >= b || col >= b || col > row) return;
  float* h = H + row * b + col;
  if (col + 3 <= row && ((uintptr_t)h & 15) == 0) {
    f32x4_t v = 2.0f * s;
    if (!sp.overwrite) v += *(const f32x4_t*)h;
    *(f32x4_t*)h = v;
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (col + q <= row) h[q] = 2.0f * s[q] + (sp.overwrite ? 0.f : h[q]);
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
// 64 x 64 tiles through LDS, 16-byte global accesses when b % 4 == 0.
__global__ __launch_bounds__(256) void flip_lower_kernel(const float* __restrict__ H,
                                                         float* __restrict__ S, int64_t b,
                                                         const DevState* st, int add_lambda) {
  __shared__ float tile[64][65];  // tile[r][c] = H[b-1-(J0+r)][b-1-(I0+c)]
  const int64_t I0 = (int64_t)blockIdx.y * 64, J0 = (int64_t)blockIdx.x * 64;
  if (J0 > I0) return;
  const int tid = threadIdx.x;
  const bool vec = (b & 3) == 0 && I0 + 64 <= b && J0 + 64 <= b;
  if (vec) {
    // row r: H columns b-I0-64 .. b-I0-1 as 16 float4; thread: row tid/16 + 16p, piece tid%16
    const int v = tid & 15;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = (tid >> 4) + 16 * p;
      const f32x4_t x = *(const f32x4_t*)(H + (b - 1 - (J0 + r)) * b + (b - I0 - 64) + 4 * v);
#pragma unroll
      for (int q = 0; q < 4; ++q) tile[r][63 - 4 * v - q] = x[q];
    }
  } else {
    for (int e = tid; e < 64 * 64; e += 256) {
      const int r = e >> 6, c = e & 63;
      const int64_t hr = b - 1 - (J0 + r), hc = b - 1 - (I0 + c);
      tile[r][c] = (hr >= 0 && hc >= 0) ? H[hr * b + hc] : 0.f;
    }
  }
  __syncthreads();
  const float lam = add_lambda ? (float)st->lambda : 0.f;
  // output row i = I0 + c, columns j = J0 + 4w .. +3 (tile[4w + q][c])
  const int w = tid & 15;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int c = (tid >> 4) + 16 * p;
    const int64_t i = I0 + c, j = J0 + 4 * w;
    if (i >= b) continue;
    f32x4_t y;
#pragma unroll
    for (int q = 0; q < 4; ++q) y[q] = tile[4 * w + q][c] + ((j + q == i) ? lam : 0.f);
    float* dst = S + i * b + j;
    if (vec && j + 3 <= i) {
      *(f32x4_t*)dst = y;
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (j + q < b && j + q <= i) dst[q] = y[q];
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

namespace {

// compute units of the current device (the persistent grid of the rectangles)
int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) {
    (void)hipGetLastError();
    return 256;
  }
  return n;
}

int64_t rect_tiles(int64_t b) {
  const int nstrips = (int)cdiv(b, kRR);
  int64_t n = 0;
  for (int r = 0; r < nstrips; ++r) n += rect_cols(r, b);
  return n;
}

// The rectangles pay when every workgroup gets at least 64 stages (2048 tokens).
bool rect_applies(int64_t t, int64_t b, int P) {
  return t >= kDBK && rect_tiles(b) * (t / kDBK) >= (int64_t)64 * P;
}

// Whole tiles in complete rounds of P, the rest cut into m pieces each (m = 0 when
// nothing is cut): m minimises the rounds the pieces take, in tiles' time, among
// 1..min(nk / 32, 4P / T) (pieces of at least 32 stages, at most 4P slots); m = 1
// runs those tiles whole as well. m_force > 0 fixes m (1 <= m_force <= nk).
RectSplit rect_split(int64_t ntiles, int nk, int P, int m_force) {
  RectSplit sp;
  sp.nk = nk;
  sp.F = (int)(ntiles / P * P);
  sp.T = (int)(ntiles - sp.F);
  sp.m = 0;
  if (sp.T > 0) {
    if (m_force > 0) {
      sp.m = m_force;
    } else {
      int mmax = nk / 32;
      if (mmax > 4 * P / sp.T) mmax = 4 * P / sp.T;
      double best = 1.0;  // m = 1: one more round of whole tiles
      sp.m = 1;
      for (int m = 2; m <= mmax; ++m) {
        const double cost = (double)cdiv((int64_t)sp.T * m, P) / m;
        if (cost < best - 1e-9) {
          best = cost;
          sp.m = m;
        }
      }
    }
    if (sp.m == 1) {
      sp.F = (int)ntiles;
      sp.T = 0;
      sp.m = 0;
    }
  }
  sp.per_xcd = (int)cdiv(sp.F, 8);
  sp.pper_xcd = (int)cdiv((int64_t)sp.T * sp.m, 8);
  sp.overwrite = 0;
  return sp;
}

// the pieces' slots, then one int per cut tile (its coordinates, for the fix-up)
size_t rect_workspace_floats(const RectSplit& sp) {
  return sp.T > 0 ? (size_t)sp.T * sp.m * kRTileElems + sp.T : 0;
}

}  // namespace

size_t syrk_bf16_workspace_floats(int64_t t, int64_t b) {
  const int splits = syrk_bf16_splits(t, b);
  const int64_t nt = cdiv(b, kTile);
  // the square tiles' token splits (also taken when ldx rules out the rectangles)
  const size_t sq = splits > 1 ? (size_t)splits * (size_t)(nt * (nt + 1) / 2) * kTile * kTile : 0;
  const int P = device_cus();
  if (!rect_applies(t, b, P)) return sq;
  const size_t r = rect_workspace_floats(rect_split(rect_tiles(b), (int)(t / kDBK), P, 0));
  return r > sq ? r : sq;
}

size_t syrk_rect_workspace_floats(int64_t t, int64_t b, int P, int m) {
  if (t < kDBK) return 0;
  return rect_workspace_floats(rect_split(rect_tiles(b), (int)(t / kDBK), P, m));
}

hipError_t launch_syrk_rect(float* H, const unsigned short* X, int64_t t, int64_t b, int64_t ldx,
                            float* part, int P, int m, hipStream_t s, bool overwrite) {
  const int64_t tf = t / kDBK * kDBK;  // whole stages; the rest goes to the square tiles
  if (tf > 0) {
    const int nstrips = (int)cdiv(b, kRR);
    RectSplit sp = rect_split(rect_tiles(b), (int)(tf / kDBK), P, m);
    sp.overwrite = overwrite ? 1 : 0;
    const int grid = 8 * (sp.per_xcd + sp.pper_xcd);
    hipLaunchKernelGGL(syrk_rect_kernel, dim3(grid), dim3(kDThreads), 0, s, H, X, tf, b, ldx,
                       nstrips, sp, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (sp.T > 0) {
      // 96 groups of 1024 floats per tile, four per thread
      hipLaunchKernelGGL(syrk_rect_fix_kernel, dim3(96, sp.T), dim3(256), 0, s, H, part, b, sp);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (tf == t) return hipSuccess;
  return launch_syrk_bf16(H, X + tf * ldx, t - tf, b, ldx, nullptr, 1, s);
}

namespace {
// the rectangles are taken with a workspace, when the work is large enough and
// the per-lane load offsets of 32 token rows stay below 2^31 bytes
bool rect_taken(int64_t t, int64_t b, int64_t ldx, const float* partials, int P) {
  return partials != nullptr && (int64_t)64 * ldx < ((int64_t)1 << 31) && rect_applies(t, b, P);
}
}  // namespace

hipError_t launch_syrk_bf16_set(float* H, const unsigned short* X, int64_t t, int64_t b,
                                int64_t ldx, float* partials, int splits, hipStream_t s) {
  const int P = device_cus();
  if (t > 0 && b > 0 && rect_taken(t, b, ldx, partials, P))
    return launch_syrk_rect(H, X, t, b, ldx, partials, P, 0, s, true);
  const hipError_t e = launch_zero(H, (size_t)b * b * sizeof(float), s);
  if (e != hipSuccess) return e;
  return launch_syrk_bf16(H, X, t, b, ldx, partials, splits, s);
}

hipError_t launch_syrk_bf16(float* H, const unsigned short* X, int64_t t, int64_t b, int64_t ldx,
                            float* partials, int splits, hipStream_t s) {
  if (t <= 0 || b <= 0) return hipSuccess;
  {
    const int P = device_cus();
    if (rect_taken(t, b, ldx, partials, P)) return launch_syrk_rect(H, X, t, b, ldx, partials, P, 0, s, false);
  }
  const int nt = (int)cdiv(b, kTile);
  const int ntiles = nt * (nt + 1) / 2;
  const int per_xcd = (int)cdiv(ntiles, 8);
  if (partials == nullptr) splits = 1;
  int64_t tps = cdiv(cdiv(t, splits), kBK) * kBK;
  splits = (int)cdiv(t, tps);
  dim3 grid(per_xcd * 8, splits);
  hipLaunchKernelGGL(syrk_bf16_kernel, grid, dim3(kDThreads), 0, s, H, X, t, b, ldx, nt, ntiles,
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
  const int nt = (int)cdiv(b, 64);
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
