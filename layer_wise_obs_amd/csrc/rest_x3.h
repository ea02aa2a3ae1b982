// The bulk of a pair's trailing update in the factorisation sweep, on pre-split
// operands.
//
// For a pair of steps (k, k+1) every tile (i, j) of the rest set (block rows
// i >= k+4, j <= i, j not in {k+2, k+3}; see factor.hip) is updated as
//   S[i, j] -= sum_{kk < 256} Y[kk, i] Y[kk, j]        (C from zero for j in {k, k+1}),
// where Y (256 x b) is the pair's panel laid out k-major: Y[:, i] = [Lp_i(k);
// Lp_i(k+1)] for block columns i >= k+2, and Y[:, j] = rows k, k+1 of S (the final
// rows of L^-1, and [X_kk; S(k+1,k)], [0; X_{k+1,k+1}] for j = k, k+1) otherwise.
// The update is thus a symmetric rank-256 product of Y with itself, like the
// Hessian's syrk.
//
// Y arrives split into three bf16 planes (y = h + m + l, each part rounded to
// nearest even, |y - h - m - l| <= 2^-24 |y|; built once per pair by
// ybuild_kernel), so the tiles run the syrk's pipeline without converting
// anything: 256 x 256 output tiles on four waves of 128 x 128 (accumulators in
// AGPRs), k-major planes copied into LDS by direct global->LDS loads (16-byte
// pieces XOR-swizzled by k & 3), MFMA operands formed by ds_read_b64_tr_b16, and
// six v_mfma_f32_32x32x16_bf16 per block and 16 k (h h, h m, m h, m m, h l, l h,
// accumulated smallest first: the products of weight >= 2^-16, errors of the
// order of fp32 accumulation). Three LDS stages of 16 k rows (48 KB each).
#pragma once

#include "x3_pipe.h"

namespace th {

// Rest set of pair (k, k+1): tiles of 256 x 256 over block-row pairs pi >= (k+4)/2
// and block-column pairs pj <= pi, pj != (k+2)/2 (row-major), one persistent
// workgroup per slot. Y: three planes [3][256][ldy] of bf16 bits. Only 128-blocks
// on or below the block diagonal and inside b are stored.
__global__ __launch_bounds__(256, 1) void rest_x3_kernel(float* __restrict__ S, int64_t b, int k,
                                                          const unsigned short* __restrict__ Y,
                                                          int64_t ldy, int64_t ntiles) {
  __shared__ __attribute__((aligned(1024))) unsigned char sm0[kX3StageBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char sm1[kX3StageBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char sm2[kX3StageBytes];
  auto buf = [&](auto U) -> unsigned char* {
    constexpr int u = decltype(U)::value;
    if constexpr (u == 0) return sm0;
    else if constexpr (u == 1) return sm1;
    else return sm2;
  };
  // the wave index through readfirstlane: everything derived from it (tile
  // corners, buffer resources) is then known to be uniform and stays in SGPRs
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wrow = wave >> 1, wcol = wave & 1;
  const int lr = lane & 31, lk = lane >> 5;
  const int pr0 = (k + 4) / 2, pskip = (k + 2) / 2, pzero = k / 2;
  const int64_t pstride = (int64_t)kX3Rows * ldy;
  constexpr int nst = kX3Rows / kX3StageK;  // 16 stages per tile

  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    int64_t rem = t;
    int pi = pr0;
    while (rem >= pi) { rem -= pi; ++pi; }
    const int pj = (int)rem < pskip ? (int)rem : (int)rem + 1;
    const int64_t row0 = (int64_t)pi * kX3Tile, col0 = (int64_t)pj * kX3Tile;

    // chunk m of this wave: c = wave + 4 m; plane c / 16, operand (c / 8) % 2
    // (0: rows of the tile, 1: columns), k-row pair c % 8 of the stage. Byte
    // offsets from the stage's first k row (fixed for the tile; at most 3 planes
    // of 256 rows of b elements, far below 4 GB).
    unsigned vo[12];
#pragma unroll
    for (int m = 0; m < 12; ++m) {
      const int c = wave + 4 * m;
      const int p = c >> 4, o = (c >> 3) & 1, r = c & 7;
      const int tr = 2 * r + lk;  // k row inside the stage
      const int fg = lr ^ ((tr & 3) << 2);
      vo[m] = (unsigned)((p * pstride + (int64_t)tr * ldy + (o ? col0 : row0) + fg * 8) * 2);
    }
    auto issue = [&](int st, unsigned char* sbase) {
      x3d::dma12s(vo, Y + (int64_t)st * kX3StageK * ldy, sbase + wave * 1024);
    };

    f32x16_t acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[a][c][r] = 0.f;

    // Per block the six products accumulate smallest first (l h, h l, m m, m h,
    // h m, h h). A stage's 24 operand fragments (three planes of the row and the
    // column panels) are read into one of two register sets while the previous
    // stage's products run: the barrier that releases stage it+1 sits before the
    // last 16 products of stage it, and stage it+1's reads go out behind it.
    struct Frags {
      bf16x8_t ah[4], bh[4], al[4], bl[4], am[4], bm[4];
    };
    auto read_frags = [&](const unsigned char* sb, Frags& F) {
      // panel (plane p, operand o) at sb + (2 p + o) * kX3PanelBytes
      auto fa = [&](int p, int a) { return x3d::frag(sb + (2 * p) * kX3PanelBytes, wrow * 128 + a * 32, lane); };
      auto fbf = [&](int p, int c) { return x3d::frag(sb + (2 * p + 1) * kX3PanelBytes, wcol * 128 + c * 32, lane); };
#pragma unroll
      for (int a = 0; a < 4; ++a) { F.ah[a] = fa(0, a); F.al[a] = fa(2, a); F.am[a] = fa(1, a); }
#pragma unroll
      for (int c = 0; c < 4; ++c) { F.bh[c] = fbf(0, c); F.bl[c] = fbf(2, c); F.bm[c] = fbf(1, c); }
    };
    auto products_12 = [&](const Frags& F) {  // l h, h l, m m, m h, h m
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F.al[a], F.bh[c], acc[a][c], 0, 0, 0);
          acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F.ah[a], F.bl[c], acc[a][c], 0, 0, 0);
        }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F.am[a], F.bm[c], acc[a][c], 0, 0, 0);
          acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F.am[a], F.bh[c], acc[a][c], 0, 0, 0);
          acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F.ah[a], F.bm[c], acc[a][c], 0, 0, 0);
        }
    };
    auto products_3 = [&](const Frags& F) {  // h h
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F.ah[a], F.bh[c], acc[a][c], 0, 0, 0);
    };

    __syncthreads();  // the previous tile's last reads are done before its buffers refill
    issue(0, sm0);
    issue(1, sm1);
    issue(2, sm2);
    __asm__ volatile("s_waitcnt vmcnt(24)" ::: "memory");  // stage 0 (this wave's part)
    __syncthreads();
    Frags F0, F1;
    read_frags(sm0, F0);
    // Unrolled by 6 (two register sets, three buffers) so that every index is a
    // constant. Stage s lives in buffer s % 3.
    for (int it0 = 0; it0 < nst; it0 += 6) {
      static_for<0, 6>([&](auto U) __attribute__((always_inline)) {
        constexpr int u = U;
        const int it = it0 + u;
        if (it < nst) {
          Frags& cur = (u % 2 == 0) ? F0 : F1;
          Frags& nxt = (u % 2 == 0) ? F1 : F0;
          products_12(cur);
          // keep those products (and the last use of the l and m fragments) above
          // the barrier, so that the next stage's fragments can take their registers
          __builtin_amdgcn_sched_barrier(0);
          if (it + 1 < nst) {
            // stage it+1 complete for this wave (stage it+2's twelve loads may be in
            // flight); after the barrier it is complete for all, and every wave's
            // reads of stage it (done before its products above) are over
            if (it + 2 < nst) __asm__ volatile("s_waitcnt vmcnt(12)" ::: "memory");
            else __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (it + 3 < nst) issue(it + 3, buf(std::integral_constant<int, u % kX3Stages>{}));
            read_frags(buf(std::integral_constant<int, (u + 1) % kX3Stages>{}), nxt);
          }
          products_3(cur);
        }
      });
    }

    // S = C - acc (C = 0 for block columns k, k+1): read-modify-write in four
    // groups of 64 values per lane (one row of 32 x 32 blocks each), the loads of
    // group a+1 in flight while group a is stored. Buffer accesses: one resource
    // per group starting at its first row (so a group's 32 rows need 32-bit
    // offsets only, whatever b), rows past b fall outside the resource (loads give
    // 0, stores are dropped), columns past b get an offset outside it. Whether a
    // 32 x 32 block lies on or below the block diagonal is uniform per wave.
    const bool from_zero = pj == pzero;
    const int64_t wr0 = row0 + wrow * 128, wc0 = col0 + wcol * 128;
    auto rsrc_of = [&](int a) {
      const int64_t rb = wr0 + a * 32;
      const int64_t left = (rb < b ? b - rb : 0) * b * 4;  // bytes from the group's first row
      const int nrec = (int)(left < 0x7fffffff ? left : 0x7fffffff);
      return __builtin_amdgcn_make_buffer_rsrc(S + (rb < b ? rb : 0) * b, 0, nrec, 0x00020000);
    };
    auto voff = [&](int c) {  // this lane's column in block c, row offset 4 lk
      const int64_t col = wc0 + c * 32 + lr;
      return col < b ? (int)((4 * lk * b + col) * 4) : 0x7fffffff;
    };
    // row 8 (r/4) + (r%4) of the lane's block rows: its offset goes into the
    // per-lane offset, which the range check covers (the scalar offset of a buffer
    // access is added to the address outside that check); an out-of-range column's
    // marker stays at or above 2^31 - 1, past every record count
    auto row_off = [&](int vo, int r) {
      return (int)((unsigned)vo + (unsigned)((8 * (r >> 2) + (r & 3)) * b * 4));
    };
    auto on = [&](int a, int c) { return ((wc0 + c * 32) >> 7) <= ((wr0 + a * 32) >> 7); };
    auto load_group = [&](int a, float (&v)[64]) {
      const auto rs = rsrc_of(a);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int vo = voff(c);
        const bool use = !from_zero && on(a, c);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          v[c * 16 + r] = use ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                    rs, row_off(vo, r), 0, 0))
                              : 0.f;
      }
    };
    float cur[64], nxt[64];
    load_group(0, cur);
    static_for<0, 4>([&](auto A) __attribute__((always_inline)) {
      constexpr int a = A;
      if constexpr (a + 1 < 4) load_group(a + 1, nxt);
      const auto rs = rsrc_of(a);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (!on(a, c)) continue;
        const int vo = voff(c);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          __builtin_amdgcn_raw_buffer_store_b32(
              __builtin_bit_cast(unsigned, cur[c * 16 + r] - acc[a][c][r]), rs,
              row_off(vo, r), 0, 0);
      }
      if constexpr (a + 1 < 4) {
#pragma unroll
        for (int e = 0; e < 64; ++e) cur[e] = nxt[e];
      }
    });
  }
}

// Y for pair (k, k+1), split into three bf16 planes. One workgroup per 64 columns x
// 64 k rows: columns of block >= k+2 come from the panel buffer P (row i, pitch
// 256: Y[kk][i] = P[i][kk], transposed through LDS), the others from rows k and
// k+1 of S (Y[kk][j] = S[128 k + kk][j], with the upper block (k, k+1) read as 0);
// columns past b are 0.
__global__ __launch_bounds__(256) void ybuild_kernel(const float* __restrict__ S, int64_t b, int k,
                                                     const float* __restrict__ P,
                                                     unsigned short* __restrict__ Y, int64_t ldy) {
  __shared__ float tile[64][65];
  const int tid = threadIdx.x;
  const int64_t c0 = (int64_t)blockIdx.x * 64;  // column
  const int k0 = blockIdx.y * 64;               // k row
  const int jb = (int)(c0 >> 7);
  const int64_t pstride = (int64_t)kX3Rows * ldy;
  if (c0 < b && jb >= k + 2) {
    // P[c0 + ci][k0 + kk], coalesced along kk
    for (int e = tid; e < 64 * 64; e += 256) {
      const int ci = e >> 6, kk = e & 63;
      const int64_t col = c0 + ci;
      tile[kk][ci] = col < b ? P[col * (2 * 128) + k0 + kk] : 0.f;
    }
  } else {
    for (int e = tid; e < 64 * 64; e += 256) {
      const int kk = e >> 6, ci = e & 63;
      const int64_t col = c0 + ci;
      const int krow = k0 + kk;
      float v = 0.f;
      if (col < b && !(krow < 128 && jb == k + 1)) v = S[((int64_t)k * 128 + krow) * b + col];
      tile[kk][ci] = v;
    }
  }
  __syncthreads();
  // each thread: one k row, 16 consecutive columns, split into the three planes
  const int kk = tid >> 2, cq = (tid & 3) * 16;
  unsigned short h[16], m[16], l[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float x = tile[kk][cq + e];
    const unsigned short xh = f32_to_bf16_rne(x);
    const float r1 = x - bf16_to_f32(xh);
    const unsigned short xm = f32_to_bf16_rne(r1);
    const float r2 = r1 - bf16_to_f32(xm);
    h[e] = xh; m[e] = xm; l[e] = f32_to_bf16_rne(r2);
  }
  const int64_t off = (int64_t)(k0 + kk) * ldy + c0 + cq;
  unsigned short* planes[3] = {Y + off, Y + pstride + off, Y + 2 * pstride + off};
  const unsigned short* vals[3] = {h, m, l};
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    u32x4_t w0, w1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      w0[q] = (unsigned)vals[p][2 * q] | ((unsigned)vals[p][2 * q + 1] << 16);
      w1[q] = (unsigned)vals[p][8 + 2 * q] | ((unsigned)vals[p][8 + 2 * q + 1] << 16);
    }
    *(u32x4_t*)(planes[p]) = w0;
    *(u32x4_t*)(planes[p] + 8) = w1;
  }
}

}  // namespace th
