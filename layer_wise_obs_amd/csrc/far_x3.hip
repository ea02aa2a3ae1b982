// Far-column updates of the N:M block loop on pre-split operands.
//
// "Pruning LLMs with Thanos", section "Contribution one: solve a selected set
// directly": every block's compensation reaches all still-active columns,
// W[:, F] -= Z [A_F]_{J,F}. The block loop applies the part for the columns past
// each group of eight blocks once per group, with K = 8B: W[:, s1:b] -= Z R with Z
// the group's coefficients (c x 8B) and R = [A_F]_{J,F} for the group's rows and
// the far columns. That product runs here like the factorisation's rest sets:
// far_build_kernel splits both operands once into three bf16 planes in one k-major
// buffer Y -- columns 0 .. ldA-1 hold Z^T (one per row of W), columns ldA .. hold R
// -- and far_x3_kernel runs 256 x 256 tiles of W on the direct global->LDS
// pipeline of x3_pipe.h with the six products per block, then writes W - acc.
// A tile takes about as long whatever the number of tiles beside it, so a launch
// costs whole rounds of one workgroup per compute unit. The tiles of a last,
// partial round are therefore cut into m pieces of consecutive k stages that
// fill one round: each piece writes its sums to a slot, and far_fix_kernel
// subtracts a tile's m slots from W in a fixed order (deterministic).
#include "x3_pipe.h"

namespace th {

namespace {


// Y (three planes of kp k rows x ldy columns): column i < ldA is row i of Z
// (Y[kk][i] = Z[i][kk], transposed through LDS), column ldA + j is column col0 + j
// of R's rows r0 .. r0+K-1; zero past c, past ncols and past K. One workgroup per
// 64 columns x 64 k rows, each thread splitting 16 consecutive columns of one k row.
__global__ __launch_bounds__(256) void far_build_kernel(const float* __restrict__ Z, int64_t ldz,
                                                        int64_t nrows, const float* __restrict__ R,
                                                        int64_t r0, int64_t b, int64_t col0,
                                                        int64_t ncols, int K,
                                                        unsigned short* __restrict__ Y,
                                                        int64_t ldy, int64_t ldA, int64_t kp) {
  __shared__ float tile[64][65];
  const int tid = threadIdx.x;
  const int64_t y0 = (int64_t)blockIdx.x * 64;  // Y column
  const int k0 = blockIdx.y * 64;               // k row
  if (y0 < ldA) {
    // Z[y0 + ci][k0 + kk], coalesced along kk
    for (int e = tid; e < 64 * 64; e += 256) {
      const int ci = e >> 6, kk = e & 63;
      const int64_t row = y0 + ci;
      tile[kk][ci] = (row < nrows && k0 + kk < K) ? Z[row * ldz + k0 + kk] : 0.f;
    }
  } else {
    for (int e = tid; e < 64 * 64; e += 256) {
      const int kk = e >> 6, ci = e & 63;
      const int64_t j = y0 - ldA + ci;
      tile[kk][ci] = (j < ncols && k0 + kk < K) ? R[(r0 + k0 + kk) * b + col0 + j] : 0.f;
    }
  }
  __syncthreads();
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
  const int64_t pstride = kp * ldy;
  const int64_t off = (int64_t)(k0 + kk) * ldy + y0 + cq;
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

// Work split of one far-column product: tiles 0 .. nwhole-1 run whole (workgroup
// w of that launch: tile (w % 8) per_xcd + w / 8, so an XCD's workgroups take
// consecutive tiles), tiles nwhole .. ntiles-1 in m pieces each (workgroup p of the
// pieces' launch: piece p % m of tile nwhole + p / m, stages [i nst / m, (i+1) nst / m)).
struct FarSplit {
  int nst, nti, ntiles, nwhole, per_xcd, m;
};

// Slot layout of a piece: float4 number (((a * 4 + cc) * 4 + r / 4) * 256 + thread)
// holds accumulator values r .. r+3 of block (a, cc) of that thread.
constexpr int kFarSlotFloats = kX3Tile * kX3Tile;

// W[0:nrows, col0:col0+ncols] -= Y[:, 0:nrows]^T Y[:, ldA:ldA+ncols] over 16-row k
// stages; tile lin -> (lin % nti, lin / nti). One workgroup per whole tile, or (PIECES)
// per piece, which writes its slot instead of W.
template <bool PIECES>
__global__ __launch_bounds__(256, 1) void far_x3_kernel(float* __restrict__ W, int64_t nrows, int64_t b,
                                                         int64_t col0, int64_t ncols,
                                                         const unsigned short* __restrict__ Y,
                                                         int64_t ldy, int64_t ldA, int64_t kp,
                                                         FarSplit sp, float* __restrict__ slots) {
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
  const int64_t pstride = kp * ldy;
  const int wg = blockIdx.x;
  int lin, st0, nst;
  if (!PIECES) {
    lin = (wg % 8) * sp.per_xcd + wg / 8;
    if (lin >= sp.nwhole) return;
    st0 = 0;
    nst = sp.nst;
  } else {
    const int piece = wg;
    lin = sp.nwhole + piece / sp.m;
    const int i = piece % sp.m;
    st0 = i * sp.nst / sp.m;
    nst = (i + 1) * sp.nst / sp.m - st0;  // at least 3 (the host's choice of m)
  }
  {
    // tiles column-major: the concurrent tiles of an XCD share column panels
    const int ti = lin % sp.nti, tj = lin / sp.nti;
    const int64_t row0 = (int64_t)ti * kX3Tile, ycol0 = ldA + (int64_t)tj * kX3Tile;

    // chunk m of this wave: c = wave + 4 m; plane c / 16, operand (c / 8) % 2
    // (0: rows of the tile, 1: columns), k-row pair c % 8 of the stage. Byte
    // offsets from the stage's first k row (fixed for the tile; three planes of kp
    // rows of ldy elements, below 2^31 bytes).
    unsigned vo[12];
#pragma unroll
    for (int m = 0; m < 12; ++m) {
      const int c = wave + 4 * m;
      const int p = c >> 4, o = (c >> 3) & 1, r = c & 7;
      const int tr = 2 * r + lk;  // k row inside the stage
      const int fg = lr ^ ((tr & 3) << 2);
      vo[m] = (unsigned)((p * pstride + (int64_t)tr * ldy + (o ? ycol0 : row0) + fg * 8) * 2);
    }
    auto issue = [&](int st, unsigned char* sbase) {
      x3d::dma12s(vo, Y + (int64_t)(st0 + st) * kX3StageK * ldy, sbase + wave * 1024);
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

    if constexpr (PIECES) {
      float4* slot = (float4*)(slots + (int64_t)wg * kFarSlotFloats);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq)
            slot[((a * 4 + cc) * 4 + rq) * 256 + tid] =
                make_float4(acc[a][cc][4 * rq], acc[a][cc][4 * rq + 1], acc[a][cc][4 * rq + 2],
                            acc[a][cc][4 * rq + 3]);
    } else {

    // W = W - acc: read-modify-write in four groups of 64 values per lane (one row
    // of 32 x 32 blocks each), the loads of group a+1 in flight while group a is
    // stored. One buffer resource per group starting at its first row: rows past c
    // fall outside it (loads give 0, stores are dropped), columns past the range
    // get an offset outside it.
    const int64_t wr0 = row0 + wrow * 128;
    const int64_t wc_rel = (int64_t)tj * kX3Tile + wcol * 128;  // from col0
    auto rsrc_of = [&](int a) {
      const int64_t rb = wr0 + a * 32;
      const int64_t left = (rb < nrows ? nrows - rb : 0) * b * 4;  // bytes from the group's first row
      const int nrec = (int)(left < 0x7fffffff ? left : 0x7fffffff);
      return __builtin_amdgcn_make_buffer_rsrc(W + (rb < nrows ? rb : 0) * b, 0, nrec, 0x00020000);
    };
    auto voff = [&](int cc) {  // this lane's column in block cc, row offset 4 lk
      const int64_t rel = wc_rel + cc * 32 + lr;
      return rel < ncols ? (int)((4 * lk * b + col0 + rel) * 4) : 0x7fffffff;
    };
    // row 8 (r/4) + (r%4) of the lane's block rows: its offset goes into the
    // per-lane offset, which the range check covers (the scalar offset of a buffer
    // access is added to the address outside that check); an out-of-range column's
    // marker stays at or above 2^31 - 1, past every record count
    auto row_off = [&](int vo, int r) {
      return (int)((unsigned)vo + (unsigned)((8 * (r >> 2) + (r & 3)) * b * 4));
    };
    auto load_group = [&](int a, float (&v)[64]) {
      const auto rs = rsrc_of(a);
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const int vo = voff(cc);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          v[cc * 16 + r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                               rs, row_off(vo, r), 0, 0));
      }
    };
    float cur[64], nxt[64];
    load_group(0, cur);
    static_for<0, 4>([&](auto A) __attribute__((always_inline)) {
      constexpr int a = A;
      if constexpr (a + 1 < 4) load_group(a + 1, nxt);
      const auto rs = rsrc_of(a);
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const int vo = voff(cc);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          __builtin_amdgcn_raw_buffer_store_b32(
              __builtin_bit_cast(unsigned, cur[cc * 16 + r] - acc[a][cc][r]), rs,
              row_off(vo, r), 0, 0);
      }
      if constexpr (a + 1 < 4) {
#pragma unroll
        for (int e = 0; e < 64; ++e) cur[e] = nxt[e];
      }
    });
    }
  }
}

// W -= the sum of a cut tile's m slots (added in slot order). Sixteen workgroups per
// cut tile, one per accumulator block (a, cc) of far_x3_kernel's threads: thread t
// takes the values thread t held there (its 16 KB of each slot are contiguous),
// reads all of W's 16 values first, then writes them back.
__global__ __launch_bounds__(256) void far_fix_kernel(float* __restrict__ W, int64_t nrows, int64_t b,
                                                      int64_t col0, int64_t ncols,
                                                      const float* __restrict__ slots, FarSplit sp) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wrow = wave >> 1, wcol = wave & 1;
  const int lr = lane & 31, lk = lane >> 5;
  const int tl = blockIdx.x >> 4, a = (blockIdx.x >> 2) & 3, cc = blockIdx.x & 3;
  const int lin = sp.nwhole + tl;
  const int ti = lin % sp.nti, tj = lin / sp.nti;
  const int64_t rel = (int64_t)tj * kX3Tile + wcol * 128 + cc * 32 + lr;
  if (rel >= ncols) return;
  const int64_t rb = (int64_t)ti * kX3Tile + wrow * 128 + a * 32 + 4 * lk;
  float* wcolp = W + col0 + rel;
  float w[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t row = rb + 8 * (r >> 2) + (r & 3);
    w[r] = row < nrows ? wcolp[row * b] : 0.f;
  }
  const float4* base = (const float4*)(slots + (int64_t)tl * sp.m * kFarSlotFloats) +
                       (a * 4 + cc) * 4 * 256 + tid;
  float4 sum[4];
#pragma unroll
  for (int rq = 0; rq < 4; ++rq) sum[rq] = base[rq * 256];
  for (int i = 1; i < sp.m; ++i) {
    const float4* sl = base + (int64_t)i * (kFarSlotFloats / 4);
    float4 v[4];
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) v[rq] = sl[rq * 256];
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      sum[rq].x += v[rq].x; sum[rq].y += v[rq].y; sum[rq].z += v[rq].z; sum[rq].w += v[rq].w;
    }
  }
#pragma unroll
  for (int rq = 0; rq < 4; ++rq) {
    const float vals[4] = {sum[rq].x, sum[rq].y, sum[rq].z, sum[rq].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t row = rb + 8 * rq + e;  // value r = 4 rq + e: row 8 (r/4) + (r%4)
      if (row < nrows) wcolp[row * b] = w[4 * rq + e] - vals[e];
    }
  }
}

constexpr int64_t kFarMinTiles = 96;  // fewer 256 x 256 tiles: the 128 x 128 update is as fast

struct FarDims {
  int64_t ldA, ldB, ldy, kp;
};
FarDims far_dims(int64_t c, int64_t ncols, int64_t K) {
  FarDims d;
  d.ldA = cdiv(c, kX3Tile) * kX3Tile;
  d.ldB = cdiv(ncols, kX3Tile) * kX3Tile;
  d.ldy = d.ldA + d.ldB;
  d.kp = cdiv(K, 64) * 64;
  return d;
}

// Y's three planes, rounded up to 256 bytes; the piece slots follow.
int64_t far_y_elems(const FarDims& d) { return cdiv(3 * d.kp * d.ldy, 128) * 128; }

constexpr int kFarMaxPieces = 256;  // slots in the workspace (256 KB each)

int far_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) {
    (void)hipGetLastError();
    return 256;
  }
  return n;
}

// Whole rounds of P tiles run whole; the T tiles of a last, partial round are cut
// into m = floor(P' / T) pieces (P' = min(P, slots)) when that gives at least two,
// each piece at least three stages (the pipeline keeps three stages in flight).
FarSplit far_split(int nti, int ntiles, int nst, int P) {
  FarSplit sp;
  sp.nst = nst;
  sp.nti = nti;
  sp.ntiles = ntiles;
  const int cap = P < kFarMaxPieces ? P : kFarMaxPieces;
  const int T = ntiles % P;
  int m = T > 0 ? cap / T : 1;
  if (m > nst / 3) m = nst / 3;
  if (m < 2) {
    sp.nwhole = ntiles;
    sp.m = 1;
  } else {
    sp.nwhole = ntiles - T;
    sp.m = m;
  }
  sp.per_xcd = (int)cdiv(sp.nwhole, 8);
  return sp;
}

}  // namespace

bool far_x3_applies(int64_t c, int64_t ncols, int64_t K) {
  if (K <= 0 || K % kX3StageK || ncols <= 0) return false;
  const FarDims d = far_dims(c, ncols, K);
  if (3 * d.kp * d.ldy * 2 >= ((int64_t)1 << 31)) return false;  // 32-bit load offsets
  return cdiv(c, kX3Tile) * cdiv(ncols, kX3Tile) >= kFarMinTiles;
}

size_t far_x3_elems(int64_t c, int64_t ncols_max, int64_t K) {
  const FarDims d = far_dims(c, ncols_max, K);
  return (size_t)(far_y_elems(d) + (int64_t)kFarMaxPieces * kFarSlotFloats * 2);
}

hipError_t launch_far_update(float* W, int64_t c, int64_t b, int64_t r0, int64_t K, int64_t ldz,
                             int64_t col0, int64_t col_end, const float* Z, const float* R,
                             unsigned short* Y, hipStream_t s) {
  const int64_t ncols = col_end - col0;
  const FarDims d = far_dims(c, ncols, K);
  hipLaunchKernelGGL(far_build_kernel, dim3((unsigned)(d.ldy / 64), (unsigned)(d.kp / 64)),
                     dim3(256), 0, s, Z, ldz, c, R, r0, b, col0, ncols, (int)K, Y, d.ldy, d.ldA,
                     d.kp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nti = (int)(d.ldA / kX3Tile), ntj = (int)(d.ldB / kX3Tile);
  const FarSplit sp = far_split(nti, nti * ntj, (int)(K / kX3StageK), far_cus());
  float* slots = (float*)(Y + far_y_elems(d));
  const int ncut = sp.ntiles - sp.nwhole;
  if (sp.nwhole > 0) {
    hipLaunchKernelGGL(far_x3_kernel<false>, dim3((unsigned)(8 * sp.per_xcd)), dim3(256), 0, s, W,
                       c, b, col0, ncols, Y, d.ldy, d.ldA, d.kp, sp, slots);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (ncut == 0) return hipSuccess;
  hipLaunchKernelGGL(far_x3_kernel<true>, dim3((unsigned)(ncut * sp.m)), dim3(256), 0, s, W, c, b,
                     col0, ncols, Y, d.ldy, d.ldA, d.kp, sp, slots);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(far_fix_kernel, dim3((unsigned)(ncut * 16)), dim3(256), 0, s, W, c, b, col0, ncols,
                     (const float*)slots, sp);
  return hipGetLastError();
}

}  // namespace th
