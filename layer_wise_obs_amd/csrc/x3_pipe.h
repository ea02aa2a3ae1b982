// Direct global->LDS pipeline pieces for products of operands pre-split into three
// bf16 planes (x = h + m + l, each part rounded to nearest even, |x - h - m - l| <=
// 2^-24 |x|), k-major: plane p, k row kk, column i. 256 x 256 output tiles on
// four waves of 128 x 128, stages of 16 k rows of both operands (48 KB) copied
// into LDS by global_load_lds_dwordx4 with 16-byte pieces XOR-swizzled by k & 3,
// MFMA operands formed by ds_read_b64_tr_b16. Used by the factorisation's rest
// sets (rest_x3.h) and the block loop's far-column updates (far_x3.hip).
#pragma once

#include "common.h"

namespace th {

constexpr int kX3Rows = 256;                       // k extent of Y (two 128-wide steps)
constexpr int kX3Tile = 256;                       // output tile edge
constexpr int kX3StageK = 16;                      // k rows per LDS stage
constexpr int kX3PanelBytes = kX3StageK * kX3Tile * 2;   // one plane, one operand: 8 KB
constexpr int kX3StageBytes = 6 * kX3PanelBytes;        // 3 planes x (A, B): 48 KB
constexpr int kX3Stages = 3;

// Row pitch (elements) of the Y planes: b rounded up to whole 256-column tiles,
// zero-filled past b, so that tile loads never leave the buffer.
__host__ __device__ inline int64_t x3_ldy(int64_t b) { return cdiv(b, kX3Tile) * kX3Tile; }
// Elements of one Y buffer (three planes).
__host__ __device__ inline int64_t x3_y_elems(int64_t b) { return 3 * (int64_t)kX3Rows * x3_ldy(b); }

namespace x3d {

__device__ __forceinline__ int piece_off(int t, int fg) {
  return t * (kX3Tile * 2) + ((fg ^ ((t & 3) << 2)) << 4);
}

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef short v8i16_t __attribute__((ext_vector_type(8)));

// 32 features x 16 k from a panel of 16 k rows (see tr_frag of the syrk).
__device__ __forceinline__ bf16x8_t frag(const unsigned char* panel, int f0, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int fb = f0 + ((g & 1) << 4) + ((s & 3) << 2);
  const int tb = ((g >> 1) << 3) + (s >> 2);
  const int fg = fb >> 3, within = (fb & 7) << 1;
  const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16_t*)(panel + piece_off(tb, fg) + within));
  const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16_t*)(panel + piece_off(tb + 4, fg) + within));
  const v8i16_t r = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, r);
}

// One stage's share of a wave: twelve 1 KB chunks, chunk m of wave w at LDS
// offset (w + 4 m) KB, i.e. lds + m * 4096 with lds = stage base + w KB. The
// s_add_u32 that step M0 write SCC, hence the clobber: the compiler may hold a
// comparison in SCC across the block (the null check of the next LDS address).
__device__ __forceinline__ void dma12(const void* const (&g)[12], const void* lds) {
  const unsigned base = __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)lds);
  unsigned saved;
  __asm__ volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, off\n\t"
      "s_add_u32 m0, %1, 4096\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %3, off\n\t"
      "s_add_u32 m0, %1, 8192\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %4, off\n\t"
      "s_add_u32 m0, %1, 12288\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %5, off\n\t"
      "s_add_u32 m0, %1, 16384\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %6, off\n\t"
      "s_add_u32 m0, %1, 20480\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %7, off\n\t"
      "s_add_u32 m0, %1, 24576\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %8, off\n\t"
      "s_add_u32 m0, %1, 28672\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %9, off\n\t"
      "s_add_u32 m0, %1, 32768\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %10, off\n\t"
      "s_add_u32 m0, %1, 36864\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %11, off\n\t"
      "s_add_u32 m0, %1, 40960\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %12, off\n\t"
      "s_add_u32 m0, %1, 45056\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %13, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(base), "v"(g[0]), "v"(g[1]), "v"(g[2]), "v"(g[3]), "v"(g[4]), "v"(g[5]), "v"(g[6]),
        "v"(g[7]), "v"(g[8]), "v"(g[9]), "v"(g[10]), "v"(g[11])
      : "scc");
}

// The same twelve loads with a wave-uniform global base (SGPR pair) and one
// 32-bit byte offset per load and lane (saddr form): the offsets stay fixed for
// a tile, and a stage only moves the base.
__device__ __forceinline__ void dma12s(const unsigned (&vo)[12], const void* gbase, const void* lds) {
  const unsigned base = __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)lds);
  const uint64_t gb = (uint64_t)(uintptr_t)gbase;
  // readfirstlane returns int: go through unsigned so the low half is not sign-extended
  const uint64_t g =
      ((uint64_t)(unsigned)__builtin_amdgcn_readfirstlane((unsigned)(gb >> 32)) << 32) |
      (uint64_t)(unsigned)__builtin_amdgcn_readfirstlane((unsigned)gb);
  unsigned saved;
  __asm__ volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %14\n\t"
      "s_add_u32 m0, %1, 4096\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %3, %14\n\t"
      "s_add_u32 m0, %1, 8192\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %4, %14\n\t"
      "s_add_u32 m0, %1, 12288\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %5, %14\n\t"
      "s_add_u32 m0, %1, 16384\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %6, %14\n\t"
      "s_add_u32 m0, %1, 20480\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %7, %14\n\t"
      "s_add_u32 m0, %1, 24576\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %8, %14\n\t"
      "s_add_u32 m0, %1, 28672\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %9, %14\n\t"
      "s_add_u32 m0, %1, 32768\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %10, %14\n\t"
      "s_add_u32 m0, %1, 36864\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %11, %14\n\t"
      "s_add_u32 m0, %1, 40960\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %12, %14\n\t"
      "s_add_u32 m0, %1, 45056\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %13, %14\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(base), "v"(vo[0]), "v"(vo[1]), "v"(vo[2]), "v"(vo[3]), "v"(vo[4]), "v"(vo[5]),
        "v"(vo[6]), "v"(vo[7]), "v"(vo[8]), "v"(vo[9]), "v"(vo[10]), "v"(vo[11]), "s"(g)
      : "scc");
}

}  // namespace x3d

}  // namespace th
