// Direct global->LDS loads shared by the bf16 matrix-core kernels.
#pragma once

#include "common.h"

namespace th {

// One stage's share of a wave: eight loads of 16 bytes per lane from global
// memory straight into LDS (global_load_lds_dwordx4; lane l writes LDS bytes
// [M0 + 16 l, M0 + 16 l + 16)). Load i writes the 1 KB chunk at lds + 0, 16384,
// 4096, 20480, 8192, 24576, 12288, 28672 for i = 0..7 (eight chunks 4 KB apart
// over a 32 KB stage; the callers interleave their panels that way). Written as
// one asm block so that the compiler does not make LDS reads of other buffers
// wait for these loads -- completion is tracked by the explicit vmcnt waits
// before each barrier -- and so that M0 is restored before the compiler sees it
// again. The loads have no result registers.
__device__ __forceinline__ void lds_dma_stage(const void* const (&g)[8], const void* lds) {
  const unsigned base = __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)lds);
  unsigned saved;
  __asm__ volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %9, off\n\t"
      "s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %10, off\n\t"
      "s_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %11, off\n\t"
      "s_mov_b32 m0, %4\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %12, off\n\t"
      "s_mov_b32 m0, %5\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %13, off\n\t"
      "s_mov_b32 m0, %6\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %14, off\n\t"
      "s_mov_b32 m0, %7\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %15, off\n\t"
      "s_mov_b32 m0, %8\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %16, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(base), "s"(base + 16384u), "s"(base + 4096u), "s"(base + 20480u),
        "s"(base + 8192u), "s"(base + 24576u), "s"(base + 12288u), "s"(base + 28672u),
        "v"(g[0]), "v"(g[1]), "v"(g[2]), "v"(g[3]), "v"(g[4]), "v"(g[5]), "v"(g[6]), "v"(g[7]));
}

}  // namespace th

namespace th {

// Ten loads of 16 bytes per lane straight into LDS, in the saddr form: per-lane
// 32-bit byte offsets vo[k] (< 2^31) from two wave-uniform 64-bit bases (SGPRs),
// g0 for the even loads and g1 for the odd ones. Load m = 2k + o takes vo[k]
// from g_o and writes the 1 KB chunk at lds + 4096 m. No result registers;
// completion is tracked by the callers' vmcnt waits. The s_add_u32 that step M0
// write SCC, which the clobber list declares.
__device__ __forceinline__ uint64_t uniform_u64(uint64_t x) {
  // readfirstlane returns int: go through unsigned so the low half is not sign-extended
  return ((uint64_t)(unsigned)__builtin_amdgcn_readfirstlane((unsigned)(x >> 32)) << 32) |
         (uint64_t)(unsigned)__builtin_amdgcn_readfirstlane((unsigned)x);
}
__device__ __forceinline__ void lds_dma10s(const unsigned (&vo)[5], const void* gbase0,
                                           const void* gbase1, const void* lds) {
  const unsigned base = __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)lds);
  const uint64_t g0 = uniform_u64((uint64_t)(uintptr_t)gbase0);
  const uint64_t g1 = uniform_u64((uint64_t)(uintptr_t)gbase1);
  unsigned saved;
  __asm__ volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %7\n\t"
      "s_add_u32 m0, %1, 4096\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %8\n\t"
      "s_add_u32 m0, %1, 8192\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %3, %7\n\t"
      "s_add_u32 m0, %1, 12288\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %3, %8\n\t"
      "s_add_u32 m0, %1, 16384\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %4, %7\n\t"
      "s_add_u32 m0, %1, 20480\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %4, %8\n\t"
      "s_add_u32 m0, %1, 24576\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %5, %7\n\t"
      "s_add_u32 m0, %1, 28672\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %5, %8\n\t"
      "s_add_u32 m0, %1, 32768\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %6, %7\n\t"
      "s_add_u32 m0, %1, 36864\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %6, %8\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(base), "v"(vo[0]), "v"(vo[1]), "v"(vo[2]), "v"(vo[3]), "v"(vo[4]), "s"(g0), "s"(g1)
      : "scc");
}

}  // namespace th
