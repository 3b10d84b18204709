// Direct global -> LDS loads, the activation-row swizzle and the NF4
// level-pair table offsets shared by the fused NF4 GEMM kernels
// (gemm_nf4f.hip: the projection y = x W; gemm_nf4t.hip: its input gradient).
#pragma once
#include "common.h"
#include <stdint.h>

namespace lsn {
namespace {

// One direct global -> LDS load of 16 (or 4) bytes per lane: lane l writes
// LDS bytes [lds + 16 l, +16) from gbase + voff (gbase and lds uniform).  M0
// carries the LDS address; one wait state separates its write from the load.
// No register is written.  The compiler uses M0 nowhere else in the kernels
// that call these (a test checks the generated code), so the asm overwrites
// it freely.
LSN_DEV void dma16(const void* gbase, uint32_t voff, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(gbase), "s"(lds)
      : "memory");
}
LSN_DEV void dma4(const void* gbase, uint32_t voff, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %0, %1"
      :
      : "v"(voff), "s"(gbase), "s"(lds)
      : "memory");
}

// The same loads with M0 set once for a group: the instruction offset OFS
// (13-bit signed) moves both the global address and the LDS address
// (M0 + OFS + 16 lane), so the per-lane global offset passed in has OFS
// already subtracted.  set_m0 includes the wait state before the first use.
LSN_DEV void set_m0(uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0" : : "s"(lds) : "memory");
}
template <int OFS>
LSN_DEV void dma16_at(const void* gbase, uint32_t voff) {
  asm volatile("global_load_lds_dwordx4 %0, %1 offset:%2" : : "v"(voff), "s"(gbase), "i"(OFS)
               : "memory");
}
template <int OFS>
LSN_DEV void dma4_at(const void* gbase, uint32_t voff) {
  asm volatile("global_load_lds_dword %0, %1 offset:%2" : : "v"(voff), "s"(gbase), "i"(OFS)
               : "memory");
}

template <typename T>
LSN_DEV uint32_t lds_addr(T* q) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)q;
}

// swizzle of the 16-byte chunk index of activation row r: rows r and r + 8
// differ in the low bit so that 16 consecutive rows reading one logical chunk
// hit 16 distinct 4-bank groups (and 8 consecutive rows 8 distinct ones)
LSN_DEV int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Work unit (tile id, k split) of this workgroup.  Workgroups go to the 8
// XCDs round robin by linear id; each XCD takes a contiguous range of the
// units ordered split-major, so the workgroups of one XCD share one split's
// K range of the activations (a working set that fits its L2) besides
// weight tiles.  Without a split this is the plain contiguous tile range.
struct WorkUnit {
  int tile, split;
};
LSN_DEV WorkUnit xcd_unit() {
  const int X = gridDim.x, U = X * gridDim.y;
  const int L = blockIdx.x + blockIdx.y * X;
  const int x = L % 8, per = U / 8, rem = U % 8;
  const int u = x * per + min(x, rem) + L / 8;
  return {u % X, u / X};
}

// byte offset 8 * (byte p of code word q) into the level-pair table
LSN_DEV uint32_t pair_off(uint32_t q, int p) {
  return ((q >> (8 * p)) & 0xFFu) << 3;
}

}  // namespace
}  // namespace lsn

// s_waitcnt with only the vector-memory count constrained (gfx9 encoding)
#define LSN_WAIT_VM(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))
