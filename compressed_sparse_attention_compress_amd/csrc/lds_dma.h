// Direct global->LDS loads and the waits that order them (gfx950).
//
// global_load_lds_dwordx4 moves 16 bytes per lane from global memory straight
// into LDS: lane i writes at (M0 + 16 i), so one wave instruction fills 1 KB of
// LDS.  Written as inline assembly so the compiler's wait analysis does not see
// it: with the builtin form it cannot tell which LDS buffer is being written and
// waits for every load in flight (vmcnt(0)) before any LDS read, which
// serialises multi-buffered pipelines.  Callers therefore order these loads
// themselves: WAIT_VMCNT(n) until the loads of the stage they need are done, then
// a workgroup barrier, then COMPILER_FENCE so no LDS read is moved above it.  The
// compiler still waits correctly for its own loads (it undercounts the loads in
// flight, so its waits can only be longer than needed, never shorter).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

typedef __attribute__((address_space(3))) unsigned char lds_u8;

// These statements write M0 without naming it as clobbered: M0 is a reserved
// register for the AMDGPU backend, which sets it immediately before each of its
// own uses and keeps no value in it across other instructions (clang warns that a
// clobber of it may not be honoured), so there is nothing to declare.

// s_waitcnt immediates (gfx9 encoding): at most n vector-memory ops of this wave
// outstanding / all LDS ops done.
#define WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | 0x70 | 0xF00)
#define WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xC07F)
#define COMPILER_FENCE() __asm__ volatile("" ::: "memory")

// 16 B per lane from a per-lane global address to LDS (wave-uniform base ldst).
__device__ __forceinline__ void dma16_asm(const void* gsrc, const lds_u8* ldst) {
  const uint32_t base = (uint32_t)(uintptr_t)ldst;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(base), "v"(gsrc) : "memory");
}
// 4 B per lane (one wave instruction fills 256 B of LDS).
__device__ __forceinline__ void dma4_asm(const void* gsrc, const lds_u8* ldst) {
  const uint32_t base = (uint32_t)(uintptr_t)ldst;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(base), "v"(gsrc) : "memory");
}
// Same with a wave-uniform 64-bit global base (SGPR pair) and a 32-bit per-lane byte offset.
__device__ __forceinline__ void dma16_asm_s(uint64_t sbase, uint32_t voff, const lds_u8* ldst) {
  const uint32_t base = (uint32_t)(uintptr_t)ldst;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(base), "v"(voff), "s"(sbase)
               : "memory");
}

}  // namespace csa2
