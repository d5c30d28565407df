// Copies from global memory straight into LDS (global_load_lds_*: no
// registers held while a copy is in flight), and waits on their count.
//
// The copies are inline asm on purpose: the compiler does not track them, so
// it neither places a vmcnt(0) before every LDS read that might alias a copy
// in flight nor at a barrier; the caller issues a fixed number of copies per
// pipeline step and waits for exactly the ones it needs (vector memory loads
// complete in order, so copies issued later only make a wait stricter).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {
namespace {

// LDS byte address of a shared-memory object
__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16 bytes per lane from global memory into LDS at m0_base + 16 * lane
// (one wave writes 1 KB).  M0 is saved and restored around the copy.
__device__ inline void copy16_to_lds(const void* gaddr, uint32_t m0_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gaddr), "s"(m0_base)
      : "memory");
}

// 4 bytes per lane into LDS at m0_base + 4 * lane (one wave writes 256 B)
__device__ inline void copy4_to_lds(const void* gaddr, uint32_t m0_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gaddr), "s"(m0_base)
      : "memory");
}

// The same copies with a scalar base: lane l reads base + voff (voff a 32-bit
// byte offset), so a loop whose lanes keep fixed offsets from a moving base
// spends no vector instructions on addresses.
__device__ inline void copy16_to_lds_s(uint32_t voff, const void* sbase, uint32_t m0_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(m0_base)
      : "memory");
}
__device__ inline void copy4_to_lds_s(uint32_t voff, const void* sbase, uint32_t m0_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(m0_base)
      : "memory");
}

// s_waitcnt vmcnt(n) for a uniform n in 0..15 (expcnt and lgkmcnt untouched)
__device__ inline void wait_vmcnt(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
    case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
    case 7: __builtin_amdgcn_s_waitcnt(0x0F77); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    case 9: __builtin_amdgcn_s_waitcnt(0x0F79); break;
    case 10: __builtin_amdgcn_s_waitcnt(0x0F7A); break;
    case 11: __builtin_amdgcn_s_waitcnt(0x0F7B); break;
    case 12: __builtin_amdgcn_s_waitcnt(0x0F7C); break;
    case 13: __builtin_amdgcn_s_waitcnt(0x0F7D); break;
    case 14: __builtin_amdgcn_s_waitcnt(0x0F7E); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F7F); break;
  }
}

}  // namespace
}  // namespace tq
