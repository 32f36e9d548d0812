// Asynchronous global -> LDS copies for gfx950 (global_load_lds_dwordx4) and
// the waits that order them; shared by the attention and projection kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) char*)(p)));
}

// vmcnt(n) with expcnt/lgkmcnt left alone (gfx9 encoding of s_waitcnt).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that neither waits for outstanding global->LDS copies nor
// lets the compiler move memory operations across it; completion of the
// copies is ordered explicitly with wait_vmcnt.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One wave-wide asynchronous copy global -> LDS: lane l's 16 bytes at
// gbase + voff land at LDS byte address lds + 16*l.  Written as inline asm so
// that the compiler does not track it (it would otherwise drain every
// outstanding copy before each LDS read it cannot prove disjoint); completion
// is ordered explicitly with wait_vmcnt + lds_barrier.  The block writes no
// VGPR; M0 (the LDS base) is saved and restored and gets one wait state.
// kStream marks the read non-temporal: for bytes read once (the latent cache
// streamed by a decode attention), so they do not displace data that later
// reads reuse.
template <bool kStream = false>
__device__ __forceinline__ void dma_block(uint64_t gbase, uint32_t voff, uint32_t lds) {
  // both bases are wave-uniform by construction; make that explicit for the SGPR
  // operands (readfirstlane yields int: widen through uint32_t, never sign-extend)
  lds = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(lds)));
  const uint32_t hi = static_cast<uint32_t>(
      __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(gbase >> 32))));
  const uint32_t lo = static_cast<uint32_t>(
      __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(gbase))));
  gbase = (static_cast<uint64_t>(hi) << 32) | static_cast<uint64_t>(lo);
  uint32_t save;
  // s_nop 4: five wait states between any VALU write of the base SGPRs and the
  // vector-memory read of them (a hazard the compiler does not see inside asm)
  if constexpr (kStream)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 4\n\t"
        "global_load_lds_dwordx4 %1, %2 nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(save)
        : "v"(voff), "s"(gbase), "s"(lds)
        : "memory");
  else
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 4\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(save)
        : "v"(voff), "s"(gbase), "s"(lds)
        : "memory");
}

}  // namespace mla
