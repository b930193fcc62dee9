// Direct global -> LDS copies (global_load_lds_dwordx4) and explicit
// vector-memory waits for gfx950 kernels that stage tiles in LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dr {

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4):
// lane l's bytes land at lds_wave_base + 16*l. Written as inline asm so that
// the compiler does not treat the destination as a pending LDS write of this
// wave (which makes it drain every load before each LDS access); callers wait
// on these loads themselves with explicit s_waitcnt vmcnt. The asm has no
// output register and the address registers are read at issue; one wait state
// separates the M0 write from the load that reads it (the compiler cannot see
// inside the asm to insert it). M0 is a reserved register: naming it as
// clobbered does not make the compiler save it, so this is sound only while no
// compiler-generated instruction of the calling kernels uses M0 (hipcc warns
// about the clobber; the codegen test checks the generated code for it).
__device__ inline void dma16(const void* gptr, unsigned char* lds_wave_base) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds_wave_base);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(gptr) : "memory", "m0");
}

// The same copy with an SGPR base and a per-lane 32-bit byte offset (saddr form).
__device__ inline void dma16_s(const void* sbase, unsigned voff, unsigned char* lds_wave_base) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds_wave_base);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m0), "v"(voff), "s"(sbase) : "memory", "m0");
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

}  // namespace dr
