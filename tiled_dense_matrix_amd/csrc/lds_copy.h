// Direct global -> LDS copies (global_load_lds_dwordx4) shared by the tiled
// matrix-core kernels, and the LDS pointer type they use.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define LDS_PTR(T) __attribute__((address_space(3))) T*

namespace tdm {

// One 16-byte-per-lane global -> LDS copy from sbase + voff: lane l's 16
// bytes land at lds_addr + 16*l. Issued as inline assembly so that the
// compiler does not treat it as an LDS write of unknown address and stall
// every later LDS read on it; completion is awaited explicitly (wait_vm)
// before the barrier that publishes the buffer. M0 carries the LDS address;
// nothing else in the kernels that use it touches M0.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory", "m0");
}

// Same, marked non-temporal: for data streamed once (the small-M paths'
// weights), so its lines do not displace reused ones in the caches. With
// operands rotated beyond the last-level cache, 16 x 8192 x 8192 with B
// stored N x K took 23.3 us with the mark, 24.7 us without.
__device__ __forceinline__ void dma16_stream(const void* sbase, uint32_t voff,
                                             uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :
               : "v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory", "m0");
}

// Same with 4 bytes per lane (global_load_lds_dword): lane l's 4 bytes land
// at lds_addr + 4*l. The global address must be 4-byte aligned.
__device__ __forceinline__ void dma4(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory", "m0");
}

// Wait until at most N of this wave's vector-memory operations are in flight
// (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Byte address of an LDS pointer, as M0 and the copy take it.
__device__ __forceinline__ uint32_t lds_offset(LDS_PTR(const uint8_t) p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

}  // namespace tdm
