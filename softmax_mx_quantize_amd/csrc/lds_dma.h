// LDS staging helpers shared by the attention kernels (gfx950 / CDNA4):
// direct buffer -> LDS loads, their waits, and the workgroup barrier of a
// prefetch ring.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fsa {

// Direct buffer -> LDS loads (lane i of the wave writes the 16 (4) bytes it
// loads at lds + 16 i (4 i)), issued as inline assembly: the compiler then
// adds no waits of its own for them.  Its own tracking of such loads loses
// precision across the unrolled sweep and made each tile wait for the loads
// issued just before it; the sweep orders them explicitly instead (a vmcnt
// wait before each workgroup barrier).  M0 carries the LDS address.  The
// compiler inserts no wait states ahead of inline assembly, so the load
// brings its own: 5, the most any of its operands needs (a buffer resource
// or offset in scalar registers the vector unit has just written, as when
// the compiler refills spilled scalar registers with v_readlane; 1 after an
// M0 write).
__device__ __forceinline__ void dma_lds16(__amdgpu_buffer_rsrc_t rs, uint32_t lds, int voff, int soff) {
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rs), "s"(soff), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void dma_lds4(__amdgpu_buffer_rsrc_t rs, uint32_t lds, int voff, int soff) {
  asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rs), "s"(soff), "{m0}"(lds) : "memory");
}
// 32-bit LDS address of a __shared__ object
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Workgroup barrier for the LDS ring.  __syncthreads() releases at
// workgroup scope, which makes the compiler wait for every LDS DMA still in
// flight (vmcnt(0)) and so drains the prefetch ring at each tile.  Here the
// waits are explicit instead: each wave has waited for the DMA of the tile
// the next phase reads (vmcnt before the call), and its own LDS reads
// complete before the barrier, so nobody refills a stage still being read.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace fsa
