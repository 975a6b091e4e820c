// LDS helpers shared by the attention kernels (gfx950): direct global->LDS loads,
// explicit waits for them, a barrier without implied waits, LDS byte addresses.
#pragma once

#include "common.hpp"

namespace vdit {
namespace {

// 16 bytes per lane from global memory straight into LDS (global_load_lds_dwordx4):
// lane l of the wave writes LDS bytes [lds + 16 l, lds + 16 l + 16); `lds` is an
// LDS byte address, the same for the whole wave. Written as inline assembly so
// that the compiler does not track these loads: every wait for them is explicit
// (wait_vm), which lets loads for later tiles stay in flight across barriers.
// The statement has no register outputs; the LDS address is an M0 input.
// Because the compiler does not see a memory instruction here, it also does not
// insert the wait states such an instruction needs after its operands are
// written: the global address therefore comes in VGPRs (dependencies on VGPRs
// are interlocked by the hardware, unlike an SGPR base written by VALU), and
// the s_nop covers the one wait state an LDS-DMA load needs after M0 is written.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}

// s_waitcnt vmcnt(N): all but the newest N vector-memory loads of this wave have
// completed (loads complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// workgroup barrier that the compiler may not move LDS accesses across; it
// waits for nothing by itself
__device__ __forceinline__ void barrier_only() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}

}  // namespace
}  // namespace vdit
