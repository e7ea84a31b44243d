// Global -> LDS DMA helpers shared by the kernels that stage operands in LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace qlora {

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void *)p));
}

// One 16-byte-per-lane global -> LDS DMA (lane i lands at dst + 16 i; dst is
// wave-uniform).  Written as asm rather than the builtin: the compiler counts
// a builtin LDS DMA as an LDS access of unknown order, which turns every later
// LDS wait into a full drain (lgkmcnt(0)).  The asm has no register results;
// callers read the destination only after an explicit vmcnt wait and barrier.
__device__ __forceinline__ void dma16(const void *src, uint32_t dst) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(dst) : "memory");
}

}  // namespace qlora
