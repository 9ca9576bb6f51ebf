// Global -> LDS copies (LDS DMA) and the waits on them, shared by the GEMM
// and router kernels.
#pragma once

#include "moe_common.h"

namespace moe {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

// 16 bytes per lane, global address per lane -> the wave's LDS block.
__device__ __forceinline__ void lds_dma16(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)g, (lds_void_t*)l, 16, 0, 0);
}

// 4 bytes per lane, global address per lane: lane l's word lands at byte 4 l
// of the wave's LDS block.
__device__ __forceinline__ void lds_dma4(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)g, (lds_void_t*)l, 4, 0, 0);
}

// 16-byte-per-lane global -> LDS copy through a raw buffer resource: a
// wave-uniform base plus a 32-bit byte offset per lane.
__device__ __forceinline__ void buf_dma16(const void* base, uint32_t voff, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  // base is wave-uniform: saying so keeps the descriptor in SGPRs (else every
  // load becomes a loop over the lanes' descriptors)
  const uint64_t b = (uint64_t)base;
  const uint64_t ub = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)ub, (short)0, -1, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, (int)voff, 0, 0, 0);
#endif
}

// s_waitcnt vmcnt(N) with expcnt/lgkmcnt left unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Rows of 128 bytes (a 64-wide bf16 K block) in LDS: physical 16-byte chunk
// of logical chunk c in row r is c ^ pp_swz(r) (an involution), which
// spreads 32-row fragment reads over the banks.
__device__ __forceinline__ int pp_swz(int r) { return (r >> 2) & 3; }

}  // namespace moe
