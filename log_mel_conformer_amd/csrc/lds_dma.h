// CDNA helpers for buffer loads that write straight into LDS, shared by the
// GEMM and the local-attention kernels.
#pragma once

#include "common.h"

namespace ae {

// Buffer loads straight to LDS (buffer_load_dwordx4 ... lds): the LLVM
// intrinsic, declared by name, with the 128-bit buffer resource as four
// dwords: base address (48 bits, stride 0), size in bytes (reads at or past
// it return zeros) and the gfx9 format word.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ void raw_buffer_load_lds(i32x4 rsrc, __attribute__((address_space(3))) void* lds,
                                    int size, uint32_t voffset, uint32_t soffset, int offset,
                                    int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xFFFF);
  r.z = __builtin_amdgcn_readfirstlane((int)bytes);
  r.w = 0x00020000;
  return r;
}

// s_waitcnt vmcnt(N) with every other counter left alone (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt lgkmcnt(0): this wavefront's LDS reads have returned.
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}

}  // namespace ae
