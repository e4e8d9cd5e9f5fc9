// Global -> LDS copies by the buffer unit (LDS-DMA), shared by the GEMM kernels.
//
// One instruction copies, for every lane l, 16, 4 or 2 bytes from
// rsrc + voff(l) to the LDS address m0 + 16 l (16-byte form) or m0 + 4 l (the
// 4- and 2-byte forms; the 2-byte form writes its bytes zero-extended to a
// dword).  A lane whose offset lies past the descriptor's range writes zeros,
// so a copy that crosses the end of an operand, or a lane given an offset past
// every range, fills its LDS slot with zeros instead of reading.
#ifndef BSG_LDS_DMA_H
#define BSG_LDS_DMA_H

#include "bsg_internal.h"

namespace bsg {

// An offset past every descriptor's range: the buffer unit returns zeros.
constexpr int kDmaOutOfRange = 0x7ffffff0;

// A raw buffer descriptor over [base, base + bytes) as four uniform dwords,
// for the inline-asm copies below.
__device__ __forceinline__ v4i make_rsrc_words(const void* base, int64_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  v4i r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(b & 0xffffffffu));
  r[1] = __builtin_amdgcn_readfirstlane((int)(b >> 32));
  r[2] = __builtin_amdgcn_readfirstlane((int)(bytes > 0 ? bytes : 0));
  r[3] = 0x00020000;
  return r;
}

// The copies are issued through inline asm so that the compiler adds no waits
// for them in front of LDS reads of other stages; callers wait for them
// explicitly (vmcnt).  m0 is saved and restored around each copy.  The LDS
// address must be the same in every lane (it is read from the first).
__device__ __forceinline__ void dma16(v4i rsrc, uint32_t lds, int voff) {
  lds = __builtin_amdgcn_readfirstlane(lds);
  int save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "s"(lds), "v"(voff), "s"(rsrc)
      : "memory");
}

__device__ __forceinline__ void dma4(v4i rsrc, uint32_t lds, int voff) {
  lds = __builtin_amdgcn_readfirstlane(lds);
  int save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "s"(lds), "v"(voff), "s"(rsrc)
      : "memory");
}

__device__ __forceinline__ void dma2(v4i rsrc, uint32_t lds, int voff) {
  lds = __builtin_amdgcn_readfirstlane(lds);
  int save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "buffer_load_ushort %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "s"(lds), "v"(voff), "s"(rsrc)
      : "memory");
}

}  // namespace bsg

#endif  // BSG_LDS_DMA_H
