// tc_dma.hpp — global -> LDS copies (buffer_load ... lds) ordered by hand,
// shared by the kernels that stage their operand tiles this way (gfx950).
//
// The copy is written as inline asm rather than with the compiler builtin so
// that the compiler adds no s_waitcnt vmcnt(0) before every later LDS read
// and every barrier: each kernel orders its copies itself with
// wait_vmcnt<n>() (tc_mfma.hpp) and a workgroup barrier.  Loads complete in
// issue order, so vmcnt(n) after a copy means "every load issued before the
// last n has landed"; stores are not counted in n, since a store may complete
// ahead of an older load (the wait is then only longer than needed).
//
// The copy takes its LDS destination from M0.  On gfx9 an SALU write of M0
// needs one wait state before an LDS-DMA instruction reads it; the hazard
// recognizer of the compiler cannot see inside an asm string, so the string
// carries its own s_nop.  Without it the load may use the previous value of
// M0 and write its 1 KiB into the previous copy's LDS slot.
#pragma once

#include "tc_common.hpp"

namespace tc {
namespace dma {

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor over [base, base + nbytes) (gfx9 layout: stride 0,
// word 3 = raw dword data, no swizzle).  A load at an offset at or past
// nbytes (or a negative offset, which wraps to a huge unsigned one) returns
// zero instead of touching memory.
__device__ __forceinline__ i32x4 raw_desc(const void* base, uint32_t nbytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{static_cast<int>(a), static_cast<int>((a >> 32) & 0xFFFF), static_cast<int>(nbytes),
               0x00020000};
}

// 16 bytes per lane global -> LDS: lane i writes lds_base + 16 i.  lds_base
// must be wave-uniform.  No register is written, and every operand is read
// when the instruction issues.
__device__ __forceinline__ void dma16(i32x4 desc, const void* lds_base, int voffset) {
  const uint32_t lds = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_base;
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds), "v"(voffset), "s"(desc)
      : "memory", "m0");
}

}  // namespace dma
}  // namespace tc
