// LDS staging helpers shared by the direct-to-LDS kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dp_common.hpp"

namespace dpk {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) unsigned char lds_uchar;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

// 16 bytes per lane from global memory straight into LDS at lds_base + 16*lane
// (global_load_lds_dwordx4, base in M0). Written as asm so that the
// compiler's wait insertion does not treat every later LDS read as aliasing
// it: the pipeline orders these loads with explicit vmcnt waits + barriers.
// The global address is a wave-uniform 64-bit base plus this lane's 32-bit
// byte offset (the instruction's SGPR-base form).
__device__ __forceinline__ void dma16(const void* gbase, uint32_t byte_off, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(byte_off), "s"(gbase),
               "s"(lds_base)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const unsigned char* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const lds_uchar*)p);
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS reads
// (lgkmcnt) but not for its global loads in flight (vmcnt), which the
// pipeline waits for explicitly. The memory clobber keeps the compiler from
// moving memory operations across it. The wait is also given as a builtin,
// which the compiler's wait insertion sees (it cannot see into the asm):
// without it the pass keeps assuming that scalar loads from before the loop
// may be outstanding, and since those return out of order it then waits for
// every LDS read of a chunk before the chunk's first MFMA.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt(63), expcnt(7): no wait
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until at most k chunks of `LPC` loads each are still in flight
// (k <= MAXK); uniform branches down to an immediate vmcnt.
template <int LPC, int MAXK>
__device__ __forceinline__ void wait_chunks(int k) {
  if constexpr (MAXK == 0) {
    wait_vmcnt<0>();
  } else {
    if (k >= MAXK)
      wait_vmcnt<LPC * MAXK>();
    else
      wait_chunks<LPC, MAXK - 1>(k);
  }
}

}  // namespace dpk
