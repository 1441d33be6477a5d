// Device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace wave {

// One 16-byte-per-lane direct global->LDS load: lane i's 16 bytes at
// base + off land at LDS address lds_addr + 16*i.  Written as inline asm so
// that the compiler does not treat the asynchronous LDS write as aliasing the
// LDS tiles being read (it would then wait for every load in flight before
// each LDS read); completion is tracked explicitly with s_waitcnt vmcnt and a
// workgroup barrier.  The instruction has no register results.  M0 is set
// here and used by nothing else in these kernels.
__device__ __forceinline__ void load_lds16(uint32_t lds_addr, const char* base, uint32_t off) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds_addr), "v"(off), "s"(base)
               : "memory", "m0");
}

}  // namespace wave
