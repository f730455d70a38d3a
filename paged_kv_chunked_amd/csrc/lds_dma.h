// Direct-to-LDS loads (global_load_lds_dwordx4) and the waits for them, used
// by the kernels that stage tiles in LDS without passing them through
// registers.
#pragma once

#include <cstdint>

namespace pkv {
namespace {

// One 16-byte direct-to-LDS load per lane: lane i's 16 bytes from `src` land
// at LDS byte address lds + 16 i.  Issued from asm so that the compiler does
// not drain the vector-memory counter before every LDS read; the kernel waits
// for these loads itself (wait_vm) before the barrier that publishes a tile.
__device__ inline void dma16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds), "v"(src)
               : "memory", "m0");
}
template <int N>
__device__ inline void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

}  // namespace
}  // namespace pkv
