// lds_copy.h -- direct global-to-LDS copies for the MFMA kernels that stream their weights
// through LDS, and the load-counter waits that go with them.
//
// A 16-byte copy instruction moves 64 lanes x 16 B (lane l's bytes land at dst + 16 l), so
// a wave can read whole 128-byte lines per instruction whatever layout the MFMA operands
// need afterwards.  The copies are issued from asm: the compiler then does not track them,
// and adds no wait for all copies before every later LDS access (without alias scopes it
// cannot tell ring slots and other LDS buffers apart).  Their completion is awaited
// explicitly (gl_wait_vm / gl_wait_n); VMEM operations the compiler does not see only make
// its own load-counter waits stricter, as the counter completes in order.  M0 carries the
// LDS address; nothing else in these kernels uses M0.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace moe {

__device__ __forceinline__ void gl_copy16(const lds_u8* dst, const uint8_t* src) {
  const uint32_t la = (uint32_t)(uintptr_t)dst;
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(la), "v"(src)
               : "memory");
}

// s_waitcnt with vmcnt = N (gfx9 encoding: vmcnt bits [3:0] and [15:14]; expcnt and
// lgkmcnt left at their no-wait values).
template <int N>
__device__ __forceinline__ void gl_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 0xF) | ((N >> 4) << 14));
}

// The same for a count known once the loop around it is unrolled.  n >= 63 needs no wait:
// a wave holds at most 63 loads in flight (the counter's width), so a copy followed by 63
// or more has landed.
template <int N>
__device__ __forceinline__ void gl_wait_upto(int n) {
  if (n == N) {
    gl_wait_vm<N>();
  } else if constexpr (N > 0) {
    gl_wait_upto<N - 1>(n);
  }
}
__device__ __forceinline__ void gl_wait_n(int n) { gl_wait_upto<63>(n); }

// lgkmcnt(0): every LDS (and scalar) access issued so far has completed, e.g. the reads of
// a ring slot before a copy overwrites it.
__device__ __forceinline__ void gl_wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

}  // namespace moe
