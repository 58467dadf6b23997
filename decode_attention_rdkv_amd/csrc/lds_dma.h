// Buffer resources and direct global -> LDS copies for gfx950, shared by the
// decode and scoring kernels.
//
// A raw buffer resource (stride 0) is range checked per dword: reads at or
// past its byte range return zeros and touch no memory, so partial tiles need
// no per-lane clamping.  `buffer_load_dword{,x4} ... lds` writes a wave's
// loaded dwords straight into LDS at M0 + instruction offset + (4 or 16) *
// lane, with no register round trip.  Kernels issue those copies as inline
// assembly (the compiler's memory-counter bookkeeping would otherwise wait for
// every outstanding copy before any LDS read) and wait for them explicitly
// with wait_vmem.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

namespace rdkv {
namespace dma {

constexpr int kBufferFlags = 0x00020000;   // raw buffer: range-checked, out-of-range reads return 0

// Raw buffer resource over [p, p + bytes) for the compiler's buffer builtins.
__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, int(bytes), kBufferFlags);
}

// The same resource as four scalar registers, for inline assembly.
typedef int rsrc4 __attribute__((ext_vector_type(4)));
__device__ inline rsrc4 buffer_rsrc4(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  rsrc4 r;
  r.x = __builtin_amdgcn_readfirstlane(int(uint32_t(a)));
  r.y = __builtin_amdgcn_readfirstlane(int(uint32_t(a >> 32) & 0xffff));   // stride 0
  r.z = __builtin_amdgcn_readfirstlane(int(bytes));
  r.w = kBufferFlags;
  return r;
}

// LDS byte address of a pointer into shared memory.
__device__ inline uint32_t lds_addr(const void* p) {
  return uint32_t(size_t((const __attribute__((address_space(3))) void*)p));
}

// Waits until at most N vector-memory instructions of this wave are in
// flight.  Loads complete in issue order, so this also completes every load
// issued before the N most recent ones.  The scheduling barriers keep the
// compiler from moving memory instructions across the wait.
template <int N>
__device__ inline void wait_vmem() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
  __builtin_amdgcn_sched_barrier(0);
}

}  // namespace dma
}  // namespace rdkv
