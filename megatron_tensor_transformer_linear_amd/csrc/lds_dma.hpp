// Device helpers for kernels that stage operands HBM -> LDS directly (gfx950): raw buffer
// resources, the LDS-direct 16-byte buffer load, vector-memory counter waits and a bare
// workgroup barrier.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace tpk {
namespace dma {

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Buffer offset past every resource range: such a load returns zeros.
constexpr uint32_t OOB = 0x80000000u;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding: vmcnt[3:0] in
// bits 3:0 and vmcnt[5:4] in bits 15:14; expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier without the release/acquire fences of __syncthreads (those would wait
// for every outstanding LDS-bound load); memory order is kept by explicit waits.
__device__ __forceinline__ void barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Raw buffer resource: base address, no stride, `bytes` bytes in range (loads at offsets at
// or past it return zeros), raw-buffer flags.  The arguments are wave-uniform; the resource
// lives in scalar registers.
__device__ __forceinline__ i32x4_t rsrc(const void* base, int64_t bytes) {
  const uint64_t a = (uint64_t)base;
  i32x4_t r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xFFFF));
  r.z = __builtin_amdgcn_readfirstlane((int)bytes);
  r.w = 0x00020000;
  return r;
}

// One LDS-direct 16-byte load per lane: lane i's 16 bytes, read from buffer offset
// voff + soff (soff wave-uniform), land at LDS address lds_base + IMM + 16 i.  Issued through
// inline assembly so that the compiler does not order later LDS reads behind a full
// vector-memory wait; completion is tracked by the caller's explicit vmcnt waits.  M0 (the LDS address of the load) is written
// here and read by nothing else.  The s_add_u32 also writes SCC, so SCC is declared clobbered.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <uint32_t IMM>
__device__ __forceinline__ void load16(uint32_t lds_base, uint32_t voff, i32x4_t res,
                                       uint32_t soff) {
  asm volatile("s_add_u32 m0, %0, %1\n\tbuffer_load_dwordx4 %2, %3, %4 offen lds"
               :: "s"(lds_base), "i"(IMM), "v"(voff), "s"(res), "s"(soff)
               : "memory", "m0", "scc");
}
#pragma clang diagnostic pop

// Compile-time loop: f(std::integral_constant<int, 0>{}) ... f(std::integral_constant<int, N-1>{}).
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

}  // namespace dma
}  // namespace tpk
