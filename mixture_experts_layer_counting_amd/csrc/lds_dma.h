// Direct global->LDS loads and the explicit waits that go with them (gfx950).
//
// buffer_load_dwordx4 ... lds writes lane l's 16 bytes to LDS at M0 + 16 l; offsets past the
// buffer descriptor's range (checked on the per-lane offset) load zeros without touching
// memory. The loads are issued from inline asm so that the compiler does not put a full
// vmcnt(0) wait in front of every later LDS read; completion is tracked explicitly with
// s_waitcnt vmcnt(N) (vector-memory loads complete in issue order).
#pragma once

#include "moe_common.h"

namespace moe {

// Buffer descriptor (base, range in bytes; raw, stride 0) in scalar registers.
__device__ __forceinline__ i32x4_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xffff);
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

// Direct global->LDS load of 16 bytes per lane (buffer_load_dwordx4 ... lds): lane l's bytes
// land at lds_base + 16*l, offsets past the descriptor's range write zeros. Written as asm so
// the compiler does not add a full vmcnt(0) wait before every later LDS read; completion is
// tracked explicitly with wait_barrier<N>() below. No output registers.
__device__ __forceinline__ void lds_dma16(i32x4_t rsrc_in, uint32_t lds_base, int voff, int soff) {
  i32x4_t rsrc;
#pragma unroll
  for (int i = 0; i < 4; ++i) rsrc[i] = __builtin_amdgcn_readfirstlane(rsrc_in[i]);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane((int)lds_base)), "v"(voff), "s"(rsrc),
                 "s"(__builtin_amdgcn_readfirstlane(soff))
               : "memory", "m0");
}

// lds_dma16 with the non-temporal cache policy (nt): for data read once, such as an expert's
// weight panel streamed from HBM, so that it does not displace lines that are still reused.
__device__ __forceinline__ void lds_dma16_nt(i32x4_t rsrc_in, uint32_t lds_base, int voff, int soff) {
  i32x4_t rsrc;
#pragma unroll
  for (int i = 0; i < 4; ++i) rsrc[i] = __builtin_amdgcn_readfirstlane(rsrc_in[i]);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane((int)lds_base)), "v"(voff), "s"(rsrc),
                 "s"(__builtin_amdgcn_readfirstlane(soff))
               : "memory", "m0");
}

// Direct global->LDS load of 4 bytes per lane (buffer_load_dword ... lds): lane l's dword lands
// at lds_base + 4*l; offsets past the descriptor's range write zeros. Counted in vmcnt like
// lds_dma16.
__device__ __forceinline__ void lds_dma4(i32x4_t rsrc_in, uint32_t lds_base, int voff, int soff) {
  i32x4_t rsrc;
#pragma unroll
  for (int i = 0; i < 4; ++i) rsrc[i] = __builtin_amdgcn_readfirstlane(rsrc_in[i]);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane((int)lds_base)), "v"(voff), "s"(rsrc),
                 "s"(__builtin_amdgcn_readfirstlane(soff))
               : "memory", "m0");
}

// Wait until at most N of this wave's vector-memory operations are outstanding, then
// barrier the workgroup. The memory clobber keeps LDS reads on their side of the barrier.
template <int N>
__device__ __forceinline__ void wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" : : "n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const MOE_LDS void*)p;
}

template <int N>
__device__ __forceinline__ void wait_barrier_dyn(int n) {
  // n in [0, N]: dispatch to the compile-time immediates
  if constexpr (N > 0) {
    if (n >= N) {
      wait_barrier<N>();
      return;
    }
    wait_barrier_dyn<N - 1>(n);
  } else {
    wait_barrier<0>();
  }
}

// Wait until at most N of this wave's vector-memory operations are outstanding (no barrier).
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// n in [0, N] at run time, uniform over the wave: dispatch to the immediates N, N-1, ..., 0
template <int N>
__device__ __forceinline__ void wait_vm_dyn(int n) {
  if constexpr (N > 0) {
    if (n >= N) {
      wait_vm<N>();
      return;
    }
    wait_vm_dyn<N - 1>(n);
  } else {
    wait_vm<0>();
  }
}

}  // namespace moe
