// pkv_ring.h -- pieces shared by the kernels fed through a direct-to-LDS ring:
// 16-byte global_load_lds_dwordx4 gathers, fence-free barriers, explicit vmcnt
// waits and the XOR chunk swizzle groups.
#pragma once

#include "pkv_device.h"

namespace pkv {

// XOR mask for chunk c of a row of NC chunks: swizzle inside aligned groups of 16, 8, 4 or 2
template <int NC>
__device__ __forceinline__ int swz_mask(int c) {
  if ((c | 15) < NC) return 15;
  if ((c | 7) < NC) return 7;
  if ((c | 3) < NC) return 3;
  if ((c | 1) < NC) return 1;
  return 0;
}

// s_barrier without the release/acquire fence of __syncthreads (the fence would
// drain the load ring); compiler-only memory clobbers keep LDS accesses in order
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0): own LDS writes done
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int N>
__device__ __forceinline__ void wait_loads() {
  asm volatile("" ::: "memory");
  wait_vmcnt<N>();
  asm volatile("" ::: "memory");
}

// One wave-instruction of the ring: lane l's 16 bytes at gptr land at
// lds_wave_base + 16 l.  Issued through inline assembly on purpose: the
// compiler treats a global_load_lds builtin as an LDS store of unknown address
// and then waits for every outstanding one (vmcnt(0)) before any later LDS
// read, which would drain the whole ring at each tile.  Here the kernels do
// that bookkeeping themselves (wait_loads before the barrier that publishes a
// stage).  M0 carries the LDS address; nothing else in these kernels uses M0.
__device__ __forceinline__ void dma16(const void* gptr, unsigned char* lds_wave_base) {
  // low word of the flat address of an LDS location = its LDS offset (the
  // shared aperture base has a zero low word); no address-space cast needed
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_wave_base);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(lds)
               : "memory", "m0");
}

// Same with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane offset
// (global SADDR form): the 64-bit address arithmetic happens once per
// wave-instruction on the scalar unit instead of in every lane.
__device__ __forceinline__ void dma16_saddr(uint64_t base, uint32_t voff, unsigned char* lds_wave_base) {
  // low word of the flat address of an LDS location = its LDS offset (the
  // shared aperture base has a zero low word); no address-space cast needed
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_wave_base);
  // the base must live in SGPRs for the SADDR form: make its uniformity explicit
  // (readfirstlane returns int: go through uint32_t so the low word is not sign-extended)
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)base);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
  const uint64_t sbase = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}

// 8 e4m3 codes (two dwords) -> 8 bf16
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(u32x2 w) {
  bf16x2 a = e4m3x2_to_bf16x2<false>(w[0]);
  bf16x2 b = e4m3x2_to_bf16x2<true>(w[0]);
  bf16x2 c = e4m3x2_to_bf16x2<false>(w[1]);
  bf16x2 d = e4m3x2_to_bf16x2<true>(w[1]);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2;

}  // namespace pkv
