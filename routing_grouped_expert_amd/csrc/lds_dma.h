// Direct-to-LDS loading on gfx950, shared by the MFMA kernels: buffer
// resources, 16-byte DMA loads straight into LDS, explicit vmcnt waits for
// them, and a workgroup barrier the scheduler cannot move work across.
// Internal to libmoe.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr uint32_t kOOB = 0x80000000u;  // buffer offset past every num_records used here
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, gfx9 family

// Workgroup barrier that also stops the scheduler from moving any instruction
// (MFMAs included) across it, so phases stay where the code puts them.
static __device__ __forceinline__ void barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// s_waitcnt vmcnt(N) lgkmcnt(0) (gfx9 encoding: vmcnt bits 3:0 and 15:14,
// expcnt 6:4 left at 7, lgkmcnt 11:8 = 0).
template <int N> static __device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Wait until at most P * PER + (st ? NST : 0) vector-memory operations are
// outstanding, for the largest P <= pend (pend <= PMAX).  PER is the number of
// load instructions per slice and NST the number of stores one epilogue
// issues; vmcnt counts loads and stores together and retires them in order.
// Counts above the 6-bit field wait for 63 instead (a stricter wait).
constexpr int vm_cap(int n) { return n > 63 ? 63 : n; }
template <int PER, int NST, int P>
static __device__ __forceinline__ void wait_pending(int pend, bool st) {
  if constexpr (P == 0) {
    if (st) wait_vm<vm_cap(NST)>(); else wait_vm<0>();
  } else {
    if (pend >= P) {
      if (st) wait_vm<vm_cap(P * PER + NST)>(); else wait_vm<vm_cap(P * PER)>();
    } else {
      wait_pending<PER, NST, P - 1>(pend, st);
    }
  }
}

// 16 bytes per lane from buffer `r` at byte offset `voff` into LDS at
// lds + 16 * lane (lds must be the same for the whole wave).  Issued as inline
// asm so the compiler does not track the LDS write: left to itself it waits for
// every outstanding load before any LDS read, which would serialise the ring.
// The waits for these loads are the explicit wait_pending<> calls.
static __device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, char *lds, uint32_t voff) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(void __attribute__((address_space(3))) *)lds;
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane(m0))
      : "memory", "m0");
}

// dma16 to LDS byte address `lds` (wave-uniform) with a wave-uniform byte
// offset added to voff in the scalar offset field: no pointer conversion and
// no per-lane add for a slice's position along K.
static __device__ __forceinline__ void dma16a(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t voff,
                                              uint32_t soff) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "buffer_load_dwordx4 %0, %1, %3 offen lds"
      :
      : "v"(voff), "s"(r), "s"(lds), "s"(soff)
      : "memory", "m0");
}

// LDS byte address of a pointer into LDS.
static __device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const void __attribute__((address_space(3))) *)p;
}

// dma16 with the non-temporal cache policy, for operands streamed once.
static __device__ __forceinline__ void dma16_nt(__amdgpu_buffer_rsrc_t r, char *lds, uint32_t voff) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(void __attribute__((address_space(3))) *)lds;
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen nt lds"
      :
      : "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane(m0))
      : "memory", "m0");
}

// 4 bytes per lane from buffer `r` at byte offset `voff` into LDS at
// lds + 4 * lane (same rules as dma16).
static __device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, char *lds, uint32_t voff) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(void __attribute__((address_space(3))) *)lds;
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "buffer_load_dword %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane(m0))
      : "memory", "m0");
}

}  // namespace moe
