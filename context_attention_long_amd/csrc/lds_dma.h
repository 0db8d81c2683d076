// Direct global -> LDS loads for the gfx950 kernels.
//
// global_load_lds_dwordx4 writes each lane's 16 bytes to LDS at
// M0 + 16 * lane (layout verified on the hardware). It is issued from inline
// assembly on purpose: the compiler tracks its own LDS-DMA builtin as a
// write to all of LDS and then waits for every outstanding load (vmcnt(0))
// before any later LDS read, which serialises the prefetch of tile i+1 with
// the compute on tile i. Here the kernels wait themselves, with an explicit
// vmcnt count, before the barrier that publishes a tile.
//
// Mixing these loads with compiler-issued vector loads is safe: vector-memory
// loads complete in issue order, so loads added behind a compiler load can
// only make the compiler's own vmcnt waits stricter.
//
// Every statement sets M0 (the LDS destination) itself and lists it as
// clobbered, so the compiler never assumes M0 survives one of them. (M0 is
// a reserved register, for which clang warns that it will not save and
// restore it around the statement; nothing here needs it restored, so that
// warning is silenced for this header.)
#pragma once

#include <hip/hip_runtime.h>

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"

namespace cpa {

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// Cache policy of the loads. Stream = data read once per launch (a decode
// shard of the KV cache): the nontemporal hint, the encoding the compiler
// itself uses for __builtin_nontemporal_load; it raised the streaming rate of
// the decode loads from 5.3 to 6.1 TB/s. Reuse = tiles that many workgroups
// read again through L2 (prefill K/V): default policy.
enum class Policy { kReuse, kStream };

// One 16-byte load per lane into LDS at lds_base + 16 * lane. `lds_base` must
// be the same for the whole wavefront.
template <Policy P = Policy::kReuse>
__device__ __forceinline__ void lds_dma16(const void* gsrc, uint32_t lds_base) {
  if constexpr (P == Policy::kStream)
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt"
                 :
                 : "v"(gsrc), "s"(__builtin_amdgcn_readfirstlane(lds_base))
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(gsrc), "s"(__builtin_amdgcn_readfirstlane(lds_base))
                 : "memory", "m0");
}

// Same, addressed as a wavefront-uniform 64-bit base plus a per-lane 32-bit
// byte offset (the base goes to SGPRs, so stepping it costs no VALU work).
template <Policy P = Policy::kReuse>
__device__ __forceinline__ void lds_dma16_sbase(const void* sbase, uint32_t voff, uint32_t lds_base) {
  const uint64_t b = reinterpret_cast<uint64_t>(sbase);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32));
  const uint64_t sb = (static_cast<uint64_t>(hi) << 32) | lo;
  if constexpr (P == Policy::kStream)
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :
                 : "v"(voff), "s"(sb), "s"(__builtin_amdgcn_readfirstlane(lds_base))
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sb), "s"(__builtin_amdgcn_readfirstlane(lds_base))
                 : "memory", "m0");
}

// Same, with the base address and the LDS address already wavefront-uniform
// values (SGPRs): no per-call readfirstlane, so a burst of loads that share
// a base costs one SALU add per load.
template <Policy P = Policy::kReuse>
__device__ __forceinline__ void lds_dma16_s(uint64_t sbase, uint32_t voff, uint32_t lds_base) {
  if constexpr (P == Policy::kStream)
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" : : "v"(voff), "s"(sbase), "s"(lds_base) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "s"(lds_base) : "memory", "m0");
}

// Wavefront-uniform copy of a pointer (its SGPR form).
__device__ __forceinline__ uint64_t uniform_ptr(const void* p) {
  const uint64_t b = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// One 4-byte load per lane into LDS at lds_base + 4 * lane.
template <Policy P = Policy::kReuse>
__device__ __forceinline__ void lds_dma4(const void* gsrc, uint32_t lds_base) {
  if constexpr (P == Policy::kStream)
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off nt"
                 :
                 : "v"(gsrc), "s"(__builtin_amdgcn_readfirstlane(lds_base))
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
                 :
                 : "v"(gsrc), "s"(__builtin_amdgcn_readfirstlane(lds_base))
                 : "memory", "m0");
}

// Same, addressed as a wavefront-uniform base (SGPRs) plus a per-lane 32-bit
// byte offset.
template <Policy P = Policy::kReuse>
__device__ __forceinline__ void lds_dma4_s(uint64_t sbase, uint32_t voff, uint32_t lds_base) {
  if constexpr (P == Policy::kStream)
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1 nt" : : "v"(voff), "s"(sbase), "s"(lds_base) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" : : "v"(voff), "s"(sbase), "s"(lds_base) : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wavefront are
// outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

}  // namespace cpa

#pragma clang diagnostic pop
