// lds_dma.h -- gfx950 helpers for kernels that stream operand tiles from HBM
// straight into an LDS ring (buffer loads with the lds modifier), waiting on
// vmcnt explicitly and synchronising with a fence-free barrier. Internal to the
// library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef int int32x4 __attribute__((ext_vector_type(4)));

// Buffer resource for a raw byte range (stride 0, 32-bit data format); loads at
// offsets >= num_bytes return zero.
__device__ __forceinline__ int32x4 buffer_rsrc(const void* base, uint32_t num_bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  int32x4 r;
  r[0] = (int)(uint32_t)a;
  r[1] = (int)(uint32_t)((a >> 32) & 0xFFFFu);
  r[2] = (int)num_bytes;
  r[3] = 0x00020000;
  return r;
}

// Asynchronous 16-byte load straight into LDS: lane l of the wave writes bytes
// lds_base + 16*l .. +15. The load counts in vmcnt; it writes no VGPR, so nothing
// in registers can be clobbered while it is in flight.
__device__ __forceinline__ void load_to_lds(uint32_t lds_base, int voffset, const int32x4& rsrc, int soffset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_base), "v"(voffset), "s"(rsrc), "s"(soffset)
               : "memory", "m0");
}

// The same load with the non-temporal hint, for data that this workgroup alone
// reads once (a weight panel streamed by exactly one tile): the hint keeps it from
// displacing reused lines in the caches.
__device__ __forceinline__ void load_to_lds_nt(uint32_t lds_base, int voffset, const int32x4& rsrc, int soffset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
               :
               : "s"(lds_base), "v"(voffset), "s"(rsrc), "s"(soffset)
               : "memory", "m0");
}

// s_waitcnt vmcnt(N) (expcnt / lgkmcnt not waited).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// s_waitcnt lgkmcnt(0): this thread's LDS reads have returned.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Wait until at most rem * LD of this thread's loads are in flight (rem = tiles
// issued after the one about to be read, LD = loads per thread per tile).
template <int LD, int MAXREM>
__device__ __forceinline__ void wait_tiles(int rem) {
  static_assert(MAXREM * LD < 64, "vmcnt range");
  if constexpr (MAXREM >= 7) {
    if (rem >= 7) { wait_vmcnt<7 * LD>(); return; }
  }
  if constexpr (MAXREM >= 6) {
    if (rem >= 6) { wait_vmcnt<6 * LD>(); return; }
  }
  if constexpr (MAXREM >= 5) {
    if (rem >= 5) { wait_vmcnt<5 * LD>(); return; }
  }
  if constexpr (MAXREM >= 4) {
    if (rem >= 4) { wait_vmcnt<4 * LD>(); return; }
  }
  if constexpr (MAXREM >= 3) {
    if (rem >= 3) { wait_vmcnt<3 * LD>(); return; }
  }
  if constexpr (MAXREM >= 2) {
    if (rem >= 2) { wait_vmcnt<2 * LD>(); return; }
  }
  if constexpr (MAXREM >= 1) {
    if (rem >= 1) { wait_vmcnt<LD>(); return; }
  }
  wait_vmcnt<0>();
}

// Barrier without a memory fence (a fence would drain the in-flight prefetches);
// the empty asm statements keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS byte address of a __shared__ object, as the M0 base of load_to_lds.
template <typename T>
__device__ __forceinline__ uint32_t lds_address(T* p) {
  typedef __attribute__((address_space(3))) T lds_t;
  return (uint32_t)(uintptr_t)(lds_t*)(p);
}

}  // namespace moe
