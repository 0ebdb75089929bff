// Low-level building blocks shared by the grouped GEMM kernels (gfx950):
// explicit wait counts, direct global->LDS loads, streamed stores, a
// fence-free workgroup barrier and a compile-time loop.
#pragma once

#include <type_traits>

#include "device_common.hpp"

namespace fp8moe {

// s_waitcnt immediates (gfx9 encoding: vmcnt bits [3:0] and [15:14], expcnt [6:4],
// lgkmcnt [11:8]).  The builtin is visible to the compiler's own wait
// insertion, which then knows which direct-to-LDS loads have landed.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4)); }
template <int N>
__device__ __forceinline__ void wait_lgkmcnt() {
  static_assert(N >= 0 && N < 16, "lgkmcnt is 4 bits");
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (N << 8));
}

// Direct global->LDS loads (a wave fills 64 consecutive 16-byte or 1-byte LDS
// slots, one per lane, from per-lane global addresses).  Wrapped in plain
// device functions: clang drops a kernel's host launch stub when this builtin
// is called straight from a generic lambda in the kernel body.
__device__ __forceinline__ void dma_16(const uint8_t* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}
// A 1-byte DMA still gives each lane a dword of LDS: lane l's byte lands at dst + 4 l.
__device__ __forceinline__ void dma_1(const uint8_t* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 1, 0, 0);
}

// 16-byte store of output the kernel never reads back: streamed (non-temporal),
// so finished tiles do not displace operand lines in L2 and leave less dirty
// data behind for the kernels that follow.
__device__ __forceinline__ void store_stream16(uint8_t* dst, u32x4 v) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(v4u{v.x, v.y, v.z, v.w}, reinterpret_cast<v4u*>(dst));
}

// LDS accesses that the compiler's wait insertion does not see.  It cannot
// tell an LDS buffer apart from the direct-to-LDS loads in flight into other
// buffers, and before an ordinary LDS access it waits for all of them; with
// these the caller orders accesses itself: lds_wait() and then lds_ready() on
// each read result before it is used (the empty asm ties the result to the
// wait, so no use is scheduled above it).  Addresses are LDS byte offsets.
typedef unsigned int lds_u2 __attribute__((ext_vector_type(2)));
typedef unsigned int lds_u4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint32_t lds_off(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>(p);   // the low half of a shared-aperture address
}
__device__ __forceinline__ void lds_write8(uint32_t a, lds_u2 v) {
  asm volatile("ds_write_b64 %0, %1" ::"v"(a), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_write16(uint32_t a, lds_u4 v) {
  asm volatile("ds_write_b128 %0, %1" ::"v"(a), "v"(v) : "memory");
}
__device__ __forceinline__ uint32_t lds_read4(uint32_t a) {
  uint32_t r;
  asm volatile("ds_read_b32 %0, %1" : "=v"(r) : "v"(a) : "memory");
  return r;
}
__device__ __forceinline__ lds_u4 lds_read16(uint32_t a) {
  lds_u4 r;
  asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(a) : "memory");
  return r;
}
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
template <typename T>
__device__ __forceinline__ void lds_ready(T& r) {
  asm volatile("" : "+v"(r));
}

// Workgroup barrier without a memory fence (a fence would wait for every
// in-flight global load, draining the pipeline); the empty asm statements keep
// the compiler from moving memory accesses across it.
__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Calls f(integral_constant<int, I>) for I = 0 .. N-1 (compile-time indices
// for builtins that take immediates).
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// Place NM MFMAs of the current scheduling region with ND LDS reads and NV
// global loads spread evenly between them.
template <int NM, int ND, int NV, int I = 0>
__device__ __forceinline__ void interleave() {
  if constexpr (I < NM) {
    constexpr int d = ((I + 1) * ND) / NM - (I * ND) / NM;
    constexpr int v = ((I + 1) * NV) / NM - (I * NV) / NM;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (d > 0) __builtin_amdgcn_sched_group_barrier(0x100, d, 0);
    if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x020, v, 0);
    interleave<NM, ND, NV, I + 1>();
  }
}

}  // namespace fp8moe
