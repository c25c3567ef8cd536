// gdn_dma.h -- buffer resources, direct global-to-LDS transfers and related primitives
// (gfx950).
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace gdn {
namespace dma {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16;

template <typename T>
__device__ __forceinline__ uint32_t lds_addr(const T* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Raw buffer resource over [base, base + bytes): loads past the end return zero, stores past
// it are dropped.  All fields are workgroup-uniform.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));  // stride 0
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;  // 32-bit data format, no swizzle, no index
  return r;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t store_rsrc(void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from buffer offset voff + soff into LDS at lds + 16 * lane.  Issued as
// inline assembly: the compiler would otherwise make every later LDS read wait for it.
__device__ __forceinline__ void dma16(const i32x4& r, uint32_t voff, uint32_t soff,
                                      uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(r), "s"(soff)
               : "memory");
}

// 4 bytes per lane from buffer offset voff + soff into LDS at lds + 4 * lane.
__device__ __forceinline__ void dma4(const i32x4& r, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(r), "s"(soff)
               : "memory");
}

// Waits until at most N vector-memory instructions of this wave are outstanding.  Loads
// (direct-to-LDS ones included) complete in issue order among themselves, but stores count
// too and may complete out of that order, so a load is known complete once N is at most the
// number of loads issued after it; stores still pending only make the wait longer.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
  asm volatile("" : : : "memory");
}

// Waits for every vector-memory load of this wave, the direct-to-LDS ones included.  Issued
// through the builtin so the compiler's own wait tracking knows all loads have completed
// (an opaque inline-assembly wait would leave it inserting further waits for them).
__device__ __forceinline__ void wait_vm0() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt and lgkmcnt left alone
  asm volatile("" : : : "memory");
}

}  // namespace dma
}  // namespace gdn
