// lds_copy.hpp -- HBM -> LDS copies, LDS barriers and transposing LDS reads shared by the kernels that stage
// their input through LDS (gfx950).
#pragma once

#include "kvc_common.hpp"

namespace kvc {

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Buffer resource for the bytes [base, base + n): no stride, raw buffer, the same flags as
// __builtin_amdgcn_make_buffer_rsrc is given elsewhere.  Reads at offsets >= n return zeros.
__device__ inline i32x4_t buffer_rsrc(const void* base, int n) {
  const uint64_t p = (uint64_t)base;
  return i32x4_t{(int)(uint32_t)p, (int)((p >> 32) & 0xFFFFu), n, 0x00020000};
}
// One copy instruction HBM -> LDS: lane i's 16 (4) bytes at byte offset voff of the buffer go to LDS byte address
// lds + 16 i (4 i).  Written as assembly, not as the compiler builtin: the compiler treats every vector-typed LDS
// read after a builtin copy as possibly aliasing it and waits for all copies in flight (vmcnt(0)), which would
// empty a staging pipeline at every such read.  The caller waits for its own copies (s_waitcnt vmcnt) before it
// reads them, and the instruction writes no register.
__device__ inline void copy16_to_lds(i32x4_t rsrc, uint32_t lds, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
__device__ inline void copy4_to_lds(i32x4_t rsrc, uint32_t lds, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(lds), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Workgroup barrier for LDS data.  Copies write LDS directly and every wave waits for its own before the
// barrier, so the fences only keep the compiler from moving LDS accesses across it (a workgroup-scope fence
// would also wait for the copies still in flight).
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}
// the same within one wave
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Two transposing 8-byte LDS reads (ds_read_b64_tr_b16) as one fp16 operand.
__device__ inline h8 lds_tr8s(const void* p0, const void* p1) {
  typedef short s4_t __attribute__((ext_vector_type(4)));
  const h4 x = __builtin_bit_cast(h4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4_t*)p0));
  const h4 y = __builtin_bit_cast(h4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4_t*)p1));
  h8 r = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  return r;
}

}  // namespace kvc
