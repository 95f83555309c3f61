// Global -> LDS copies (global_load_lds_dwordx4) and the waits and barriers
// the LDS-ring kernels build on, gfx950.
#pragma once
#include "common.hpp"

namespace moe {

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;

// 16 bytes from global memory to LDS; lane l of the wave lands at lds + 16 l.
__device__ __forceinline__ void dma16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((gbl_ptr_t)const_cast<void*>(src), (lds_ptr_t)lds_wave_base, 16, 0, 0);
}

// Buffer resource over [base, base + bytes) for raw (untyped) buffer loads;
// loads past `bytes` return zeros instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}

// 16 bytes from a buffer to LDS (buffer_load_dwordx4 ... lds): lane l reads
// the buffer at voff + soff (voff per lane, soff uniform) and lands at
// lds + 16 l.  The 32-bit offsets take no address arithmetic per copy.
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                          void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds_wave_base, 16, static_cast<int>(voff),
                                           static_cast<int>(soff), 0, 0);
}

// s_waitcnt vmcnt(N) (other counters left alone).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt vmcnt(N) lgkmcnt(0): this thread's LDS reads have returned and at
// most N of its global loads / LDS copies are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// s_waitcnt lgkmcnt(0): this thread's LDS accesses (and scalar loads) are done.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4)); }

// Workgroup barrier that waits for nothing but keeps the compiler from moving
// memory accesses across it (the LDS copies are waited for explicitly).
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// XOR swizzles of the 16-byte chunks of an LDS row by row index, for rows of
// 8 chunks (swz_a), 4 chunks (swz_b) and 16 chunks (swz_c): the 16 rows one
// MFMA operand read touches land in distinct bank groups.
__device__ __forceinline__ int swz_a(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int swz_b(int r) { return ((r >> 2) ^ (r >> 1)) & 3; }
__device__ __forceinline__ int swz_c(int r) { return r & 15; }

}  // namespace moe
