// Device helpers shared by the attention kernels (gfx950): vector types, the
// lane exchanges of a 64-lane wavefront, bf16 packing, LDS transpose reads,
// direct global-to-LDS buffer loads and the waits and barrier around them.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// Both halves of the wavefront end up with f(x_lo, x_hi) for the lane pair (l, l^32).
__device__ inline float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

__device__ inline u32x2_t lds_tr_read(const unsigned char* base, int off) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(base + off));
  return __builtin_bit_cast(u32x2_t, v);
}

// Range check of the buffer loads below: a lane whose vector offset (plus the
// instruction's immediate offset) lies at or past num_records reads zeros.
// Callers pass every variable offset as the vector offset and keep the scalar
// offset at zero, since the range check is not specified to include it.

// 4 bytes per lane from a buffer straight into LDS (buffer_load_dword ... lds):
// lane L's bytes land at lds + 4·L.
__device__ inline void load_lds4(__amdgpu_buffer_rsrc_t r, void* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, voff, 0, 0, 0);
}

// 16 bytes per lane from a buffer straight into LDS (buffer_load_dwordx4 ... lds):
// lane L's bytes [voff, +16) land at lds + 16·L (lds uniform across the
// wavefront).  Kept in a
// non-template function: used directly inside the kernel template, the
// builtin makes the host pass drop the kernel's launch stub.
__device__ inline void load_lds16(__amdgpu_buffer_rsrc_t r, void* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

// Raw buffer descriptor over `bytes` bytes at `base` (word 3: 32-bit data, no swizzle).
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// s_waitcnt that waits until at most n vector-memory loads are outstanding
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at max).
template <int n>
__device__ inline void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without a memory fence: __syncthreads() orders all memory
// and therefore waits for every outstanding load, including the direct-to-LDS
// loads of tiles that are not needed yet.  LDS written by those loads is read
// only after the writer's own s_waitcnt and this barrier; the empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ inline void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads are done
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace fa
