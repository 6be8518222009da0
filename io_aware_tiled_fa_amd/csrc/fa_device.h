// Device-side building blocks for the gfx950 (CDNA4) attention kernels:
// vector types, the bf16 matrix-core instructions, lane-layout facts of
// those instructions, cross-half lane exchange and LDS helpers.
//
// Lane layouts used throughout (checked on gfx950 hardware):
//  * v_mfma_f32_32x32x16_bf16, C[32x32] += A[32x16] * B[16x32], wave64:
//      A: lane l holds A[l % 32][8 * (l / 32) + e], e = 0..7
//      B: lane l holds B[8 * (l / 32) + e][l % 32], e = 0..7
//      C: lane l holds C[8 * (e / 4) + 4 * (l / 32) + e % 4][l % 32], e = 0..15
//    The contraction index only has to agree between A and B, so any
//    consistent relabelling of (l / 32, e) -> k gives the same product.
//  * ds_read_b64_tr_b16: in each group of 16 lanes, lane i receives element
//    (i % 4) of the 8-byte chunks read by lanes i/4, i/4 + 4, i/4 + 8 and
//    i/4 + 12 of its group (a 4 x 16 transpose of 16-bit values).
//  * v_permlane32_swap(a, b): swaps the upper 32 lanes of a with the lower
//    32 lanes of b; with a == b the pair holds (x[l], x[l ^ 32]) per lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_layout.h"

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// max(x[l], x[l ^ 32]) in every lane
__device__ __forceinline__ float max_cross_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}

// x[l] + x[l ^ 32] in every lane
__device__ __forceinline__ float sum_cross_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 b = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Buffer resource over `bytes` bytes from `base` (raw, untyped: the fourth
// descriptor word of the gfx9 family).  A load whose per-lane offset is at or
// past `bytes` reads zero and touches no memory.
typedef __amdgpu_buffer_rsrc_t buf_rsrc;
__device__ __forceinline__ buf_rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Buffer resource over the bytes [off, bytes) of the span at `base`, based
// at base + off: an empty one (every access reads zero) when off >= bytes.
// All arguments are wave-uniform, so this is a few scalar instructions; the
// kernels rebase their resources at each tile this way, which keeps a
// tile's per-lane offsets small and range-checked.
__device__ __forceinline__ buf_rsrc make_rsrc_at(const void* base, uint32_t bytes, uint32_t off) {
  // Both words are read back into scalar registers: the saturating
  // subtraction has no scalar instruction, and a 64-bit address product may
  // be formed by vector instructions; a resource the compiler finds in
  // vector registers is treated as per-lane, and every access through it
  // becomes a loop over the lanes' values.
  const uint64_t addr = reinterpret_cast<uint64_t>(static_cast<const char*>(base) + off);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)addr);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(addr >> 32));
  const uint32_t left = (uint32_t)__builtin_amdgcn_readfirstlane((int)(off < bytes ? bytes - off : 0u));
  return make_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo), left);
}

// 16-byte asynchronous copy global -> LDS through a buffer resource: lane l
// writes bytes [lds + 16 l, lds + 16 l + 16) from byte `voff` of the buffer.
// The range check of a raw buffer access compares only the per-lane offset
// (plus the instruction's immediate) with the resource's size; the scalar
// offset operand is added after the check.  So the whole offset goes into
// `voff` and the scalar operand is always 0: a row past the end of the
// buffer then reads zero instead of whatever memory follows it.  Unlike a
// flat copy this needs one VGPR per copy instead of a 64-bit address.
__device__ __forceinline__ void copy16_to_lds_buf(buf_rsrc r, uint32_t voff, lds_void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, voff, 0, 0, 0);
}

// wait until every outstanding vector-memory load of this wave has landed
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroup barrier without the memory fence of __syncthreads(): the fence
// makes the compiler wait for every outstanding vector-memory operation
// (prefetch copies) before the barrier; this one waits only for this wave's
// LDS writes (ds_write), which is what it publishes.  The empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), no vmcnt / expcnt wait
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ bf16x4 lds_read_tr16(const lds_char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
}

__device__ __forceinline__ bf16x8 lds_read16(const lds_char* p) { return *(const lds_bf16x8*)p; }

}  // namespace fa
