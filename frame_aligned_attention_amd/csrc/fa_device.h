// fa_device.h -- device helpers shared by the gfx950 attention kernels.
#pragma once

#include "fa_internal.h"

namespace fa {

typedef __attribute__((address_space(3))) char lds_char;

// The block map is read-only for the kernel's lifetime: reading it through the constant
// address space turns its loads into scalar (SMEM) loads.  Vector loads would share the
// in-order VMEM counter with the tile prefetches, and every wait on them would also wait
// for the prefetch in flight.
typedef __attribute__((address_space(4))) const DevRange cRange;
typedef __attribute__((address_space(4))) const DevTile cTile;
typedef __attribute__((address_space(4))) const DevWork cWork;
typedef __attribute__((address_space(4))) const float cFloat;

// Copies a block-map record out of the constant address space, word by word.
template <typename T, typename CT>
__device__ __forceinline__ T cload(const CT *p) {
  static_assert(sizeof(T) % 4 == 0, "block-map records are whole words");
  typedef __attribute__((address_space(4))) const int cint;
  const cint *q = (const cint *)p;
  T v;
  int *d = (int *)&v;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 4); ++i) d[i] = q[i];
  return v;
}

// Raw buffer descriptor word 3 for gfx9-family loads (32-bit data, no swizzle).
constexpr int kBufferFlags = 0x00020000;

// v_permlane32_swap with both operands = x leaves, in every lane, the pair
// (x of lane l%32, x of lane 32 + l%32).
__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// v_permlane16_swap with both operands = x: lanes l and l ^ 16 (within each half) exchange.
__device__ __forceinline__ float x16_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float x16_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Uniform 64-bit address and size -> buffer descriptor kept in SGPRs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(uint64_t base, int bytes) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
  const int num = __builtin_amdgcn_readfirstlane(bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void *)(((uint64_t)hi << 32) | lo), (short)0, num,
                                           kBufferFlags);
}

}  // namespace fa
