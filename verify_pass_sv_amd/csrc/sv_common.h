// Internal helpers shared by the HIP sources of libspecverify (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "specverify.h"

// MFMA operand / accumulator vector types.
typedef __bf16 sv_bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float sv_f32x4 __attribute__((ext_vector_type(4)));
typedef int sv_i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int sv_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int sv_u32x2 __attribute__((ext_vector_type(2)));

#define SV_LAUNCH_CHECK()                                   \
  do {                                                      \
    if (hipGetLastError() != hipSuccess) return SV_ERR_HIP; \
  } while (0)

static inline bool sv_aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

// 16-byte global load into a 4-dword vector.
__device__ __forceinline__ sv_u32x4 sv_ld16(const void* p) {
  return *reinterpret_cast<const sv_u32x4*>(p);
}
__device__ __forceinline__ sv_u32x2 sv_ld8(const void* p) {
  return *reinterpret_cast<const sv_u32x2*>(p);
}

// bf16x8 MFMA operand from four packed dwords (bit reinterpretation only).
__device__ __forceinline__ sv_bf16x8 sv_as_bf16x8(sv_u32x4 v) {
  return __builtin_bit_cast(sv_bf16x8, v);
}
__device__ __forceinline__ sv_i32x4 sv_as_i32x4(sv_u32x4 v) {
  return __builtin_bit_cast(sv_i32x4, v);
}

// fp16 stored in the low or high half of a dword -> binary32.
__device__ __forceinline__ float sv_half_lo(unsigned int w) {
  return __half2float(__ushort_as_half(static_cast<unsigned short>(w & 0xFFFFu)));
}
__device__ __forceinline__ float sv_half_hi(unsigned int w) {
  return __half2float(__ushort_as_half(static_cast<unsigned short>(w >> 16)));
}
