// Device helpers shared by the kernels that stream the packed tile-major W4
// layout (sv_qgemm_w4_packed and the pass executor): nibble -> bf16
// conversion, LDS address-space casts and explicit wait/barrier primitives.
#pragma once

#include "sv_common.h"

typedef __attribute__((address_space(3))) void sv_lds_void;

// Index of the 1 KiB weight block (and of the scale/zero record) of 16-row
// tile t and k block j in the packed layouts.  Tiles are grouped by 32
// (512 output rows); inside a group the blocks of one k block are
// consecutive, so the 32 tiles of a work item read one contiguous range per
// k block.  The last group of a matrix may hold fewer than 32 tiles.
//   KB: k blocks per row (K/128 for 4-bit codes, K/64 for 8-bit codes)
__host__ __device__ __forceinline__ int sv_pk_block(int t, int j, int KB, int ntile) {
  const int g = t >> 5;
  const int gt = ntile - 32 * g < 32 ? ntile - 32 * g : 32;
  return 32 * g * KB + j * gt + (t & 31);
}

// A constant materialised in a VGPR by an opaque move, so the compiler keeps
// it in a register instead of folding it into every v_perm.
__device__ __forceinline__ unsigned int sv_opaque_u32(unsigned int v) {
  unsigned int r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(v));
  return r;
}

// A binary32 value the compiler must keep as it is: it cannot fold the
// conversion that produced it into its users.  On gfx950 v_fma_mix_f32 (an
// f16 operand converted inside the FMA) issues at half the rate of v_fma_f32,
// so a scale used by many FMAs is converted once instead.
__device__ __forceinline__ float sv_materialize(float v) {
  asm("" : "+v"(v));
  return v;
}

// Packed word (byte b = codes b | b+4 << 4) -> four bf16 pairs holding
// 128 + c in natural k order: a mask isolates the nibbles and one byte
// permute against the 0x43 exponent byte in `magic` makes bf16 0x43cc.
__device__ __forceinline__ sv_u32x4 sv_w4_dequant8(unsigned int w, unsigned int magic) {
  const unsigned int lo = w & 0x0F0F0F0Fu;          // codes 0..3
  const unsigned int hi = (w >> 4) & 0x0F0F0F0Fu;   // codes 4..7
  sv_u32x4 o;
  o.x = __builtin_amdgcn_perm(magic, lo, 0x04010400u);
  o.y = __builtin_amdgcn_perm(magic, lo, 0x04030402u);
  o.z = __builtin_amdgcn_perm(magic, hi, 0x04010400u);
  o.w = __builtin_amdgcn_perm(magic, hi, 0x04030402u);
  return o;
}

// Workgroup barrier without the memory fence of __syncthreads (which would
// wait for every outstanding global load); the "memory" clobber keeps the
// compiler from moving memory accesses across it.  LDS data written by
// buffer -> LDS loads is covered by an explicit vmcnt wait before it.
__device__ __forceinline__ void sv_barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

// Compiler-only ordering point for memory operations (emits nothing).
__device__ __forceinline__ void sv_compiler_fence() { asm volatile("" ::: "memory"); }

// s_waitcnt immediate (gfx9 encoding) waiting for vmcnt <= n only.  Vector
// memory loads and stores of one wave complete in issue order, so the count
// of operations issued after a given load is an exact bound.
template <int n>
__device__ __forceinline__ void sv_wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((n & 0xF) | (0x7 << 4) | (0xF << 8) | ((n >> 4) << 14));
}

// Buffer offsets at or above 2^31 fail the range check of every buffer used
// here (all hold less than 2 GiB), so a load reads nothing and a store
// writes nothing.  The check covers the per-lane (VGPR) offset, which is
// where this marker goes.
constexpr unsigned int kSvOutOfRange = 0x80000000u;
