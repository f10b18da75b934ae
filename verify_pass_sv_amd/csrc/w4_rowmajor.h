// Helpers shared by the single-GEMM sources for the row-major weights of
// sv_qgemm_w4 / sv_qgemm_w4_i8 (codes [N, K/2], byte i of a row = code 2i in
// the low nibble, code 2i + 1 in the high nibble; scales and zeros
// [N, K/64] f16) and of sv_qgemm_w8 (int8 codes [N, K], scales [N] f16).
#pragma once

#include "w4_packed_dev.h"

// Row-major word -> four bf16 pairs holding 128 + c in natural k order: one
// byte permute places the low and the high nibble of byte i in the two
// halves, one and-or keeps the nibbles and inserts the bf16 exponent pattern
// `magic` = 0x43004300 (value 128).
__device__ __forceinline__ sv_u32x4 sv_w4_dequant8_natural(unsigned int w, unsigned int magic) {
  const unsigned int u = w >> 4;
  sv_u32x4 o;
  o.x = (__builtin_amdgcn_perm(u, w, 0x0C040C00u) & 0x000F000Fu) | magic;
  o.y = (__builtin_amdgcn_perm(u, w, 0x0C050C01u) & 0x000F000Fu) | magic;
  o.z = (__builtin_amdgcn_perm(u, w, 0x0C060C02u) & 0x000F000Fu) | magic;
  o.w = (__builtin_amdgcn_perm(u, w, 0x0C070C03u) & 0x000F000Fu) | magic;
  return o;
}

// Row-major word (8 codes) -> 2 dwords of bytes c0 .. c7 (values 0..15).
__device__ __forceinline__ sv_u32x2 sv_w4_expand8_natural(unsigned int w) {
  const unsigned int u = w >> 4;
  sv_u32x2 r;
  r.x = __builtin_amdgcn_perm(u, w, 0x05010400u) & 0x0F0F0F0Fu;
  r.y = __builtin_amdgcn_perm(u, w, 0x07030602u) & 0x0F0F0F0Fu;
  return r;
}

// 4 int8 codes (one dword) -> 2 dwords of bf16 pairs holding 128 + c: the
// sign flip makes the unsigned byte 128 + c (1 .. 255), whose binary32 value
// v_cvt_f32_ubyte forms exactly and whose upper half is the exact bf16.
__device__ __forceinline__ sv_u32x2 sv_w8_cvt4_bias128(unsigned int d) {
  const unsigned int u = d ^ 0x80808080u;
  const unsigned int f0 = __float_as_uint(static_cast<float>(u & 0xFFu));
  const unsigned int f1 = __float_as_uint(static_cast<float>((u >> 8) & 0xFFu));
  const unsigned int f2 = __float_as_uint(static_cast<float>((u >> 16) & 0xFFu));
  const unsigned int f3 = __float_as_uint(static_cast<float>(u >> 24));
  sv_u32x2 r;
  r.x = __builtin_amdgcn_perm(f1, f0, 0x07060302u);
  r.y = __builtin_amdgcn_perm(f3, f2, 0x07060302u);
  return r;
}

// Host side: the streaming kernel of sv_qgemm_w4_packed run on the row-major
// codes, scales and zeros of sv_qgemm_w4 (m in 1..32, N % 16 == 0,
// K % 512 == 0, N * K / 2 < 2^31, all pointers 16-byte aligned; the caller
// checks).
__attribute__((visibility("hidden"))) sv_status sv_w4_rowmajor_gemm(
    const uint16_t* x, int m, int K, const uint8_t* codes, const uint16_t* scales,
    const uint16_t* zeros, int N, float* y, hipStream_t stream);

// The same kernel for sv_qgemm_w4_i8: int8 activations xq [m, K] with the
// per-row scale xscale [m] (same conditions).
__attribute__((visibility("hidden"))) sv_status sv_w4_i8_rowmajor_gemm(
    const int8_t* xq, const float* xscale, int m, int K, const uint8_t* codes,
    const uint16_t* scales, const uint16_t* zeros, int N, float* y, hipStream_t stream);

// The same kernel for sv_qgemm_w8: row-major int8 codes [N, K], one fp16
// scale per channel (m in 1..32, N % 16 == 0, K % 64 == 0, N * K < 2^31, all
// pointers 16-byte aligned; the caller checks).
__attribute__((visibility("hidden"))) sv_status sv_w8_rowmajor_gemm(
    const uint16_t* x, int m, int K, const int8_t* codes, const uint16_t* scales, int N,
    float* y, hipStream_t stream);
