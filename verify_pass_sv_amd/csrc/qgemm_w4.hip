// sv_qgemm_w4: dequant-fused skinny GEMM over 4-bit asymmetric group-quantized
// weights, Y[r, n] = sum_k X[r, k] (C[n, k] - Z[n, g]) S[n, g], g = k / 64,
// on the row-major codes / scales / zeros of the contract.
//
// Source: Karpathy's Trick for Faster Local LLMs, "How Uzu optimizes bytes and
// tokens per pass" (Medium tier = 4-bit asymmetric integer quantization, one
// scale per group) and "Why batch-one decoding is memory-bound" (every weight
// is streamed once per pass); Speculative Decoding Clearly Explained, "Check
// the guesses together" (all draft positions scored in one pass).
//
// K % 512 == 0 (the common case): the streaming kernel of
// sv_qgemm_w4_packed in its row-major mode (qgemm_w4_packed.hip): activations
// staged once per workgroup in LDS for T consecutive 16-channel tiles, weight
// chunks in flight through a ring of LDS / register slots, one 16-byte load
// per lane and k block straight from the row-major codes, made into MFMA
// operands by one lane swap.
// Other K (a multiple of 64) take the plain kernel below.
//
// Plain kernel:
//  * One workgroup owns 16 output channels; its waves split K.  Every code
//    byte is loaded exactly once (8 bytes per lane = one 64-wide group of one
//    row across 4 lanes) and dequantized once for all m rows.
//  * The MFMA v_mfma_f32_16x16x32_bf16 takes A = activations (16 draft rows)
//    and B = weights (16 channels).  A nibble c becomes the exact bf16 value
//    128 + c with one byte permute and one and-or (0x4300 | c); the product
//    therefore carries 128 + c.  A second MFMA against an all-ones B gives the
//    group sums of X in exactly the accumulator layout, and the per-group fold
//        y += s * (acc - (128 + z) * xsum)
//    removes the bias and applies zero point and scale in binary32.  For
//    integer z and a one-hot activation row the result is exactly
//    (c - z) * s.
//  * Split-K partials of the waves are reduced through LDS in a fixed order,
//    so results are deterministic.
#include "w4_rowmajor.h"

namespace {

constexpr int kGroup = 64;

template <int MT, int W, bool VEC_SZ>
__global__ __launch_bounds__(64 * W) void qgemm_w4_kernel(
    const uint16_t* __restrict__ x, int m, int K, const uint8_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int N,
    float* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;  // weight channel within the tile / draft row of A
  const int q = lane >> 4;    // 16-wide slice of the 64-wide group
  const int n0 = blockIdx.x * 16;
  const int G = K / kGroup;

  // Groups handled by this wave: a multiple of 8 per wave when VEC_SZ.
  int gpw = (G + W - 1) / W;
  if (VEC_SZ) gpw = (gpw + 7) & ~7;
  const int gb = min(G, wave * gpw);
  const int ge = min(G, gb + gpw);

  const uint8_t* wrow = codes + (size_t)(n0 + col) * (size_t)(K / 2) + q * 8;
  const uint16_t* srow = scales + (size_t)(n0 + col) * G;
  const uint16_t* zrow = zeros + (size_t)(n0 + col) * G;

  // A-operand rows beyond m read row 0: they only feed output rows that are
  // never stored, so no zero padding (and no divergent branch) is needed.
  const uint16_t* xrow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int r = col + 16 * t;
    xrow[t] = x + (size_t)(r < m ? r : 0) * K + q * 16;
  }
  const unsigned int magic = sv_opaque_u32(0x43004300u);

  const sv_u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const sv_f32x4 fzero = {0.f, 0.f, 0.f, 0.f};
  sv_f32x4 yacc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) yacc[t] = fzero;

  // One group: dequantize the lane's 16 nibbles, two MFMAs against the
  // weights, two against all-ones, then fold bias, zero point and scale.
  auto do_group = [&](sv_u32x2 wv, float s, float zb, const sv_u32x4 (&xa)[MT][2]) {
    const sv_u32x4 b0 = sv_w4_dequant8_natural(wv.x, magic);
    const sv_u32x4 b1 = sv_w4_dequant8_natural(wv.y, magic);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      sv_f32x4 acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          sv_as_bf16x8(xa[t][0]), sv_as_bf16x8(b0), fzero, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sv_as_bf16x8(xa[t][1]), sv_as_bf16x8(b1),
                                                    acc, 0, 0, 0);
      sv_f32x4 xs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          sv_as_bf16x8(xa[t][0]), sv_as_bf16x8(ones), fzero, 0, 0, 0);
      xs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sv_as_bf16x8(xa[t][1]), sv_as_bf16x8(ones),
                                                   xs, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) yacc[t][i] = fmaf(s, fmaf(-zb, xs[i], acc[i]), yacc[t][i]);
    }
  };

  if (VEC_SZ) {
    // Batches of 8 groups: all code, scale, zero and activation loads of the
    // batch are issued before any of them is consumed.
    for (int g0 = gb; g0 < ge; g0 += 8) {
      const uint8_t* wb = wrow + (size_t)g0 * 32;
      sv_u32x2 wv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) wv[j] = sv_ld8(wb + j * 32);
      const sv_u32x4 sv = sv_ld16(srow + g0);
      const sv_u32x4 zv = sv_ld16(zrow + g0);
      sv_u32x4 xa[8][MT][2];
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const uint16_t* xp = xrow[t] + (size_t)g0 * kGroup + j * kGroup;
          xa[j][t][0] = sv_ld16(xp);
          xa[j][t][1] = sv_ld16(xp + 8);
        }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const unsigned int sw = sv[j >> 1], zw = zv[j >> 1];
        const float s = (j & 1) ? sv_half_hi(sw) : sv_half_lo(sw);
        const float zb = 128.0f + ((j & 1) ? sv_half_hi(zw) : sv_half_lo(zw));
        do_group(wv[j], s, zb, xa[j]);
      }
    }
  } else {
    for (int g = gb; g < ge; ++g) {
      const sv_u32x2 wv = sv_ld8(wrow + (size_t)g * 32);
      const float s = __half2float(__ushort_as_half(srow[g]));
      const float zb = 128.0f + __half2float(__ushort_as_half(zrow[g]));
      sv_u32x4 xa[MT][2];
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        xa[t][0] = sv_ld16(xrow[t] + (size_t)g * kGroup);
        xa[t][1] = sv_ld16(xrow[t] + (size_t)g * kGroup + 8);
      }
      do_group(wv, s, zb, xa);
    }
  }

  // Fixed-order reduction of the W split-K partials through LDS.
  __shared__ float red[W][MT][4][64];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][t][i][lane] = yacc[t][i];
  __syncthreads();
  for (int e = threadIdx.x; e < MT * 4 * 64; e += 64 * W) {
    const int t = e / 256, i = (e / 64) & 3, l = e & 63;
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) acc += red[w][t][i][l];
    const int r = 16 * t + 4 * (l >> 4) + i;
    if (r < m) y[(size_t)r * N + n0 + (l & 15)] = acc;
  }
}

template <int MT, int W>
void launch_w4(bool vec, dim3 grid, hipStream_t st, const uint16_t* x, int m, int K,
               const uint8_t* codes, const uint16_t* s, const uint16_t* z, int N, float* y) {
  if (vec)
    hipLaunchKernelGGL((qgemm_w4_kernel<MT, W, true>), grid, dim3(64 * W), 0, st, x, m, K,
                       codes, s, z, N, y);
  else
    hipLaunchKernelGGL((qgemm_w4_kernel<MT, W, false>), grid, dim3(64 * W), 0, st, x, m, K,
                       codes, s, z, N, y);
}




}  // namespace

extern "C" sv_status sv_qgemm_w4(const void* x, int m, int K, const uint8_t* codes,
                                 const void* scales, const void* zeros, int N, int group,
                                 float* y, hipStream_t stream) {
  if (!x || !codes || !scales || !zeros || !y) return SV_ERR_NULL;
  if (m < 1 || m > SV_MAX_ROWS || K < 64 || N < 16) return SV_ERR_INVALID_ARG;
  if (group != kGroup) return SV_ERR_UNSUPPORTED;
  if (K % kGroup != 0 || N % 16 != 0) return SV_ERR_INVALID_ARG;
  if (!sv_aligned16(x) || !sv_aligned16(codes) || !sv_aligned16(scales) ||
      !sv_aligned16(zeros) || !sv_aligned16(y))
    return SV_ERR_ALIGN;
  const int G = K / kGroup;
  const uint16_t* xs = static_cast<const uint16_t*>(x);
  const uint16_t* ss = static_cast<const uint16_t*>(scales);
  const uint16_t* zs = static_cast<const uint16_t*>(zeros);
  // Buffer-resource offsets are 32-bit: the streaming kernel takes matrices
  // of less than 2 GiB of codes (and activations of less than 2 GiB).
  if (K % 512 == 0 && static_cast<long long>(N) * K / 2 < (1LL << 31) &&
      static_cast<long long>(SV_MAX_ROWS) * K * 2 < (1LL << 31))
    return sv_w4_rowmajor_gemm(xs, m, K, codes, ss, zs, N, y, stream);
  const bool vec = (G % 8) == 0;
  const dim3 grid(N / 16);
  if (m <= 16)
    launch_w4<1, 8>(vec, grid, stream, xs, m, K, codes, ss, zs, N, y);
  else
    launch_w4<2, 8>(vec, grid, stream, xs, m, K, codes, ss, zs, N, y);
  SV_LAUNCH_CHECK();
  return SV_OK;
}
