// sv_qgemm_w8: skinny GEMM over 8-bit symmetric per-output-channel weights,
// Y[r, n] = S[n] * sum_k X[r, k] C[n, k].
//
// Source: Karpathy's Trick for Faster Local LLMs, "How Uzu optimizes bytes and
// tokens per pass" (Large tier = 8-bit symmetric quantization).
//
// The product runs on the streaming kernel of sv_qgemm_w4_packed in its
// 8-bit mode (qgemm_w4_packed.hip, sv_w8_rowmajor_gemm): activations staged
// once per workgroup in LDS for T consecutive 16-channel tiles, 512-wide
// chunks of 64-wide blocks through a ring of slots, each lane streaming its
// row's 16 code bytes of a block with one 128-bit load.  A code byte c
// becomes the exact bf16 value 128 + c (sign flip to an unsigned byte,
// v_cvt_f32_ubyte, upper half of the binary32 pattern); the MFMAs accumulate
// over the whole of K, a second MFMA against an all-ones operand accumulates
// sum_k X[r, k], and y = S[n] * (acc - 128 * xsum) once per channel.
#include "w4_rowmajor.h"

extern "C" sv_status sv_qgemm_w8(const void* x, int m, int K, const int8_t* codes,
                                 const void* scales, int N, float* y, hipStream_t stream) {
  if (!x || !codes || !scales || !y) return SV_ERR_NULL;
  if (m < 1 || m > SV_MAX_ROWS || K < 64 || N < 16) return SV_ERR_INVALID_ARG;
  if (K % 64 != 0 || N % 16 != 0) return SV_ERR_INVALID_ARG;
  if (!sv_aligned16(x) || !sv_aligned16(codes) || !sv_aligned16(scales) || !sv_aligned16(y))
    return SV_ERR_ALIGN;
  // Buffer-resource offsets are 32-bit: one matrix holds less than 2 GiB of
  // codes (and the activations less than 2 GiB).
  if (static_cast<long long>(N) * K >= (1LL << 31) ||
      static_cast<long long>(SV_MAX_ROWS) * K * 2 >= (1LL << 31))
    return SV_ERR_UNSUPPORTED;
  return sv_w8_rowmajor_gemm(static_cast<const uint16_t*>(x), m, K, codes,
                             static_cast<const uint16_t*>(scales), N, y, stream);
}
