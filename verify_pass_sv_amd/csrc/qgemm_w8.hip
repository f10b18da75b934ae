// sv_qgemm_w8: skinny GEMM over 8-bit symmetric per-output-channel weights,
// Y[r, n] = S[n] * sum_k X[r, k] C[n, k].
//
// Source: Karpathy's Trick for Faster Local LLMs, "How Uzu optimizes bytes and
// tokens per pass" (Large tier = 8-bit symmetric quantization).
//
// Design: one workgroup per 16 output channels, waves split K in 64-wide
// blocks; each lane streams 16 code bytes per block with one 128-bit load.
// A code byte c becomes the exact bf16 value 128 + c (sign flip to an
// unsigned byte, v_cvt_f32_ubyteN, upper half of the binary32 pattern); a
// second MFMA against an all-ones operand accumulates sum_k X[r, k], and the
// epilogue forms S[n] * (acc - 128 * xsum) once per channel.
#include "w4_rowmajor.h"

namespace {

template <int MT, int W>
__global__ __launch_bounds__(64 * W) void qgemm_w8_kernel(
    const uint16_t* __restrict__ x, int m, int K, const int8_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, int N, float* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int q = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int NB = K / 64;  // 64-wide blocks along K
  const int bpw = (NB + W - 1) / W;
  const int bb = min(NB, wave * bpw);
  const int be = min(NB, bb + bpw);

  const int8_t* wrow = codes + (size_t)(n0 + col) * K + q * 16;
  const uint16_t* xrow[MT];
  bool xok[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int r = col + 16 * t;
    xok[t] = r < m;
    xrow[t] = x + (size_t)(xok[t] ? r : 0) * K + q * 16;
  }
  const sv_u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const sv_u32x4 zero4 = {0u, 0u, 0u, 0u};
  const sv_f32x4 fzero = {0.f, 0.f, 0.f, 0.f};
  sv_f32x4 acc[MT], xs[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = xs[t] = fzero;

  constexpr int UNR = 4;
  for (int b0 = bb; b0 < be; b0 += UNR) {
    sv_u32x4 wv[UNR];
#pragma unroll
    for (int j = 0; j < UNR; ++j)
      wv[j] = (b0 + j < be) ? sv_ld16(wrow + (size_t)(b0 + j) * 64) : zero4;
#pragma unroll
    for (int j = 0; j < UNR; ++j) {
      if (b0 + j >= be) break;
      const sv_u32x2 p0 = sv_w8_cvt4_bias128(wv[j].x), p1 = sv_w8_cvt4_bias128(wv[j].y);
      const sv_u32x2 p2 = sv_w8_cvt4_bias128(wv[j].z), p3 = sv_w8_cvt4_bias128(wv[j].w);
      const sv_u32x4 bl = {p0.x, p0.y, p1.x, p1.y};
      const sv_u32x4 bh = {p2.x, p2.y, p3.x, p3.y};
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int kk = (b0 + j) * 64;
        const sv_u32x4 a0 = xok[t] ? sv_ld16(xrow[t] + kk) : zero4;
        const sv_u32x4 a1 = xok[t] ? sv_ld16(xrow[t] + kk + 8) : zero4;
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sv_as_bf16x8(a0), sv_as_bf16x8(bl),
                                                         acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sv_as_bf16x8(a1), sv_as_bf16x8(bh),
                                                         acc[t], 0, 0, 0);
        xs[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sv_as_bf16x8(a0), sv_as_bf16x8(ones),
                                                        xs[t], 0, 0, 0);
        xs[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sv_as_bf16x8(a1), sv_as_bf16x8(ones),
                                                        xs[t], 0, 0, 0);
      }
    }
  }

  __shared__ float red[W][MT][4][64];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][t][i][lane] = fmaf(-128.0f, xs[t][i], acc[t][i]);
  __syncthreads();
  for (int e = threadIdx.x; e < MT * 4 * 64; e += 64 * W) {
    const int t = e / 256, i = (e / 64) & 3, l = e & 63;
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) a += red[w][t][i][l];
    const int r = 16 * t + 4 * (l >> 4) + i;
    const int n = n0 + (l & 15);
    if (r < m) y[(size_t)r * N + n] = a * __half2float(__ushort_as_half(scales[n]));
  }
}

}  // namespace

extern "C" sv_status sv_qgemm_w8(const void* x, int m, int K, const int8_t* codes,
                                 const void* scales, int N, float* y, hipStream_t stream) {
  if (!x || !codes || !scales || !y) return SV_ERR_NULL;
  if (m < 1 || m > SV_MAX_ROWS || K < 64 || N < 16) return SV_ERR_INVALID_ARG;
  if (K % 64 != 0 || N % 16 != 0) return SV_ERR_INVALID_ARG;
  if (!sv_aligned16(x) || !sv_aligned16(codes) || !sv_aligned16(scales) || !sv_aligned16(y))
    return SV_ERR_ALIGN;
  const dim3 grid(N / 16);
  const uint16_t* xs = static_cast<const uint16_t*>(x);
  const uint16_t* ss = static_cast<const uint16_t*>(scales);
  // Buffer-resource offsets are 32-bit: the streaming kernel takes matrices
  // of less than 2 GiB of codes (and activations of less than 2 GiB).
  if (static_cast<long long>(N) * K < (1LL << 31) &&
      static_cast<long long>(SV_MAX_ROWS) * K * 2 < (1LL << 31))
    return sv_w8_rowmajor_gemm(xs, m, K, codes, ss, N, y, stream);
  if (m <= 16)
    hipLaunchKernelGGL((qgemm_w8_kernel<1, 8>), grid, dim3(512), 0, stream, xs, m, K, codes,
                       ss, N, y);
  else
    hipLaunchKernelGGL((qgemm_w8_kernel<2, 8>), grid, dim3(512), 0, stream, xs, m, K, codes,
                       ss, N, y);
  SV_LAUNCH_CHECK();
  return SV_OK;
}
