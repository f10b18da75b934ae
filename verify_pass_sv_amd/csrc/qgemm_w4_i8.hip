// sv_qgemm_w4_i8: the int8 matrix path -- int8 activations times 4-bit
// asymmetric weights with exact int32 per-group partials,
//   Y[r, n] = xscale[r] * sum_g S[n, g] * (I[r, n, g] - Z[n, g] * Xg[r, g]).
//
// Source: Local LLM 4x Faster (the 4-bit checkpoint runs on the GPU's int8
// matrix path); Karpathy's Trick for Faster Local LLMs, "How Uzu optimizes
// bytes and tokens per pass" (activations quantized to 8 bits on the fly so
// both operands of each matrix multiplication are integers).
//
// Design: the gfx950 v_mfma_i32_16x16x64_i8 has a K depth of 64 -- exactly
// one quantization group -- so each group is one MFMA per 16x16 tile: A =
// 16 int8 activations per lane (one 128-bit load), B = the lane's 16 nibbles
// of one channel expanded to bytes 0..15 (one byte permute pair per dword).
// A second MFMA against all-ones bytes gives Xg in the accumulator layout.
// I and Xg are exact; the zero point and scale fold is binary32.
//
// With K % 512 == 0 the call runs the streaming kernel of
// sv_qgemm_w4_packed in its row-major int8 mode (qgemm_w4_packed.hip):
// activations staged once per workgroup in LDS for T consecutive 16-channel
// tiles, 1024-wide chunks through a ring of slots, the same per-group
// arithmetic.  Other K take the plain kernel below: one workgroup per 16
// channels, waves split K.
#include "w4_rowmajor.h"

namespace {

constexpr int kGroup = 64;

template <int MT, int W, bool VEC_SZ>
__global__ __launch_bounds__(64 * W) void qgemm_w4_i8_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ xscale, int m, int K,
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ zeros, int N, float* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int q = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int G = K / kGroup;
  int gpw = (G + W - 1) / W;
  if (VEC_SZ) gpw = (gpw + 7) & ~7;
  const int gb = min(G, wave * gpw);
  const int ge = min(G, gb + gpw);

  const uint8_t* wrow = codes + (size_t)(n0 + col) * (size_t)(K / 2) + q * 8;
  const uint16_t* srow = scales + (size_t)(n0 + col) * G;
  const uint16_t* zrow = zeros + (size_t)(n0 + col) * G;
  const int8_t* xrow[MT];
  bool xok[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int r = col + 16 * t;
    xok[t] = r < m;
    xrow[t] = xq + (size_t)(xok[t] ? r : 0) * K + q * 16;
  }
  const sv_u32x4 ones = {0x01010101u, 0x01010101u, 0x01010101u, 0x01010101u};
  const sv_u32x4 zero4 = {0u, 0u, 0u, 0u};
  const sv_i32x4 izero = {0, 0, 0, 0};
  sv_f32x4 yacc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) yacc[t] = sv_f32x4{0.f, 0.f, 0.f, 0.f};

  auto do_group = [&](sv_u32x2 wv, float s, float z, int g) {
    const sv_u32x2 lo = sv_w4_expand8_natural(wv.x), hi = sv_w4_expand8_natural(wv.y);
    const sv_u32x4 bw = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const sv_u32x4 a = xok[t] ? sv_ld16(xrow[t] + (size_t)g * kGroup) : zero4;
      const sv_i32x4 acc =
          __builtin_amdgcn_mfma_i32_16x16x64_i8(sv_as_i32x4(a), sv_as_i32x4(bw), izero, 0, 0, 0);
      const sv_i32x4 xs =
          __builtin_amdgcn_mfma_i32_16x16x64_i8(sv_as_i32x4(a), sv_as_i32x4(ones), izero, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        yacc[t][i] = fmaf(s, fmaf(-z, static_cast<float>(xs[i]), static_cast<float>(acc[i])),
                          yacc[t][i]);
    }
  };

  if (VEC_SZ) {
    for (int g0 = gb; g0 < ge; g0 += 8) {
      sv_u32x2 wv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) wv[j] = sv_ld8(wrow + (size_t)(g0 + j) * 32);
      const sv_u32x4 sv = sv_ld16(srow + g0);
      const sv_u32x4 zv = sv_ld16(zrow + g0);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const unsigned int sw = sv[j >> 1], zw = zv[j >> 1];
        const float s = (j & 1) ? sv_half_hi(sw) : sv_half_lo(sw);
        const float z = (j & 1) ? sv_half_hi(zw) : sv_half_lo(zw);
        do_group(wv[j], s, z, g0 + j);
      }
    }
  } else {
    for (int g = gb; g < ge; ++g) {
      const sv_u32x2 wv = sv_ld8(wrow + (size_t)g * 32);
      do_group(wv, __half2float(__ushort_as_half(srow[g])),
               __half2float(__ushort_as_half(zrow[g])), g);
    }
  }

  __shared__ float red[W][MT][4][64];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][t][i][lane] = yacc[t][i];
  __syncthreads();
  for (int e = threadIdx.x; e < MT * 4 * 64; e += 64 * W) {
    const int t = e / 256, i = (e / 64) & 3, l = e & 63;
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) a += red[w][t][i][l];
    const int r = 16 * t + 4 * (l >> 4) + i;
    if (r < m) y[(size_t)r * N + n0 + (l & 15)] = a * xscale[r];
  }
}

template <int MT, int W>
void launch_i8(bool vec, dim3 grid, hipStream_t st, const int8_t* xq, const float* xs, int m,
               int K, const uint8_t* codes, const uint16_t* s, const uint16_t* z, int N,
               float* y) {
  if (vec)
    hipLaunchKernelGGL((qgemm_w4_i8_kernel<MT, W, true>), grid, dim3(64 * W), 0, st, xq, xs, m,
                       K, codes, s, z, N, y);
  else
    hipLaunchKernelGGL((qgemm_w4_i8_kernel<MT, W, false>), grid, dim3(64 * W), 0, st, xq, xs,
                       m, K, codes, s, z, N, y);
}

}  // namespace

extern "C" sv_status sv_qgemm_w4_i8(const int8_t* xq, const float* xscale, int m, int K,
                                    const uint8_t* codes, const void* scales, const void* zeros,
                                    int N, int group, float* y, hipStream_t stream) {
  if (!xq || !xscale || !codes || !scales || !zeros || !y) return SV_ERR_NULL;
  if (m < 1 || m > SV_MAX_ROWS || K < 64 || N < 16) return SV_ERR_INVALID_ARG;
  if (group != kGroup) return SV_ERR_UNSUPPORTED;
  if (K % kGroup != 0 || N % 16 != 0) return SV_ERR_INVALID_ARG;
  if (!sv_aligned16(xq) || !sv_aligned16(xscale) || !sv_aligned16(codes) ||
      !sv_aligned16(scales) || !sv_aligned16(zeros) || !sv_aligned16(y))
    return SV_ERR_ALIGN;
  const bool vec = ((K / kGroup) % 8) == 0;
  const dim3 grid(N / 16);
  const uint16_t* ss = static_cast<const uint16_t*>(scales);
  const uint16_t* zs = static_cast<const uint16_t*>(zeros);
  // Buffer-resource offsets are 32-bit: the streaming kernel takes matrices
  // of less than 2 GiB of codes (and activations of less than 2 GiB).
  if (K % 512 == 0 && static_cast<long long>(N) * K / 2 < (1LL << 31) &&
      static_cast<long long>(SV_MAX_ROWS) * K < (1LL << 31))
    return sv_w4_i8_rowmajor_gemm(xq, xscale, m, K, codes, ss, zs, N, y, stream);
  if (m <= 16)
    launch_i8<1, 8>(vec, grid, stream, xq, xscale, m, K, codes, ss, zs, N, y);
  else
    launch_i8<2, 8>(vec, grid, stream, xq, xscale, m, K, codes, ss, zs, N, y);
  SV_LAUNCH_CHECK();
  return SV_OK;
}
