// sv_hadamard_i8: randomized block-diagonal Hadamard rotation + per-token
// symmetric int8 quantization of the activations.
//
// Source: Karpathy's Trick for Faster Local LLMs, "How Uzu optimizes bytes and
// tokens per pass": random sign flips, then mixing by a +-1 Hadamard matrix
// with one overall scale, each block on its own, exactly reversible; the
// activations are then quantized to 8 bits on the fly.  The pages' Apple
// kernel mixes 32-value blocks to match a 32-thread SIMD group; here the
// block is a parameter (up to 4096) and one workgroup owns one token row.
//
// Design: the row is staged in LDS as binary64 after the sign flip, an
// in-place fast Walsh-Hadamard transform (log2(block) butterfly stages, all
// blocks of the row at once) runs in binary64, and each value is rounded once
// to binary32 after the b^-1/2 scale.  The row maximum, the scale amax/127
// and the round-half-to-even decision are binary32.  Negligible bytes:
// latency-bound.
#include "sv_common.h"

namespace {

constexpr int kThreads = 512;
constexpr int kMaxK = 16384;
constexpr int kMaxPerThread = kMaxK / kThreads;

__global__ __launch_bounds__(kThreads) void hadamard_i8_kernel(
    const uint16_t* __restrict__ x, int K, const int8_t* __restrict__ signs, int block,
    int log2b, int8_t* __restrict__ xq, float* __restrict__ xscale) {
  extern __shared__ double buf[];  // K values
  __shared__ float wmax[kThreads / 64];
  const int r = blockIdx.x;
  const uint16_t* xr = x + (size_t)r * K;

  for (int i = threadIdx.x; i < K; i += kThreads) {
    const float v = __uint_as_float(static_cast<unsigned int>(xr[i]) << 16);
    buf[i] = static_cast<double>(v) * static_cast<double>(signs[i]);
  }
  __syncthreads();

  const int half = K >> 1;
  for (int s = 0; s < log2b; ++s) {
    const int h = 1 << s;
    for (int j = threadIdx.x; j < half; j += kThreads) {
      const int i = ((j >> s) << (s + 1)) | (j & (h - 1));
      const double a = buf[i], b = buf[i + h];
      buf[i] = a + b;
      buf[i + h] = a - b;
    }
    __syncthreads();
  }

  // Each thread keeps its own K / kThreads rotated values in registers.
  const double norm = sqrt(static_cast<double>(block));
  float vals[kMaxPerThread];
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxPerThread; ++j) {
    const int i = threadIdx.x + j * kThreads;
    vals[j] = 0.f;
    if (i < K) {
      vals[j] = static_cast<float>(buf[i] / norm);
      amax = fmaxf(amax, fabsf(vals[j]));
    }
  }
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
  __syncthreads();
  float rmax = 0.f;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) rmax = fmaxf(rmax, wmax[w]);
  const float scale = rmax > 0.f ? rmax / 127.0f : 1.0f;
  if (threadIdx.x == 0) xscale[r] = scale;

  int8_t* out = xq + (size_t)r * K;
#pragma unroll
  for (int j = 0; j < kMaxPerThread; ++j) {
    const int i = threadIdx.x + j * kThreads;
    if (i < K) {
      const float q = rintf(vals[j] / scale);
      out[i] = static_cast<int8_t>(fminf(127.f, fmaxf(-127.f, q)));
    }
  }
}

}  // namespace

extern "C" sv_status sv_hadamard_i8(const void* x, int m, int K, const int8_t* signs,
                                    int block, int8_t* xq, float* xscale, hipStream_t stream) {
  if (!x || !signs || !xq || !xscale) return SV_ERR_NULL;
  // one workgroup per row: any number of token rows (up to 2^20) in one call
  if (m < 1 || m > (1 << 20) || K < 64 || K % 64 != 0 || K > kMaxK) return SV_ERR_INVALID_ARG;
  if (block < 2 || block > 4096 || (block & (block - 1)) != 0 || K % block != 0)
    return SV_ERR_INVALID_ARG;
  if (!sv_aligned16(x) || !sv_aligned16(signs) || !sv_aligned16(xq) || !sv_aligned16(xscale))
    return SV_ERR_ALIGN;
  int log2b = 0;
  while ((1 << log2b) < block) ++log2b;
  const size_t lds = static_cast<size_t>(K) * sizeof(double);
  if (lds > 65536) {
    // Rows above 8192 values need more than the default 64 KiB of LDS
    // (gfx950 provides 160 KiB per workgroup).  Setting the attribute is
    // idempotent and allocates nothing.
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(hadamard_i8_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(kMaxK * sizeof(double))) != hipSuccess)
      return SV_ERR_HIP;
  }
  hipLaunchKernelGGL(hadamard_i8_kernel, dim3(m), dim3(kThreads), lds, stream,
                     static_cast<const uint16_t*>(x), K, signs, block, log2b, xq, xscale);
  SV_LAUNCH_CHECK();
  return SV_OK;
}
