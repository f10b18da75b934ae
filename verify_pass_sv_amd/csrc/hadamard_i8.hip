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
// Design: one workgroup per token row.  The rotation is a fast
// Walsh-Hadamard transform (log2(block) butterfly stages) in binary64 after
// the sign flip; each value is rounded once to binary32 after the b^-1/2
// scale.  The row maximum, the scale amax/127 and the round-half-to-even
// decision are binary32.  Negligible bytes: latency-bound.
//   * block 4096 (the verify pass's block), calls of 256 rows or more: one
//     wave per 4096-wide block.  Each lane holds 64 contiguous values in
//     registers; the six stages with partners inside a lane run in
//     registers, a padded LDS transpose then gives each lane the values 64
//     apart, and the last six stages run in registers again.  No workgroup
//     barrier until the row maximum.
//   * block 4096, fewer rows (one link's k rows): four waves per block, 16
//     values per lane, two LDS transposes; a quarter of the serial
//     instruction stream per wave.
//   * other blocks: the row is staged in LDS and all blocks of the row are
//     transformed in place, stage by stage.
// Both orders of butterflies are the same, so both give identical binary64
// values.
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


// ---- block 4096: registers + one LDS transpose ---------------------------------
constexpr int kB4 = 4096;
// doubles per wave of transpose area: the transpose runs in two phases of 32
// publishing lanes (65 doubles each, padded), so a 4096-block holds 16.6 KB
// of LDS and two waves fit per SIMD
constexpr int kPadRow = 32 * 65;

__device__ __forceinline__ void bfly(double& a, double& b) {
  const double s = a + b, d = a - b;
  a = s;
  b = d;
}

__global__ __launch_bounds__(256) void hadamard4096_i8_kernel(
    const uint16_t* __restrict__ x, int K, const int8_t* __restrict__ signs,
    int8_t* __restrict__ xq, float* __restrict__ xscale) {
  extern __shared__ double tbuf[];               // kPadRow doubles per wave
  __shared__ float wmax[4];
  const int r = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;                // K / 4096 blocks in the row
  const int base = wv * kB4;

  // 64 contiguous values per lane (element 64 lane + i of the block)
  double v[64];
  {
    const uint16_t* xr = x + static_cast<size_t>(r) * K + base + lane * 64;
    const int8_t* sg = signs + base + lane * 64;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const sv_u32x4 w = sv_ld16(xr + 8 * t);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[8 * t + 2 * e] = static_cast<double>(__uint_as_float(w[e] << 16));
        v[8 * t + 2 * e + 1] = static_cast<double>(__uint_as_float(w[e] & 0xFFFF0000u));
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const sv_u32x4 sw = sv_ld16(sg + 16 * t);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int sgn = static_cast<int8_t>((sw[e >> 2] >> (8 * (e & 3))) & 0xFFu);
        v[16 * t + e] *= static_cast<double>(sgn);
      }
    }
  }
  // stages h = 1 .. 32: partners inside the lane
#pragma unroll
  for (int h = 1; h < 64; h <<= 1)
#pragma unroll
    for (int i = 0; i < 64; ++i)
      if ((i & h) == 0) bfly(v[i], v[i + h]);
  // transpose: lane L takes elements L + 64 j, held by lane j in register L.
  // Phase A: lanes 0..31 publish (slot 65 lane + i) and every lane reads
  // j < 32 into w; phase B: lanes 32..63 publish into the same slots and
  // every lane reads j >= 32.  LDS operations of a wave execute in order, so
  // a lane reads what other lanes wrote, and phase B's writes follow phase A's
  // reads; the compiler must only keep program order.
  double* tb = tbuf + wv * kPadRow;
  double w[32];
  if (lane < 32) {
#pragma unroll
    for (int i = 0; i < 64; ++i) tb[65 * lane + i] = v[i];
  }
  asm volatile("" ::: "memory");
#pragma unroll
  for (int j = 0; j < 32; ++j) w[j] = tb[lane + 65 * j];
  asm volatile("" ::: "memory");
  if (lane >= 32) {
#pragma unroll
    for (int i = 0; i < 64; ++i) tb[65 * (lane - 32) + i] = v[i];
  }
  asm volatile("" ::: "memory");
#pragma unroll
  for (int j = 0; j < 32; ++j) v[32 + j] = tb[lane + 65 * j];
#pragma unroll
  for (int j = 0; j < 32; ++j) v[j] = w[j];
  // stages h = 64 .. 2048: element lane + 64 j pairs with j ^ (h / 64)
#pragma unroll
  for (int hj = 1; hj < 64; hj <<= 1)
#pragma unroll
    for (int j = 0; j < 64; ++j)
      if ((j & hj) == 0) bfly(v[j], v[j + hj]);

  float f[64];
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 64; ++j) {
    f[j] = static_cast<float>(v[j] / 64.0);      // 4096^-1/2, exact
    amax = fmaxf(amax, fabsf(f[j]));
  }
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if (lane == 0) wmax[wv] = amax;
  __syncthreads();
  float rmax = 0.f;
  for (int w = 0; w < nw; ++w) rmax = fmaxf(rmax, wmax[w]);
  const float scale = rmax > 0.f ? rmax / 127.0f : 1.0f;
  if (threadIdx.x == 0) xscale[r] = scale;
  int8_t* out = xq + static_cast<size_t>(r) * K + base + lane;
#pragma unroll
  for (int j = 0; j < 64; ++j) {
    const float q = rintf(f[j] / scale);
    out[64 * j] = static_cast<int8_t>(fminf(127.f, fmaxf(-127.f, q)));
  }
}

// ---- block 4096, few rows: four waves per block ------------------------------
// The latency form, for calls with few rows (a verify pass rotating one
// link's k rows at a time): four waves per 4096-block, 16 values per lane.
// Stages h = 1..8 run in registers on the lane's 16 contiguous values; a
// padded LDS transpose gives each lane the 16 values of index bits 4-7
// (stages h = 16..128), a second one those of bits 8-11 (h = 256..2048).
// The stages run in the same ascending order on the same pairs as in the
// one-wave kernel, so every binary64 value and code is the same.
constexpr int kPadB = kB4 + kB4 / 16;             // doubles per block: one pad per 16
constexpr int kFewRows = 256;                     // calls below this many rows

__device__ __forceinline__ int padx(int e) { return e + (e >> 4); }

__global__ __launch_bounds__(1024) void hadamard4096x4_i8_kernel(
    const uint16_t* __restrict__ x, int K, const int8_t* __restrict__ signs,
    int8_t* __restrict__ xq, float* __restrict__ xscale) {
  extern __shared__ double tb4[];                // kPadB doubles per block
  __shared__ float wmax[16];
  const int r = blockIdx.x;
  const int t = threadIdx.x & 255;               // thread of the block
  const int base = (threadIdx.x >> 8) * kB4;     // the block's first element
  double* const tb = tb4 + (threadIdx.x >> 8) * kPadB;
  // element 16 t + i of the block
  double v[16];
  {
    const uint16_t* xr = x + static_cast<size_t>(r) * K + base + 16 * t;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const sv_u32x4 w = sv_ld16(xr + 8 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[8 * h + 2 * e] = static_cast<double>(__uint_as_float(w[e] << 16));
        v[8 * h + 2 * e + 1] = static_cast<double>(__uint_as_float(w[e] & 0xFFFF0000u));
      }
    }
    const sv_u32x4 sw = sv_ld16(signs + base + 16 * t);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int sgn = static_cast<int8_t>((sw[e >> 2] >> (8 * (e & 3))) & 0xFFu);
      v[e] *= static_cast<double>(sgn);
    }
  }
  // index bits 0-3
#pragma unroll
  for (int h = 1; h < 16; h <<= 1)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if ((i & h) == 0) bfly(v[i], v[i + h]);
  // transpose 1: thread t takes the elements ((t >> 4) << 8) | (j << 4) | (t & 15)
  const int e1 = ((t >> 4) << 8) | (t & 15);
#pragma unroll
  for (int i = 0; i < 16; ++i) tb[padx(16 * t + i)] = v[i];
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = tb[padx(e1 | (j << 4))];
  // index bits 4-7
#pragma unroll
  for (int h = 1; h < 16; h <<= 1)
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if ((j & h) == 0) bfly(v[j], v[j + h]);
  __syncthreads();                               // transpose 1 read everywhere
  // transpose 2: thread t takes the elements (j << 8) | t
#pragma unroll
  for (int j = 0; j < 16; ++j) tb[padx(e1 | (j << 4))] = v[j];
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = tb[padx((j << 8) | t)];
  // index bits 8-11
#pragma unroll
  for (int h = 1; h < 16; h <<= 1)
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if ((j & h) == 0) bfly(v[j], v[j + h]);

  float f[16];
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    f[j] = static_cast<float>(v[j] / 64.0);      // 4096^-1/2, exact
    amax = fmaxf(amax, fabsf(f[j]));
  }
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
  __syncthreads();
  float rmax = 0.f;
  const int nw = blockDim.x >> 6;
  for (int w = 0; w < nw; ++w) rmax = fmaxf(rmax, wmax[w]);
  const float scale = rmax > 0.f ? rmax / 127.0f : 1.0f;
  if (threadIdx.x == 0) xscale[r] = scale;
  int8_t* out = xq + static_cast<size_t>(r) * K + base + t;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float q = rintf(f[j] / scale);
    out[256 * j] = static_cast<int8_t>(fminf(127.f, fmaxf(-127.f, q)));
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
  if (block == kB4 && K % kB4 == 0 && m < kFewRows) {
    const int nb = K / kB4;                        // 1 to 4 blocks: 256 to 1024 threads
    const size_t lds = static_cast<size_t>(nb) * kPadB * sizeof(double);
    if (lds > 65536 &&
        hipFuncSetAttribute(reinterpret_cast<const void*>(hadamard4096x4_i8_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(4 * kPadB * sizeof(double))) != hipSuccess)
      return SV_ERR_HIP;
    hipLaunchKernelGGL(hadamard4096x4_i8_kernel, dim3(m), dim3(256 * nb), lds, stream,
                       static_cast<const uint16_t*>(x), K, signs, xq, xscale);
    SV_LAUNCH_CHECK();
    return SV_OK;
  }
  if (block == kB4 && K % kB4 == 0) {
    const int nw = K / kB4;
    const size_t lds4 = static_cast<size_t>(nw) * kPadRow * sizeof(double);
    if (lds4 > 65536 &&
        hipFuncSetAttribute(reinterpret_cast<const void*>(hadamard4096_i8_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(4 * kPadRow * sizeof(double))) != hipSuccess)
      return SV_ERR_HIP;
    hipLaunchKernelGGL(hadamard4096_i8_kernel, dim3(m), dim3(64 * nw), lds4, stream,
                       static_cast<const uint16_t*>(x), K, signs, xq, xscale);
    SV_LAUNCH_CHECK();
    return SV_OK;
  }
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
