// Library-level entry points of libspecverify: status strings, version, and a
// plain HBM read probe used to state the measured read peak next to the
// roofline fractions of the verify-pass kernels.
#include "sv_common.h"

namespace {

constexpr int kProbeBlocks = 2048;
constexpr int kProbeThreads = 256;

// Grid-stride 16-byte loads; the xor of everything read is written per
// workgroup so the loads cannot be elided.
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const sv_u32x4* __restrict__ src,
                                                                   size_t n16,
                                                                   uint32_t* __restrict__ sink) {
  // Each workgroup streams one contiguous share with non-temporal 16-byte
  // loads, eight in flight per lane -- the access pattern of the verify-pass
  // weight stream.
  unsigned int acc = 0;
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t lo = static_cast<size_t>(blockIdx.x) * per;
  const size_t hi = lo + per < n16 ? lo + per : n16;
  size_t i = lo + threadIdx.x;
  constexpr int U = 8;
  for (; i + (U - 1) * kProbeThreads < hi; i += U * kProbeThreads) {
    sv_u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * kProbeThreads);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < hi; i += kProbeThreads) {
    const sv_u32x4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  __shared__ unsigned int wacc[kProbeThreads / 64];
  if ((threadIdx.x & 63) == 0) wacc[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned int t = 0;
    for (int w = 0; w < kProbeThreads / 64; ++w) t ^= wacc[w];
    sink[blockIdx.x] = t;
  }
}

}  // namespace

extern "C" const char* sv_status_str(sv_status status) {
  switch (status) {
    case SV_OK: return "SV_OK";
    case SV_ERR_NULL: return "SV_ERR_NULL";
    case SV_ERR_INVALID_ARG: return "SV_ERR_INVALID_ARG";
    case SV_ERR_ALIGN: return "SV_ERR_ALIGN";
    case SV_ERR_UNSUPPORTED: return "SV_ERR_UNSUPPORTED";
    case SV_ERR_WORKSPACE: return "SV_ERR_WORKSPACE";
    case SV_ERR_HIP: return "SV_ERR_HIP";
  }
  return "SV_ERR_UNKNOWN";
}

extern "C" int sv_version(void) { return 200; }  // 0.2.0: chains, plan status

extern "C" int sv_read_probe_sink_words(void) { return kProbeBlocks; }

extern "C" sv_status sv_read_bandwidth_probe(const void* src, size_t bytes, uint32_t* sink,
                                             hipStream_t stream) {
  if (!src || !sink) return SV_ERR_NULL;
  if (bytes == 0 || bytes % 16 != 0) return SV_ERR_INVALID_ARG;
  if (!sv_aligned16(src) || !sv_aligned16(sink)) return SV_ERR_ALIGN;
  hipLaunchKernelGGL(read_probe_kernel, dim3(kProbeBlocks), dim3(kProbeThreads), 0, stream,
                     static_cast<const sv_u32x4*>(src), bytes / 16, sink);
  SV_LAUNCH_CHECK();
  return SV_OK;
}
