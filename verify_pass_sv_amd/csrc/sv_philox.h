// Device Philox4x32-10 and the 24-bit uniforms drawn from it, shared by the
// accept kernels.
#pragma once

#include "sv_common.h"

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two 32x32
// multiplies with the published multipliers, key bumped by the published
// Weyl constants between rounds.
__device__ __forceinline__ void sv_philox_rounds(unsigned int c[4], unsigned int k0,
                                                 unsigned int k1) {
#pragma unroll
  for (int rnd = 0; rnd < 10; ++rnd) {
    const unsigned int lo0 = 0xD2511F53u * c[0];
    const unsigned int hi0 = __umulhi(0xD2511F53u, c[0]);
    const unsigned int lo1 = 0xCD9E8D57u * c[2];
    const unsigned int hi1 = __umulhi(0xCD9E8D57u, c[2]);
    const unsigned int n0 = hi1 ^ c[1] ^ k0;
    const unsigned int n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

__device__ __forceinline__ float sv_u24(unsigned int w) {
  return static_cast<float>(w >> 8) * (1.0f / 16777216.0f);
}

