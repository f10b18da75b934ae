// sv_w4_pack + sv_qgemm_w4_packed: the verify GEMM over 4-bit asymmetric
// group-quantized weights stored in a tile-major layout made for gfx950 (and
// the streaming kernel of the single-GEMM entry points on row-major weights).
//
// Source: Karpathy's Trick for Faster Local LLMs, "How Uzu optimizes bytes and
// tokens per pass" (4-bit asymmetric integer quantization, one scale per
// group; checkpoint format and kernels designed together) and "Why batch-one
// decoding is memory-bound" (every weight streamed once per pass);
// Speculative Decoding Clearly Explained, "Check the guesses together".
//
// Packed layout (made once from the row-major codes by sv_w4_pack):
//   codes: one 1 KiB block per 16-row tile t and 128-wide k block j, at
//          byte sv_pk_block(t, j, K/128, N/16) * 1024 (tiles grouped by 32;
//          inside a group the blocks of one k block are consecutive).  Bytes
//          [16l, 16l+16) of the block belong to lane l of a wave: row
//          16t + (l & 15), slice q = l >> 4; bytes 0-7 hold the row's codes
//          for k = 128j + 16q + [0, 16), bytes 8-15 for k = 128j + 64 + 16q +
//          [0, 16).  Inside each 4-byte word covering k0..k0+7, byte b holds
//          code k0+b in its low nibble and code k0+b+4 in its high nibble, so
//          masking the low and the high nibbles yields codes in natural k
//          order.
//   sz:    a 128-byte record per (t, j) at sv_pk_block(t, j, K/128, N/16) *
//          128; row n of the tile owns 8 bytes [s(2j), z(2j), s(2j+1),
//          z(2j+1)] (fp16).
// A wave reads every code byte once with fully contiguous 1 KiB loads,
// already in the lane order of the MFMA B operand.
//
// Kernel design (one workgroup of 8 waves per T consecutive row tiles):
//  * Activations of each K chunk are copied once per workgroup into LDS by
//    asynchronous global->LDS loads (global_load_lds_dwordx4) into a double
//    buffer; all T tiles reuse them, so activation traffic per weight byte
//    is 4m / (16 T).  The row pitch is padded by 16 bytes so the MFMA
//    A-operand reads are bank-conflict free.
//  * Weights are read with buffer loads at scalar offsets, one chunk ahead
//    into a register double buffer, so HBM streams while a chunk computes.
//  * A nibble pair becomes two bf16 values 128 + c with a mask and one byte
//    permute against a 0x43 exponent byte (7 VALU per 8 weights).  The MFMA
//    v_mfma_f32_16x16x32_bf16 (A = 16 draft rows, B = 16 channels) forms
//    sum x (128 + c) per group for every tile before any of them is folded;
//    an MFMA against all-ones gives sum x once per group for all T tiles; the
//    fold  y += s * (acc - (128 + z) * xsum)  removes the bias and applies
//    zero point and scale in binary32 (exact (c - z) * s for a one-hot row
//    and integer z).
//  * Split-K partials of the 8 waves are summed through LDS in a fixed order.
//
// The same kernel serves the single-GEMM entry points on the row-major
// formats (see the kernel's RM, I8 and W8 notes):
//  * sv_qgemm_w4 (K % 512 == 0, sv_w4_rowmajor_gemm): each lane loads its 16
//    bytes of a row's k block directly and one lane swap turns them into
//    MFMA operands; scales and zeros are copied from their row-major arrays;
//  * sv_qgemm_w4_i8 (K % 512 == 0, sv_w4_i8_rowmajor_gemm): the same weights
//    against int8 activations, one v_mfma_i32_16x16x64_i8 per group;
//  * sv_qgemm_w8 (sv_w8_rowmajor_gemm): 8-bit codes in 64-wide blocks,
//    accumulated over the whole of K, one scale per channel.
#include "w4_rowmajor.h"

namespace {

constexpr int kGroup = 64;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kLdsBytes = 160 * 1024;  // gfx950 LDS per workgroup

// ---- packing ----------------------------------------------------------------
// Row-major word (byte i = codes 2i | 2i+1 << 4) -> packed word
// (byte b = codes b | b+4 << 4).
__device__ __forceinline__ unsigned int regroup8(unsigned int w) {
  unsigned int out = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const unsigned int c_lo = (w >> (4 * b)) & 0xFu;        // code b
    const unsigned int c_hi = (w >> (4 * (b + 4))) & 0xFu;  // code b + 4
    out |= (c_lo | (c_hi << 4)) << (8 * b);
  }
  return out;
}
__global__ void pack_codes_kernel(const uint8_t* __restrict__ codes, int N, int K,
                                  uint8_t* __restrict__ out) {
  const size_t piece = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int KB = K / 128;
  const size_t total = static_cast<size_t>(N / 16) * KB * 64;
  if (piece >= total) return;
  const int l = static_cast<int>(piece & 63);
  const size_t blk = piece >> 6;
  const int j = static_cast<int>(blk % KB);
  const int t = static_cast<int>(blk / KB);
  const int n = 16 * t + (l & 15), q = l >> 4;
  const uint8_t* row = codes + static_cast<size_t>(n) * (K / 2);
  const sv_u32x2 lo = sv_ld8(row + 64 * j + 8 * q);
  const sv_u32x2 hi = sv_ld8(row + 64 * j + 32 + 8 * q);
  sv_u32x4 v = {regroup8(lo.x), regroup8(lo.y), regroup8(hi.x), regroup8(hi.y)};
  const size_t dst = static_cast<size_t>(sv_pk_block(t, j, KB, N / 16)) * 1024 + l * 16;
  *reinterpret_cast<sv_u32x4*>(out + dst) = v;
}

__global__ void pack_sz_kernel(const uint16_t* __restrict__ scales,
                               const uint16_t* __restrict__ zeros, int N, int K,
                               uint16_t* __restrict__ out) {
  const size_t item = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int KB = K / 128, G = K / kGroup;
  const size_t total = static_cast<size_t>(N / 16) * KB * 16;
  if (item >= total) return;
  const int n16 = static_cast<int>(item & 15);
  const size_t blk = item >> 4;
  const int j = static_cast<int>(blk % KB);
  const int t = static_cast<int>(blk / KB);
  const size_t src = static_cast<size_t>(16 * t + n16) * G + 2 * j;
  uint16_t* o = out + static_cast<size_t>(sv_pk_block(t, j, KB, N / 16)) * 64 + n16 * 4;
  o[0] = scales[src];
  o[1] = zeros[src];
  o[2] = scales[src + 1];
  o[3] = zeros[src + 1];
}

// ---- GEMM ---------------------------------------------------------------------
// MT: 16-row activation tiles (m <= 16 * MT); T: row tiles per workgroup;
// PPW: 128-wide k blocks per wave per chunk (chunk = 8 * PPW * 128 k);
// P: pipeline slots (P - 1 chunks in flight while one computes).
// RM: the weights are the row-major codes / scales / zeros of sv_qgemm_w4
// (sz0 = scales, sz1 = zeros) instead of the packed layout (sz0 = records).
// I8 (with RM, for sv_qgemm_w4_i8): x is int8 [m, K] with a per-row scale
// xsc [m]; each group is one v_mfma_i32_16x16x64_i8 per tile (A = the lane's
// 16 activations, B = its 16 codes expanded to bytes), exact in int32, with
// the group sums Xg from an all-ones MFMA; the fold is
//     y += s * (I - z * Xg)   (binary32),  y *= xsc[r] at the end.
// W8 (with RM, for sv_qgemm_w8): row-major int8 codes [N, K] with one fp16
// scale per channel (sz0).  A k block is 64 wide (a lane's 16 codes, one
// 16-byte load), a chunk 512; a code c becomes bf16 128 + c through
// v_cvt_f32_ubyte; the MFMAs accumulate over the whole of K (no groups), an
// all-ones MFMA the row sums, and y = s * (acc - 128 xsum) at the end.
//  * Codes: lane l loads the 16 bytes 16q .. 16q + 15 (q = l >> 4) of row
//    16t + (l & 15)'s 64-byte block; lane q then holds codes k = 32q +
//    [0, 32) of the block, half a group.  One v_permlane32_swap per dword
//    pair trades the upper 8 bytes of lanes q = 0, 1 for the lower 8 bytes of
//    lanes q = 2, 3: every lane then holds 16 codes of each of the block's two
//    groups, at group offset oq = 32 (q & 1) + 16 (q >> 1) (16 q in the packed
//    layout), and reads its activation operand at the same offset.
//  * Scales and zeros of a chunk (16 groups x 16 rows = 512 bytes per tile
//    and array) come in by buffer -> LDS copies of 1 KiB that each take the
//    scales (or zeros) of two tiles.
template <int MT, int T, int PPW, int P, bool RM, bool I8, bool W8>
__global__ __launch_bounds__(kThreads) void qgemm_w4p_kernel(
    const void* __restrict__ x, const float* __restrict__ xsc, int m, int K,
    const uint8_t* __restrict__ pcodes, const uint16_t* __restrict__ sz0,
    const uint16_t* __restrict__ sz1, int N, float* __restrict__ y) {
  static_assert(RM || !I8, "int8 activations come with row-major weights");
  static_assert(RM || !W8, "8-bit weights are row-major");
  static_assert(!(I8 && W8), "one mode at a time");
  constexpr int XB = I8 ? 1 : 2;                  // bytes per activation
  constexpr int KBK = W8 ? 64 : 128;              // k per block (one 16-byte load per lane)
  constexpr int KC = PPW * KBK * kWaves;          // k per chunk
  constexpr int PITCHB = KC * XB + 16;            // bytes per LDS row (16-byte pad)
  constexpr int PITCH = PITCHB / 2;               // the same in 16-bit units
  constexpr int BUF = 16 * MT * PITCH;            // 16-bit units per LDS slot
  constexpr int SEGS = KC * XB / 1024;            // 1 KiB DMA pieces per row
  constexpr int D = 16 * MT * SEGS / kWaves;      // activation DMA pieces per wave per chunk
  // scale/zero copies of 1 KiB per chunk: one per tile (packed), one per
  // tile pair and array (row-major)
  constexpr int NSZ = W8 ? 0 : RM ? 2 * ((T + 1) / 2) : T;
  constexpr int DS = (NSZ + kWaves - 1) / kWaves; // scale/zero DMA pieces per wave per chunk
  constexpr int L = T * PPW + D + DS;             // loads per wave per chunk
  constexpr int SZB = W8 ? 0 : (NSZ + 1) * 512;   // u16 per LDS slot of scales/zeros: the
                                                  // copies plus 1 KiB that absorbs dummy loads
  static_assert(PPW == 1, "one 128-wide k block per wave per chunk");
  static_assert((16 * MT * SEGS) % kWaves == 0, "uneven DMA split");
  static_assert(P * (BUF + SZB) * 2 <= kLdsBytes, "pipeline slots do not fit LDS");
  static_assert(T * MT * 256 * kWaves * 4 <= kLdsBytes, "reduction does not fit LDS");
  static_assert(L * (P - 1) < 64, "too many loads in flight for vmcnt");
  extern __shared__ __align__(16) uint16_t lds[];

  const int lane = threadIdx.x & 63;
  // wave-uniform by construction; readfirstlane lets the compiler keep the
  // buffer offsets derived from it in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;
  const int q = lane >> 4;
  const int ntile = N / 16;
  const int t0 = blockIdx.x * T;
  const int KB = K / KBK;
  const int G = K / kGroup;
  const int nchunk = (K + KC - 1) / KC;
  const int oq = RM ? 32 * (q & 1) + 16 * (q >> 1) : 16 * q;  // group offset of the lane's codes
  const unsigned int magic = sv_opaque_u32(RM ? 0x43004300u : 0x43434343u);
  const sv_u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const sv_u32x4 ones8 = {0x01010101u, 0x01010101u, 0x01010101u, 0x01010101u};
  const sv_i32x4 izero = {0, 0, 0, 0};
  const sv_f32x4 fz = {0.f, 0.f, 0.f, 0.f};
  // N * K / 2 bytes of 4-bit codes in either layout, N * K of 8-bit ones
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(pcodes), 0, W8 ? N * K : N * (K / 2), 0x00020000);
  // packed records (N * K / 16 bytes), or the row-major scales (N * G * 2)
  const int szbytes = RM ? N * G * 2 : static_cast<int>(ntile * KB * 128u);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(sz0), 0, szbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t zrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(RM ? sz1 : sz0), 0, szbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(x), 0, m * K * XB, 0x00020000);

  sv_f32x4 yacc[T][MT];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int a = 0; a < MT; ++a) yacc[t][a] = fz;

  sv_u32x4 wb[P][T][PPW];
  // W8: row sums of the activations over all of K, per row tile
  sv_f32x4 xsacc[MT];
#pragma unroll
  for (int a = 0; a < MT; ++a) xsacc[a] = fz;
  uint16_t* const szl = lds + P * BUF;            // P slots of T KiB: scales/zeros

  // Issue all L loads of chunk c into slot `slot`: this wave's weight blocks
  // (registers), D pieces of the activation chunk and DS of the chunk's
  // scale/zero blocks (1 KiB per tile: 8 k blocks x 16 rows x 8 bytes, already
  // contiguous in the packed layout), both buffer -> LDS.  Every
  // load is a range-checked buffer load, so the count is the same for every
  // wave and step, including the steps past the last chunk, whose loads carry
  // an out-of-range offset and touch no memory (their register or LDS
  // destinations are never consumed).  That keeps the vmcnt waits exact.
  auto issue = [&](const int slot, int c) {
    const bool live = c < nchunk;
    const int jb = c * (KC / KBK) + wave * PPW;
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int p = 0; p < PPW; ++p) {
        const bool ok = live && (t0 + t < ntile) && (jb + p < KB);
        if constexpr (RM) {
          // row 16 (t0 + t) + col, bytes 16q .. 16q + 15 of its k block
          // (64 bytes per block and row in either width)
          const unsigned int off =
              ok ? static_cast<unsigned>(16 * (t0 + t) + col) *
                           static_cast<unsigned>(W8 ? K : K / 2) +
                       64u * (jb + p) + 16u * q
                 : kSvOutOfRange;
          wb[slot][t][p] = __builtin_amdgcn_raw_buffer_load_b128(wrs, off, 0, 0);
        } else {
          const int blk = ok ? sv_pk_block(t0 + t, jb + p, KB, ntile) : 0;
          wb[slot][t][p] = __builtin_amdgcn_raw_buffer_load_b128(
              wrs, ok ? lane * 16 : kSvOutOfRange, blk * 1024, 0);
        }
      }
#pragma unroll
    for (int i = 0; i < DS; ++i) {
      const int piece = wave + kWaves * i;        // this wave's copy (>= NSZ: dummy)
      if constexpr (RM) {
        // copy (tile pair piece / 2, scales if piece is even else zeros):
        // lane -> tile 2 (piece / 2) + lane / 32, row (lane / 2) % 16, groups
        // 16 c + 8 (lane % 2) .. + 7 of the chunk
        const int t = 2 * (piece >> 1) + (lane >> 5);
        const int gg = c * (KC / kGroup) + 8 * (lane & 1);
        const bool ok = live && piece < NSZ && t < T && (t0 + t < ntile) && gg < G;
        const unsigned int off =
            ok ? static_cast<unsigned>(((16 * (t0 + t) + ((lane >> 1) & 15)) * G + gg) * 2)
               : kSvOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            (piece & 1) ? zrs : srs,
            (sv_lds_void*)(szl + slot * SZB + (piece < NSZ ? piece : NSZ) * 512), 16, off, 0, 0, 0);
      } else {
        const int t = piece;                      // this piece's tile
        // lane -> k block c * 8 + lane / 8 of the tile, 16-byte piece lane % 8
        const int jj = c * (KC / 128) + (lane >> 3);
        const bool ok = live && t < T && (t0 + t < ntile) && jj < KB;
        const unsigned int off =
            ok ? sv_pk_block(t0 + t, jj, KB, ntile) * 128 + (lane & 7) * 16 : kSvOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            srs, (sv_lds_void*)(szl + slot * SZB + (t < T ? t : T) * 512), 16, off, 0, 0, 0);
      }
    }
    const int k0 = c * KC;
    uint16_t* dst = lds + slot * BUF;
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const int piece = wave + kWaves * i;
      const int r = piece / SEGS, seg = piece - r * SEGS;
      // rows >= m are not read (their LDS rows only feed discarded output
      // rows); lanes past K land in the next row (ignored) or fail the range
      // check past the end of x
      const unsigned int off =
          live && r < m ? (r * K + k0) * XB + seg * 1024 + lane * 16 : kSvOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (sv_lds_void*)(dst + r * PITCH + seg * 512), 16,
                                               off, 0, 0, 0);
    }
  };

  auto compute = [&](const int slot, int c) {
    const int jb = c * (KC / KBK) + wave * PPW;
    const uint16_t* buf = lds + slot * BUF;
    // this wave's k block inside the chunk is block `wave` of each tile's KiB
    // (packed); row-major: groups 2 wave, 2 wave + 1 of the lane's row in the
    // tile's scale and zero copies
    const uint16_t* szp = RM ? szl + slot * SZB + col * 16 + 2 * wave
                             : szl + slot * SZB + (wave * 16 + col) * 4;
#pragma unroll
    for (int p = 0; p < PPW; ++p) {
      if (jb + p >= KB) break;
      const int kl = (wave * PPW + p) * KBK;       // k offset inside the chunk
      if constexpr (RM && !W8) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
          sv_u32x4 v = wb[slot][t][p];
          const auto s0 = __builtin_amdgcn_permlane32_swap(v.x, v.z, false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(v.y, v.w, false, false);
          v.x = s0[0];
          v.z = s0[1];
          v.y = s1[0];
          v.w = s1[1];
          wb[slot][t][p] = v;
        }
      }
      if constexpr (I8) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {              // the two groups of the block
          const uint8_t* const xb = reinterpret_cast<const uint8_t*>(buf);
          sv_u32x4 a8[MT];
          sv_f32x4 xg[MT];
#pragma unroll
          for (int a = 0; a < MT; ++a) {
            a8[a] = *reinterpret_cast<const sv_u32x4*>(xb + (col + 16 * a) * PITCHB + kl +
                                                       64 * h + oq);
            // exact group sums Xg (all-ones B): lane (col, q) gets rows 4q .. 4q + 3
            const sv_i32x4 g = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                sv_as_i32x4(a8[a]), sv_as_i32x4(ones8), izero, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) xg[a][i] = static_cast<float>(g[i]);
          }
          sv_i32x4 acc[T][MT];
#pragma unroll
          for (int t = 0; t < T; ++t) {
            const sv_u32x4 w = wb[slot][t][p];
            const sv_u32x2 lo = sv_w4_expand8_natural(h ? w.z : w.x);
            const sv_u32x2 hi = sv_w4_expand8_natural(h ? w.w : w.y);
            const sv_u32x4 bw = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
            for (int a = 0; a < MT; ++a)
              acc[t][a] = __builtin_amdgcn_mfma_i32_16x16x64_i8(sv_as_i32x4(a8[a]),
                                                                sv_as_i32x4(bw), izero, 0, 0, 0);
          }
#pragma unroll
          for (int t = 0; t < T; ++t) {
            const uint16_t* sp = szp + (t >> 1) * 1024 + (t & 1) * 256;
            const unsigned int sw = *reinterpret_cast<const unsigned int*>(sp);
            const unsigned int zw = *reinterpret_cast<const unsigned int*>(sp + 512);
            const float sg = h ? sv_half_hi(sw) : sv_half_lo(sw);
            const float zg = h ? sv_half_hi(zw) : sv_half_lo(zw);
#pragma unroll
            for (int a = 0; a < MT; ++a)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                yacc[t][a][i] = fmaf(sg, fmaf(-zg, xg[a][i], static_cast<float>(acc[t][a][i])),
                                     yacc[t][a][i]);
          }
        }
      } else if constexpr (W8) {
        // one 64-wide block: the lane's codes 16q .. 16q + 15 against
        // activations 16q .. 16q + 15 (two MFMA k slices of 8)
        sv_u32x4 a0[MT], a1[MT];
#pragma unroll
        for (int a = 0; a < MT; ++a) {
          const uint16_t* ap = buf + (col + 16 * a) * PITCH + kl + 16 * q;
          a0[a] = *reinterpret_cast<const sv_u32x4*>(ap);
          a1[a] = *reinterpret_cast<const sv_u32x4*>(ap + 8);
          xsacc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sv_as_bf16x8(a0[a]),
                                                             sv_as_bf16x8(ones), xsacc[a], 0, 0, 0);
          xsacc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sv_as_bf16x8(a1[a]),
                                                             sv_as_bf16x8(ones), xsacc[a], 0, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const sv_u32x4 w = wb[slot][t][p];
          const sv_u32x2 c0 = sv_w8_cvt4_bias128(w.x), c1 = sv_w8_cvt4_bias128(w.y);
          const sv_u32x2 c2 = sv_w8_cvt4_bias128(w.z), c3 = sv_w8_cvt4_bias128(w.w);
          const sv_u32x4 b0 = {c0.x, c0.y, c1.x, c1.y};
          const sv_u32x4 b1 = {c2.x, c2.y, c3.x, c3.y};
#pragma unroll
          for (int a = 0; a < MT; ++a) {
            yacc[t][a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                sv_as_bf16x8(a0[a]), sv_as_bf16x8(b0), yacc[t][a], 0, 0, 0);
            yacc[t][a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                sv_as_bf16x8(a1[a]), sv_as_bf16x8(b1), yacc[t][a], 0, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {                // the two groups of the block
          sv_u32x4 a0[MT], a1[MT];
          sv_f32x4 xs[MT];
#pragma unroll
          for (int a = 0; a < MT; ++a) {
            const uint16_t* ap = buf + (col + 16 * a) * PITCH + kl + 64 * h + oq;
            a0[a] = *reinterpret_cast<const sv_u32x4*>(ap);
            a1[a] = *reinterpret_cast<const sv_u32x4*>(ap + 8);
            xs[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sv_as_bf16x8(a0[a]),
                                                            sv_as_bf16x8(ones), fz, 0, 0, 0);
            xs[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sv_as_bf16x8(a1[a]),
                                                            sv_as_bf16x8(ones), xs[a], 0, 0, 0);
          }
          sv_f32x4 acc[T][MT];
#pragma unroll
          for (int t = 0; t < T; ++t) {
            const sv_u32x4 w = wb[slot][t][p];
            const sv_u32x4 b0 = RM ? sv_w4_dequant8_natural(h ? w.z : w.x, magic)
                                   : sv_w4_dequant8(h ? w.z : w.x, magic);
            const sv_u32x4 b1 = RM ? sv_w4_dequant8_natural(h ? w.w : w.y, magic)
                                   : sv_w4_dequant8(h ? w.w : w.y, magic);
#pragma unroll
            for (int a = 0; a < MT; ++a) {
              acc[t][a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  sv_as_bf16x8(a0[a]), sv_as_bf16x8(b0), fz, 0, 0, 0);
              acc[t][a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  sv_as_bf16x8(a1[a]), sv_as_bf16x8(b1), acc[t][a], 0, 0, 0);
            }
          }
#pragma unroll
          for (int t = 0; t < T; ++t) {
            float s, zb;
            if constexpr (RM) {
              const uint16_t* sp = szp + (t >> 1) * 1024 + (t & 1) * 256;
              const unsigned int sw = *reinterpret_cast<const unsigned int*>(sp);
              const unsigned int zw = *reinterpret_cast<const unsigned int*>(sp + 512);
              s = h ? sv_half_hi(sw) : sv_half_lo(sw);
              zb = 128.0f + (h ? sv_half_hi(zw) : sv_half_lo(zw));
            } else {
              const sv_u32x2 sbt = *reinterpret_cast<const sv_u32x2*>(szp + t * 512);
              const unsigned int sz = h ? sbt.y : sbt.x;
              s = sv_half_lo(sz);
              zb = 128.0f + sv_half_hi(sz);
            }
#pragma unroll
            for (int a = 0; a < MT; ++a)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                yacc[t][a][i] = fmaf(s, fmaf(-zb, xs[a][i], acc[t][a][i]), yacc[t][a][i]);
          }
        }
      }
    }
  };

  // Ring of P slots: at step c the loads of chunks c+1 .. c+P-2 stay in
  // flight while this wave waits for chunk c; the barrier then publishes
  // chunk c's LDS data and guarantees every wave has finished chunk c-1, whose
  // slot the issue of chunk c+P-1 reuses.  Steps run in whole rounds of P so
  // every step issues and waits alike; only the compute is skipped past the
  // last chunk.
#pragma unroll
  for (int i = 0; i < P - 1; ++i) issue(i, i);
  for (int c0 = 0; c0 < nchunk; c0 += P) {
#pragma unroll
    for (int s = 0; s < P; ++s) {
      const int c = c0 + s;
      sv_wait_vmcnt<L * (P - 2)>();
      sv_barrier_no_fence();
      issue((s + P - 1) % P, c + P - 1);
      if (c < nchunk) compute(s, c);
    }
  }
  __syncthreads();

  // W8: the 128 bias of the codes leaves once, y = acc - 128 * xsum (the
  // channel scale is applied at the store)
  if constexpr (W8) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) yacc[t][a][i] = fmaf(-128.0f, xsacc[a][i], yacc[t][a][i]);
  }

  // Fixed-order reduction of the 8 waves' partials through LDS.
  float* red = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int a = 0; a < MT; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        red[(((wave * T + t) * MT + a) * 4 + i) * 64 + lane] = yacc[t][a][i];
  __syncthreads();
  for (int e = threadIdx.x; e < T * MT * 256; e += kThreads) {
    const int l = e & 63, i = (e >> 6) & 3, ta = e >> 8;
    const int t = ta / MT, a = ta - t * MT;
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) acc += red[(((w * T + t) * MT + a) * 4 + i) * 64 + l];
    const int r = 16 * a + 4 * (l >> 4) + i;
    const int n = 16 * (t0 + t) + (l & 15);
    if (r < m && t0 + t < ntile)
      y[static_cast<size_t>(r) * N + n] =
          W8 ? acc * sv_half_lo(sz0[n]) : I8 ? acc * xsc[r] : acc;
  }
}

template <int MT, int T, bool RM, bool I8, bool W8>
sv_status launch_packed(const void* x, const float* xsc, int m, int K, const uint8_t* pc,
                        const uint16_t* sz0, const uint16_t* sz1, int N, float* y,
                        hipStream_t st) {
  // Chunks of 1024 k; three LDS slots for m <= 16 (two chunks in flight),
  // two for m <= 32 (32 activation rows per slot).
  constexpr int PPW = 1;
  constexpr int P = MT == 1 ? 3 : 2;
  constexpr int NSZ = W8 ? 0 : RM ? 2 * ((T + 1) / 2) : T;
  auto kern = qgemm_w4p_kernel<MT, T, PPW, P, RM, I8, W8>;
  // LDS: P slots of activations + scales/zeros, reused for the final reduction.
  constexpr int kBuf = 16 * MT * ((PPW * (W8 ? 64 : 128) * kWaves * (I8 ? 1 : 2) + 16) / 2) +
                       (W8 ? 0 : (NSZ + 1) * 512);
  constexpr int kLds = (P * kBuf * 2 > T * MT * 256 * kWaves * 4) ? P * kBuf * 2
                                                                  : T * MT * 256 * kWaves * 4;
  const dim3 grid((N / 16 + T - 1) / T);
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kLds) != hipSuccess)
    return SV_ERR_HIP;
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), kLds, st, x, xsc, m, K, pc, sz0, sz1, N, y);
  SV_LAUNCH_CHECK();
  return SV_OK;
}

// Row tiles per workgroup: spread the N/16 tiles over at most 256
// workgroups (one per compute unit) so each reuses its staged activations
// across as many tiles as possible.
template <bool RM, bool I8, bool W8 = false>
sv_status dispatch(const void* x, const float* xsc, int m, int K, const uint8_t* pc,
                   const uint16_t* sz0, const uint16_t* sz1, int N, float* y, hipStream_t st) {
  const int T = (N / 16 + 255) / 256;
#define SV_LAUNCH_T(mt, t) \
  launch_packed<mt, t, RM, I8, W8>(x, xsc, m, K, pc, sz0, sz1, N, y, st)
  if (m <= 16) {
    if (T <= 1) return SV_LAUNCH_T(1, 1);
    if (T <= 2) return SV_LAUNCH_T(1, 2);
    if (T <= 3) return SV_LAUNCH_T(1, 3);
    if (T <= 4) return SV_LAUNCH_T(1, 4);
    return SV_LAUNCH_T(1, 6);
  }
  if (T <= 1) return SV_LAUNCH_T(2, 1);
  if (T <= 2) return SV_LAUNCH_T(2, 2);
  if (T <= 3) return SV_LAUNCH_T(2, 3);
  if (T <= 4) return SV_LAUNCH_T(2, 4);
  return SV_LAUNCH_T(2, 6);
#undef SV_LAUNCH_T
}

}  // namespace

extern "C" size_t sv_w4_packed_codes_bytes(int N, int K) {
  return static_cast<size_t>(N) * static_cast<size_t>(K) / 2;
}
extern "C" size_t sv_w4_packed_sz_bytes(int N, int K, int group) {
  return group > 0 ? static_cast<size_t>(N) * static_cast<size_t>(K / group) * 4 : 0;
}

extern "C" sv_status sv_w4_pack(const uint8_t* codes, const void* scales, const void* zeros,
                                int N, int K, int group, uint8_t* packed_codes,
                                void* packed_sz, hipStream_t stream) {
  if (!codes || !scales || !zeros || !packed_codes || !packed_sz) return SV_ERR_NULL;
  if (group != kGroup) return SV_ERR_UNSUPPORTED;
  if (N < 16 || N % 16 != 0 || K < 128 || K % 128 != 0) return SV_ERR_INVALID_ARG;
  if (!sv_aligned16(codes) || !sv_aligned16(scales) || !sv_aligned16(zeros) ||
      !sv_aligned16(packed_codes) || !sv_aligned16(packed_sz))
    return SV_ERR_ALIGN;
  const size_t pieces = static_cast<size_t>(N / 16) * (K / 128) * 64;
  const size_t items = static_cast<size_t>(N / 16) * (K / 128) * 16;
  hipLaunchKernelGGL(pack_codes_kernel, dim3(static_cast<unsigned>((pieces + 255) / 256)),
                     dim3(256), 0, stream, codes, N, K, packed_codes);
  SV_LAUNCH_CHECK();
  hipLaunchKernelGGL(pack_sz_kernel, dim3(static_cast<unsigned>((items + 255) / 256)), dim3(256),
                     0, stream, static_cast<const uint16_t*>(scales),
                     static_cast<const uint16_t*>(zeros), N, K,
                     static_cast<uint16_t*>(packed_sz));
  SV_LAUNCH_CHECK();
  return SV_OK;
}

extern "C" sv_status sv_qgemm_w4_packed(const void* x, int m, int K, const uint8_t* packed_codes,
                                        const void* packed_sz, int N, int group, float* y,
                                        hipStream_t stream) {
  if (!x || !packed_codes || !packed_sz || !y) return SV_ERR_NULL;
  if (m < 1 || m > SV_MAX_ROWS) return SV_ERR_INVALID_ARG;
  if (group != kGroup) return SV_ERR_UNSUPPORTED;
  if (N < 16 || N % 16 != 0 || K < 128 || K % 128 != 0) return SV_ERR_INVALID_ARG;
  // Buffer-resource offsets are 32-bit: one matrix holds less than 2 GiB of codes.
  if (static_cast<long long>(N) * K / 2 >= (1LL << 31)) return SV_ERR_UNSUPPORTED;
  if (!sv_aligned16(x) || !sv_aligned16(packed_codes) || !sv_aligned16(packed_sz) ||
      !sv_aligned16(y))
    return SV_ERR_ALIGN;
  const uint16_t* ps = static_cast<const uint16_t*>(packed_sz);
  return dispatch<false, false>(x, nullptr, m, K, packed_codes, ps, ps, N, y, stream);
}

sv_status sv_w4_rowmajor_gemm(const uint16_t* x, int m, int K, const uint8_t* codes,
                              const uint16_t* scales, const uint16_t* zeros, int N, float* y,
                              hipStream_t stream) {
  return dispatch<true, false>(x, nullptr, m, K, codes, scales, zeros, N, y, stream);
}

sv_status sv_w8_rowmajor_gemm(const uint16_t* x, int m, int K, const int8_t* codes,
                              const uint16_t* scales, int N, float* y, hipStream_t stream) {
  return dispatch<true, false, true>(x, nullptr, m, K, reinterpret_cast<const uint8_t*>(codes),
                                     scales, scales, N, y, stream);
}

sv_status sv_w4_i8_rowmajor_gemm(const int8_t* xq, const float* xscale, int m, int K,
                                 const uint8_t* codes, const uint16_t* scales,
                                 const uint16_t* zeros, int N, float* y, hipStream_t stream) {
  return dispatch<true, true>(xq, xscale, m, K, codes, scales, zeros, N, y, stream);
}
