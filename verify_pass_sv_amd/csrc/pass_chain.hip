// Verify pass in model order: a chain of W4 GEMMs run by one persistent
// launch, each GEMM complete before a later GEMM that reads its output starts.
//
// Source: Karpathy's Trick for Faster Local LLMs, "How Uzu optimizes bytes and
// tokens per pass" (a forward pass hands intermediate values from layer to
// layer) and "Why batch-one decoding is memory-bound" (the runtime reads the
// weight blocks of every layer once and computes the next-token scores);
// Speculative Decoding Clearly Explained, "Check the guesses together" (all
// draft positions are scored in that one pass).
//
// A chain is an ordered list of links.  Link i computes
//   y_i = x_i W_i^T     (f32 [m, N_i]; W4: 4-bit group-64 weights, W8: 8-bit
//                        codes with one scale per output channel)
// and, optionally, the input of a later link
//   xo_i = bf16_rne(alpha_i * y_i[:, :xo_cols_i])   (bf16 [m, xo_cols_i]).
// A link whose x is an earlier link's xo waits, at a device-wide phase
// barrier, until every earlier link is complete; any other link follows its
// predecessor without a barrier.  The weights do not depend on activations,
// so the weight stream runs ahead across barriers: only the activation loads
// and the arithmetic wait.
//
// Work split (every link spans the whole grid, one workgroup per compute
// unit): tile i (16 output channels) of a link belongs to workgroup i mod G.
// A link with more than 6 G tiles runs as several rounds of at most 6 tiles
// per workgroup.  Inside a workgroup the 8 stream waves split K: of the
// blocks of 128 k, wave j takes blocks j, j + 8, j + 16, .. for every tile of
// the round, so one activation operand (read once from LDS) feeds up to 6
// tiles.
// Partial sums of the 8 waves meet in LDS at the end of the round and are
// added in a fixed order (deterministic results).
//
// Wave roles:
//   * 8 stream waves: each streams its own operands -- the weight units of
//     its k-blocks (a register ring of 4 to 6 units of 1 KiB, its first units
//     issued before the round's barrier is passed) and the activation blocks
//     of the same k-blocks (buffer -> LDS loads into the wave's own ring of 2
//     blocks of 4 KiB, 8 KiB at m > 16), then dequantization, bf16
//     MFMAs, the per-group fold and zero-point correction, the reduction, and
//     the y and xo stores.  A wave reads no other wave's blocks, so nothing
//     synchronizes the waves inside a round, and each keeps its loads in
//     flight up to the exact count the next step needs.
//   * 1 IO wave: the phase barrier (arrive, bounded poll); its vector-memory
//     queue holds only the poll loads.
//
// Phase barrier: 16 counters (64-bit, 4 KiB apart); workgroup w adds 1 to
// counter w mod 16 after its part of a link that a waiting link follows, and
// a waiting workgroup polls all 16 (agent-scope loads) until each reaches its
// target.  Counters only grow; the launch index is recovered from the
// counter value at entry.  The xo data are written with agent-scope (sc1)
// stores and completed (s_waitcnt vmcnt(0)) before the arrival; consumers
// read them with plain loads, which is safe because no xo buffer is read
// before the link that writes it is complete (the plan checks that each xo
// is a whole number of 128-byte lines and is not read by an earlier link),
// and every workgroup invalidates its caches at entry (stale lines from an
// earlier launch).  A poll that exceeds its bound sets the plan's status word
// and the launch ends early.
//
// Arithmetic per 1 KiB unit (tile t, block b; the packed layout of
// sv_w4_pack): bf16 128 + c from a mask and a byte permute, two
// v_mfma_f32_16x16x32_bf16 per group give acc = sum x (128 + c), the fold
// t = s0 acc0 + s1 acc1, and the bias and zero point leave through one
// rank-2 v_mfma_f32_16x16x4_f32 update t -= sum_g xsum[r, g] s[n, g]
// (128 + z[n, g]) whose row sums come from all-ones MFMAs on the same
// activation operand.  For a one-hot row and integer z every step is exact.
//
// W8 (two 1 KiB units of 64 k per block, the layout of sv_w8_pack): bf16
// 128 + c by a sign flip and byte conversions, the MFMAs accumulate
// sum x (128 + c) over the whole round, all-ones MFMAs the row sums; each
// wave subtracts 128 times its row sums before the reduction, and the
// channel scale (loaded first in the round) multiplies the sum.
#include <algorithm>
#include <cstddef>
#include <type_traits>
#include <vector>

#include "w4_packed_dev.h"
#include "w4_rowmajor.h"

namespace {

constexpr uint32_t kChainMagic = 0x4F565653u;   // "SVVO"
constexpr uint32_t kChainVersion = 1;
constexpr int kSW = 8;                          // stream waves
constexpr int kThreadsC = 64 * (kSW + 1);       // + the IO wave
constexpr int kTmax = 6;                        // tile accumulators (switch cases)
// tiles per workgroup per round: 6 at m <= 16; 3 at m > 16, where the two
// row tiles double the accumulators and activation operands
__host__ __device__ constexpr int round_tiles(int mt) { return mt == 1 ? 6 : 3; }
constexpr int kNG = 16;                         // barrier counters
constexpr int kSyncStride = 4096;               // bytes between counters
constexpr int kMaxGridC = 1024;
constexpr int kSpinLimit = 1 << 20;             // polls before a barrier gives up (~1 s)
constexpr int kStreamC = 2;                     // non-temporal (weights, records, y)
constexpr int kSc1 = 16;                        // agent-scope coherent (xo stores)

constexpr uint32_t kFlagWait = 1;               // round waits for all earlier links
constexpr uint32_t kFlagSignal = 2;             // workgroups arrive after this round

struct ChainHeader {                            // 128 bytes
  uint32_t magic, version;
  int32_t format, m, grid, nrounds, nlinks, nsignals;
  int32_t spin_limit;                           // polls before a barrier gives up
  uint32_t reserved1;
  int32_t group_size[kNG];                      // workgroups per counter
  uint32_t pad[6];
};
struct ChainRound {                             // 128 bytes
  const uint8_t* codes;
  const void* sz;
  const void* x;
  float* y;
  void* xo;
  float alpha;
  int32_t K, N, xo_cols;
  int32_t tile0, ntiles;                        // tiles [tile0, tile0 + ntiles) of the link
  int32_t signal_index;                         // waiting rounds: arrivals to wait for (per launch)
  uint32_t flags;
  int32_t pad[14];
};
static_assert(sizeof(ChainHeader) == 128, "chain header layout");
static_assert(sizeof(ChainRound) == 128, "chain round layout");

constexpr size_t kRoundsOff = sizeof(ChainHeader);
__host__ __device__ inline size_t sync_off(int nrounds) {
  return (kRoundsOff + sizeof(ChainRound) * static_cast<size_t>(nrounds) + kSyncStride - 1) /
         kSyncStride * kSyncStride;
}
// Sync area: kNG barrier counters, then the status word, each on its own 4 KiB.
constexpr size_t kStatusOff = kNG * kSyncStride;
__host__ __device__ inline size_t chain_bytes(int nrounds) {
  return sync_off(nrounds) + (kNG + 1) * kSyncStride;
}

template <int MT>
struct ChainGeo {
  static constexpr int A = 2;                            // activation blocks per wave ring
  static constexpr int BLKB = 16 * MT * 256;             // bytes per block: 16 MT rows x 128 k
  static constexpr int BLOADS = BLKB / 1024;             // 1 KiB loads per block
  static constexpr int WAVEB = A * BLKB;                 // one wave's ring
  static constexpr int TPOSE = kSW * WAVEB;              // per-wave transposes (after the rings)
  static constexpr int LDS = TPOSE + kSW * 1024;
  static_assert(kSW * kTmax * MT * 1024 <= kSW * WAVEB, "reduction area fits the rings");
  static_assert(LDS <= 160 * 1024, "LDS budget of a gfx950 workgroup");
};

// Wave-uniform copies (scalar registers) of values the compiler cannot prove
// uniform: buffer descriptors built from them need no per-lane loop, and the
// loads of the plan they index go through the scalar cache.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
template <class T>
__device__ __forceinline__ T* uni(T* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint64_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(u)));
  const uint64_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(u >> 32)));
  return reinterpret_cast<T*>(lo | (hi << 32));
}

// 16 bytes per lane from a buffer into LDS (lane l -> lds + 16 l).  A plain
// device function: the builtin called from a lambda inside a generic lambda
// makes the host-side compile drop the kernel's launch stub.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t rs, uint8_t* lds_dst,
                                           unsigned int off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (sv_lds_void*)lds_dst, 16, off, 0, 0, 0);
}

__device__ __forceinline__ unsigned int bf16_rne(float f) {
  const unsigned int u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;   // NaN stays NaN
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int MT, int F>
// `plan` (header and rounds) is only read; `sync` (counters and status, at
// plan + sync_off(nrounds)) is written.  Kept as two restrict pointers so the
// plan's uniform fields load through the scalar cache.
__global__ __launch_bounds__(kThreadsC) void chain_kernel(const uint8_t* __restrict__ plan,
                                                          uint8_t* __restrict__ sync, int m,
                                                          int nrounds) {
  using G = ChainGeo<MT>;
  extern __shared__ __align__(16) uint8_t lds[];
  const ChainHeader* hdr = reinterpret_cast<const ChainHeader*>(plan);
  unsigned int* const status = reinterpret_cast<unsigned int*>(sync + kStatusOff);
  if (hdr->magic != kChainMagic) return;                 // not a chain plan: touch nothing
  if (hdr->version != kChainVersion || hdr->format != F || hdr->m != m ||
      hdr->grid != static_cast<int>(gridDim.x) || hdr->nrounds != nrounds) {
    if (threadIdx.x == 0) atomicOr(status, SV_PASS_STATUS_STALE);
    return;
  }
  const ChainRound* rounds = reinterpret_cast<const ChainRound*>(plan + kRoundsOff);
  uint64_t* const counters = reinterpret_cast<uint64_t*>(sync);
  const int wg = blockIdx.x, grid = gridDim.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, q = lane >> 4;
  // Abort flag of the workgroup, an LDS word (its reads wait on lgkmcnt only,
  // never on the weight loads in flight).
  __shared__ int abort_flag;                    // read after barriers (their asm clobbers memory)

  // Stale lines of buffers that an earlier launch read and a later one
  // rewrote (agent-scope acquire: invalidates this compute unit's L1 and its
  // L2 lines that are not coherent across the device).
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  if (threadIdx.x == 0) abort_flag = 0;
  __syncthreads();

  // Tiles of this workgroup in a round: wg, wg + grid, ... below ntiles
  // (at most TM: the plan's rounds hold at most TM per workgroup).
  constexpr int TM = round_tiles(MT);

  if (wave == kSW) {
    // ======================= IO wave =======================
    uint64_t epoch = 0;
    const int g = wg % kNG;
    const int nsig = hdr->nsignals;
    if (nsig > 0) {
      const uint64_t c = __hip_atomic_load(counters + g * (kSyncStride / 8), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
      epoch = c / (static_cast<uint64_t>(nsig) * hdr->group_size[g]);
    }
    // The fields of the round, read one round ahead so their scalar loads
    // are not waited for when the round starts.
    struct Cur {
      int sig;
      uint32_t flags;
    };
    auto fetch = [&](int ri) {
      const ChainRound& rd = rounds[ri < nrounds ? ri : nrounds - 1];
      return Cur{uni(rd.signal_index), static_cast<uint32_t>(uni(static_cast<int>(rd.flags)))};
    };
    Cur cur = fetch(0);
    for (int ri = 0; ri < nrounds; ++ri) {
      const Cur nxt = fetch(ri + 1);
      if (cur.flags & kFlagWait) {
        // every earlier link complete on every workgroup
        const int gi = lane < kNG ? lane : 0;
        const uint64_t target =
            (epoch * nsig + cur.sig) * static_cast<uint64_t>(hdr->group_size[gi]);
        bool ok = false;
        const int limit = hdr->spin_limit;
        for (int n = 0; n < limit; ++n) {
          const uint64_t c = lane < kNG ? __hip_atomic_load(counters + gi * (kSyncStride / 8),
                                                             __ATOMIC_RELAXED,
                                                             __HIP_MEMORY_SCOPE_AGENT)
                                        : target;
          if (__all(c >= target)) {
            ok = true;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        if (!ok) {
          if (lane == 0) atomicOr(status, SV_PASS_STATUS_TIMEOUT);
          abort_flag = 1;
          sv_barrier_no_fence();                  // B0: the stream waves see the abort
          sv_wait_vmcnt<0>();
          return;
        }
      }
      sv_barrier_no_fence();                      // B0: the round's inputs are complete
      sv_barrier_no_fence();                      // E1: partial sums may overwrite the blocks
      sv_barrier_no_fence();                      // E2: partial sums written
      sv_barrier_no_fence();                      // E3: every stream wave's xo stores complete
      if (cur.flags & kFlagSignal) {
        if (lane == 0)
          __hip_atomic_fetch_add(counters + g * (kSyncStride / 8), static_cast<uint64_t>(1),
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      cur = nxt;
    }
    sv_wait_vmcnt<0>();
    return;
  }

  // ======================= stream waves =======================
  const unsigned int magic = sv_opaque_u32(0x43434343u);
  const sv_u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const sv_f32x4 fz = {0.f, 0.f, 0.f, 0.f};

  constexpr bool W8 = F == SV_PASS_W8;
  sv_f32x4 yacc[TM][MT];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int a = 0; a < MT; ++a) yacc[i][a] = fz;
  // W8: the wave's activation row sums (lane (col, q): rows 4q .. 4q + 3)
  sv_f32x4 xacc[MT];
#pragma unroll
  for (int a = 0; a < MT; ++a) xacc[a] = fz;
  float csc = 0.f;                                // W8: channel scale of the wave's output pair

  float* const tpose = reinterpret_cast<float*>(lds + G::TPOSE) + wave * 256;
  uint8_t* const act = lds + wave * G::WAVEB;     // this wave's activation block ring

  // One round of T tiles.  Step w of a wave covers its k-block b = 8 w +
  // wave for every tile of the round: the activation block (16 MT rows x 128
  // k, bf16) comes into the wave's own LDS ring of A blocks, the weight units
  // (tile i, block b) into a register ring of P steps x T units (wb[p][i]:
  // 1 KiB of codes, szr[p][i]: the lane's 8 bytes of the scale/zero record).
  // Issue order: the weights of steps 0 .. P-1 when the round starts (they do
  // not depend on earlier links, so they stream while the barrier is polled),
  // the activation blocks of steps 0 .. A-1 once the barrier is passed, then
  // per step w: after unit (w, i) the unit (w + P, i), after the last unit
  // the activation block of step w + A (out of range past the round's last
  // step).  The number of loads issued after those a step needs is then the
  // same at every step (one value for the first max(A, P) steps, one after),
  // so the wait before a step is exact.  No step synchronizes the waves: each
  // reads only its own blocks.
  // The fields of a round in scalar registers, read one round ahead.
  struct Info {
    const uint8_t* codes;
    const void* sz;
    const void* x;
    float* y;
    void* xo;
    float alpha;
    int K, N, xo_cols, tile0, ntiles;
  };
  auto fetch = [&](int ri) {
    const ChainRound& rd = rounds[ri < nrounds ? ri : nrounds - 1];
    return Info{uni(rd.codes), uni(rd.sz), uni(rd.x), uni(rd.y), uni(rd.xo),
                __int_as_float(uni(__float_as_int(rd.alpha))), uni(rd.K), uni(rd.N),
                uni(rd.xo_cols), uni(rd.tile0), uni(rd.ntiles)};
  };

  auto run_round = [&](auto tc, auto pc, const Info& rd) {
    constexpr int T = decltype(tc)::value;
    constexpr int P = decltype(pc)::value;
    constexpr int A = G::A;
    constexpr int AL = G::BLOADS;                 // loads per activation block
    // loads a step may leave in flight: see the issue order above
    constexpr int kAfterW = AL + (P - 1) * (2 * T + AL);
    constexpr int kAfterA = (A - 1) * (2 * T + AL);
    constexpr int kWaitSteady = kAfterW < kAfterA ? kAfterW : kAfterA;
    constexpr int kWaitEarly = kAfterW < AL * (A - 1) ? kAfterW : AL * (A - 1);
    constexpr int kEarly = A > P ? A : P;
    static_assert(kWaitSteady <= 63 && kWaitEarly <= kWaitSteady, "vmcnt field");
    const int K = rd.K, N = rd.N;
    const int KB = K / 128;
    const int W = (KB + kSW - 1) / kSW;
    const int ntile = N / 16;
    const int t0 = rd.tile0 + wg;
    // W4: 1 KiB units of 128 k and their scale/zero records; W8: two 1 KiB
    // units of 64 k per 128-k block and the f16 channel scales
    const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(rd.codes), 0, W8 ? N * K : N * (K / 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(rd.sz), 0, W8 ? N * 2 : N * (K / 64) * 4, 0x00020000);
    if constexpr (W8) {
      // the channel scale of this wave's output pair, issued before every
      // other load of the round (so it is not counted in any wait below)
      const int tile = t0 + (wave / MT) * grid;
      const unsigned int off = wave < T * MT ? static_cast<unsigned int>((16 * tile + col) * 2)
                                             : kSvOutOfRange;
      csc = __half2float(__builtin_bit_cast(
          __half, static_cast<unsigned short>(__builtin_amdgcn_raw_buffer_load_b16(
                      srs, off, 0, kStreamC))));
    }
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(rd.x), 0, m * K * 2, 0x00020000);
    sv_u32x4 wb[P][T];
    // W4: the lane's 8 bytes of the record; W8: the second 64-k unit
    std::conditional_t<W8, sv_u32x4, sv_u32x2> szr[P][T];
    // unit (w, i) -> ring slot [w % P][i]; two loads per unit in both formats
    auto issue = [&](const int p, const int i, const int w) {
      const int b = w * kSW + wave;
      const bool ok = w < W && b < KB;
      if constexpr (W8) {
        const int blk = ok ? sv_pk_block(t0 + i * grid, 2 * b, 2 * KB, ntile) : 0;
        const int blk1 = ok ? sv_pk_block(t0 + i * grid, 2 * b + 1, 2 * KB, ntile) : 0;
        wb[p][i] = __builtin_amdgcn_raw_buffer_load_b128(crs, ok ? lane * 16 : kSvOutOfRange,
                                                         blk * 1024, kStreamC);
        szr[p][i] = __builtin_amdgcn_raw_buffer_load_b128(crs, ok ? lane * 16 : kSvOutOfRange,
                                                          blk1 * 1024, kStreamC);
      } else {
        const int blk = ok ? sv_pk_block(t0 + i * grid, b, KB, ntile) : 0;
        wb[p][i] = __builtin_amdgcn_raw_buffer_load_b128(crs, ok ? lane * 16 : kSvOutOfRange,
                                                         blk * 1024, kStreamC);
        szr[p][i] = __builtin_amdgcn_raw_buffer_load_b64(srs, ok ? col * 8 : kSvOutOfRange,
                                                         blk * 128, kStreamC);
      }
    };
    // activation block of step w -> ring slot w % A.  Load L brings rows
    // 4 L .. 4 L + 3 (lane l: row 4 L + l / 16, LDS column l % 16, which
    // holds global column (l % 16) ^ (row % 16), so the 16 rows of an MFMA
    // operand read 16 different bank groups)
    // (row 4 L + l / 16 has row % 16 = 4 (L % 4) + l / 16, whose XOR with the
    // LDS column is xl ^ 4 (L % 4) for xl = (l % 16) ^ (l / 16))
    const int lrow = lane >> 4;
    const int lx16 = 16 * ((lane & 15) ^ lrow);
    const int lbase = lrow * K * 2;
    // (the loads are issued on every path, the offsets chosen by per-lane
    // selects: a load under a branch would leave the compiler's own count of
    // the loads in flight short, and its waits stricter than these)
    auto issue_act = [&](const int w) {
      const int b = w * kSW + wave;
      const int lim = uni(w < W && b < KB ? m : 0);   // rows to load (0: none)
      uint8_t* const dst = act + (w % A) * G::BLKB;
      const int ub = uni(256 * b);
      unsigned int o[AL];
#pragma unroll
      for (int L = 0; L < AL; ++L) {
        const int off = lbase + (lx16 ^ (64 * (L & 3))) + (ub + L * 8 * K);
        o[L] = lrow + 4 * L < lim ? static_cast<unsigned int>(off) : kSvOutOfRange;
      }
      sv_compiler_fence();
#pragma unroll
      for (int L = 0; L < AL; ++L)
        lds_load16(xrs, dst + L * 1024, o[L]);
    };
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int i = 0; i < T; ++i) issue(p, i, p);
    sv_barrier_no_fence();                        // B0: the round's inputs are complete
    if (abort_flag) return false;
    sv_compiler_fence();
#pragma unroll
    for (int a = 0; a < A; ++a) issue_act(a);
    sv_compiler_fence();
    for (int w0 = 0; w0 < W; w0 += P) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        // Every step issues its loads, also past the round's last step (out
        // of range), so that every path through the loop keeps the same
        // loads in flight and the compiler's own waits stay as exact as ours.
        const int w = w0 + p;
        const int b = w * kSW + wave;
        const bool valid = w < W && b < KB;       // wave-uniform
        if (w < kEarly) sv_wait_vmcnt<kWaitEarly>();
        else sv_wait_vmcnt<kWaitSteady>();
        {
          const uint8_t* const blk = act + (w % A) * G::BLKB;
          // activation operands of block b: row tile a, group h, two 32-k slices
          sv_u32x4 a0[2][MT], a1[2][MT];
          float xsA[MT];
          if (valid) {
#pragma unroll
            for (int a = 0; a < MT; ++a) {
              const uint8_t* rp = blk + (16 * a + col) * 256;
#pragma unroll
              for (int h = 0; h < 2; ++h) {
                const int c0 = 8 * h + 2 * q;     // 16-byte column in the block row
                a0[h][a] = *reinterpret_cast<const sv_u32x4*>(rp + ((c0 ^ col) << 4));
                a1[h][a] = *reinterpret_cast<const sv_u32x4*>(rp + (((c0 + 1) ^ col) << 4));
              }
              if constexpr (W8) {
                // row sums in the output layout: activations times all-ones
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                  xacc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                      sv_as_bf16x8(a0[h][a]), sv_as_bf16x8(ones), xacc[a], 0, 0, 0);
                  xacc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                      sv_as_bf16x8(a1[h][a]), sv_as_bf16x8(ones), xacc[a], 0, 0, 0);
                }
              } else {
              // group row sums: an all-ones A operand puts the sum of row col
              // on lane (col, q); the correction wants group q on lane (col, q)
              sv_f32x4 g0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  sv_as_bf16x8(ones), sv_as_bf16x8(a0[0][a]), fz, 0, 0, 0);
              g0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sv_as_bf16x8(ones),
                                                           sv_as_bf16x8(a1[0][a]), g0, 0, 0, 0);
              sv_f32x4 g1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  sv_as_bf16x8(ones), sv_as_bf16x8(a0[1][a]), fz, 0, 0, 0);
              g1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sv_as_bf16x8(ones),
                                                           sv_as_bf16x8(a1[1][a]), g1, 0, 0, 0);
              xsA[a] = q == 0 ? g0[0] : (q == 1 ? g1[0] : 0.0f);
              }
            }
          }
#pragma unroll
          for (int i = 0; i < T; ++i) {
            if constexpr (W8) {
             if (valid) {
              // unit 2b + h holds k = 64 h + 16 q + [0, 16) of the block for
              // channel col: the k of a0[h] then a1[h]
#pragma unroll
              for (int h = 0; h < 2; ++h) {
                const sv_u32x4 wv = h ? szr[p][i] : wb[p][i];
                const sv_u32x2 l0 = sv_w8_cvt4_bias128(wv.x), l1 = sv_w8_cvt4_bias128(wv.y);
                const sv_u32x2 h0 = sv_w8_cvt4_bias128(wv.z), h1 = sv_w8_cvt4_bias128(wv.w);
                const sv_u32x4 b0 = {l0.x, l0.y, l1.x, l1.y};
                const sv_u32x4 b1 = {h0.x, h0.y, h1.x, h1.y};
#pragma unroll
                for (int a = 0; a < MT; ++a) {
                  yacc[i][a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                      sv_as_bf16x8(a0[h][a]), sv_as_bf16x8(b0), yacc[i][a], 0, 0, 0);
                  yacc[i][a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                      sv_as_bf16x8(a1[h][a]), sv_as_bf16x8(b1), yacc[i][a], 0, 0, 0);
                }
              }
             }
            } else if (valid) {
              const sv_u32x4 wv = wb[p][i];
              const sv_u32x2 sv = szr[p][i];
              sv_f32x4 t[MT];
#pragma unroll
              for (int h = 0; h < 2; ++h) {
                const sv_u32x4 b0 = sv_w4_dequant8(h ? wv.z : wv.x, magic);
                const sv_u32x4 b1 = sv_w4_dequant8(h ? wv.w : wv.y, magic);
                const float sc = sv_materialize(sv_half_lo(h ? sv.y : sv.x));
#pragma unroll
                for (int a = 0; a < MT; ++a) {
                  sv_f32x4 acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                      sv_as_bf16x8(a0[h][a]), sv_as_bf16x8(b0), fz, 0, 0, 0);
                  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sv_as_bf16x8(a1[h][a]),
                                                                sv_as_bf16x8(b1), acc, 0, 0, 0);
#pragma unroll
                  for (int j = 0; j < 4; ++j) t[a][j] = h ? fmaf(sc, acc[j], t[a][j]) : sc * acc[j];
                }
              }
              // bias and zero point of the block's two groups (lanes q >= 2 add 0)
              const unsigned int szq = q == 0 ? sv.x : sv.y;
              const float v = -(sv_half_lo(szq) * (128.0f + sv_half_hi(szq)));
              const float nsz = q < 2 ? v : 0.0f;
#pragma unroll
              for (int a = 0; a < MT; ++a) {
                t[a] = __builtin_amdgcn_mfma_f32_16x16x4f32(xsA[a], nsz, t[a], 0, 0, 0);
                yacc[i][a] += t[a];
              }
            }
            sv_compiler_fence();
            issue(p, i, w + P);                   // unit (w + P, i) into the freed slot
            sv_compiler_fence();
          }
        }
        // the block's operands are in registers (the MFMAs above used them):
        // its slot takes the block of step w + A
        sv_compiler_fence();
        issue_act(w + A);
        sv_compiler_fence();
      }
    }
    return true;
  };

  Info rd = fetch(0);
  for (int ri = 0; ri < nrounds; ++ri) {
    const Info nxt = fetch(ri + 1);
    const int tt = (rd.ntiles - wg + grid - 1) / grid;
    const int T = tt < TM ? tt : TM;
    // ring depth P T: 4 to 6 units of 1 KiB per wave (measured: deeper
    // rings queue the activation loads behind more weight loads and run
    // slower; at m > 16 the same depths fit the registers)
    bool go = true;
    constexpr int P1 = 4, P2 = 2, P3 = 2;
    switch (T) {
      case 1: go = run_round(std::integral_constant<int, 1>{}, std::integral_constant<int, P1>{}, rd); break;
      case 2: go = run_round(std::integral_constant<int, 2>{}, std::integral_constant<int, P2>{}, rd); break;
      case 3: go = run_round(std::integral_constant<int, 3>{}, std::integral_constant<int, P3>{}, rd); break;
      case 4: go = run_round(std::integral_constant<int, 4>{}, std::integral_constant<int, 1>{}, rd); break;
      case 5:
      case 6:
        if constexpr (TM >= 6) {
          if (T == 5) go = run_round(std::integral_constant<int, 5>{}, std::integral_constant<int, 1>{}, rd);
          else go = run_round(std::integral_constant<int, 6>{}, std::integral_constant<int, 1>{}, rd);
        }
        break;
      default:                                    // no tile of this round here
        sv_barrier_no_fence();                    // B0
        go = !abort_flag;
        break;
    }
    if (!go) {
      sv_wait_vmcnt<0>();
      return;
    }
    // every activation load of the round has landed (the tail's out-of-range
    // ones included) before the partial sums overwrite the blocks
    sv_wait_vmcnt<0>();

    // ---- end of the round: fixed-order sum of the 8 waves' partial sums ----
    sv_barrier_no_fence();                        // E1: every wave done with its blocks
    if constexpr (W8) {
      // W8: y = s (sum x (128 + c) - 128 sum x), the bias folded per wave
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int a = 0; a < MT; ++a)
#pragma unroll
          for (int j = 0; j < 4; ++j) yacc[i][a][j] = fmaf(-128.0f, xacc[a][j], yacc[i][a][j]);
#pragma unroll
      for (int a = 0; a < MT; ++a) xacc[a] = fz;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if (i < T) {
#pragma unroll
        for (int a = 0; a < MT; ++a)
          *reinterpret_cast<sv_f32x4*>(lds + (((i * MT + a) * kSW + wave) * 1024) + lane * 16) =
              yacc[i][a];
      }
#pragma unroll
      for (int a = 0; a < MT; ++a) yacc[i][a] = fz;
    }
    sv_barrier_no_fence();                        // E2: partial sums in LDS
    if (T > 0) {
      const int N = rd.N, xo_cols = rd.xo_cols, tile0 = rd.tile0;
      const bool has_xo = rd.xo != nullptr;
      const float alpha = rd.alpha;
      const __amdgpu_buffer_rsrc_t yrs =
          __builtin_amdgcn_make_buffer_rsrc(rd.y, 0, m * N * 4, 0x00020000);
      const __amdgpu_buffer_rsrc_t ors =
          __builtin_amdgcn_make_buffer_rsrc(rd.xo, 0, has_xo ? m * xo_cols * 2 : 0, 0x00020000);
      // one (tile, row tile) pair per wave at most: T * MT <= 6 < kSW
      static_assert(TM * MT <= kSW, "one output pair per stream wave");
      const int v = wave;
      if (v < T * MT) {
        sv_f32x4 s = *reinterpret_cast<const sv_f32x4*>(lds + (v * kSW) * 1024 + lane * 16);
#pragma unroll
        for (int j = 1; j < kSW; ++j) {
          const sv_f32x4 p =
              *reinterpret_cast<const sv_f32x4*>(lds + (v * kSW + j) * 1024 + lane * 16);
#pragma unroll
          for (int i = 0; i < 4; ++i) s[i] += p[i];
        }
        if constexpr (W8) {
#pragma unroll
          for (int i = 0; i < 4; ++i) s[i] *= csc;    // lane (col, q): channel col
        }
        // MFMA layout (lane (col, q): rows 4q .. 4q + 3 of channel col) ->
        // lane l: row l / 4, channels 4 (l % 4) .. + 3
#pragma unroll
        for (int i = 0; i < 4; ++i) tpose[(4 * q + i) * 16 + col] = s[i];
        sv_compiler_fence();
        const sv_f32x4 o = *reinterpret_cast<const sv_f32x4*>(tpose + (lane >> 2) * 16 +
                                                               4 * (lane & 3));
        sv_compiler_fence();
        const int tile = tile0 + wg + (v / MT) * grid;
        const int n0 = 16 * tile;
        const int row = 16 * (v % MT) + (lane >> 2);
        // the hand-off first (the next link reads it), then y
        if (has_xo && n0 < xo_cols) {
          sv_u32x2 pk;
          pk.x = bf16_rne(alpha * o[0]) | (bf16_rne(alpha * o[1]) << 16);
          pk.y = bf16_rne(alpha * o[2]) | (bf16_rne(alpha * o[3]) << 16);
          const unsigned int xoff =
              row < m ? static_cast<unsigned int>((row * xo_cols + n0 + 4 * (lane & 3)) * 2)
                      : kSvOutOfRange;
          __builtin_amdgcn_raw_buffer_store_b64(pk, ors, xoff, 0, kSc1);
        }
        sv_compiler_fence();
        const unsigned int off =
            row < m ? static_cast<unsigned int>((row * N + n0 + 4 * (lane & 3)) * 4)
                    : kSvOutOfRange;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(sv_u32x4, o), yrs, off, 0,
                                               kStreamC);
      }
    }
    // The hand-off is complete at agent scope before the IO wave arrives.
    // No load of this wave is in flight here (the round's rings are consumed
    // and drained before E1; the next round's start after E3), and stores
    // complete in issue order, so allowing the one y store to stay in flight
    // waits exactly for the xo store before it (and for the y store of the
    // previous round).  That y store completes before any load of the next
    // round does (in-order counting), and so before this wave writes y again.
    if (T > 0 && wave < T * MT)
      sv_wait_vmcnt<1>();
    else
      sv_wait_vmcnt<0>();
    sv_barrier_no_fence();                        // E3
    rd = nxt;
  }
  sv_wait_vmcnt<0>();
}

template <int MT, int F>
sv_status launch_chain(void* plan, int nrounds, int m, int grid, hipStream_t st) {
  auto kern = chain_kernel<MT, F>;
  constexpr int kLds = ChainGeo<MT>::LDS;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kLds) != hipSuccess)
    return SV_ERR_HIP;
  uint8_t* const p = static_cast<uint8_t*>(plan);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreadsC), kLds, st, p, p + sync_off(nrounds), m,
                     nrounds);
  SV_LAUNCH_CHECK();
  return SV_OK;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na > 0 && nb > 0 && x < y + nb && y < x + na;
}

// Validates the links and counts the rounds (0 on error, status in *st).
int chain_rounds(int format, const sv_pass_link* links, int count, int m, int grid,
                 sv_status* st) {
  const int tm = round_tiles(m > 16 ? 2 : 1);
  *st = SV_OK;
  if (format != SV_PASS_W4 && format != SV_PASS_W8) {
    *st = format == SV_PASS_W4_I8 ? SV_ERR_UNSUPPORTED : SV_ERR_INVALID_ARG;
    return 0;
  }
  if (!links) {
    *st = SV_ERR_NULL;
    return 0;
  }
  if (count < 1 || m < 1 || m > SV_MAX_ROWS) {
    *st = SV_ERR_INVALID_ARG;
    return 0;
  }
  long long nr = 0;
  for (int i = 0; i < count; ++i) {
    const sv_pass_link& e = links[i];
    if (!e.x || !e.codes || !e.scales || !e.y || (e.xo_cols > 0) != (e.xo != nullptr)) {
      *st = SV_ERR_NULL;
      return 0;
    }
    if (e.N < 16 || e.N % 16 != 0 || e.K < 128 || e.K % 128 != 0 || e.xo_cols < 0 ||
        e.xo_cols > e.N || e.xo_cols % 64 != 0) {
      *st = SV_ERR_INVALID_ARG;
      return 0;
    }
    if (static_cast<long long>(e.N) * e.K / (format == SV_PASS_W8 ? 1 : 2) >= (1LL << 31) ||
        static_cast<long long>(m) * e.N * 4 >= (1LL << 31) ||
        static_cast<long long>(m) * e.K * 2 >= (1LL << 31)) {
      *st = SV_ERR_UNSUPPORTED;
      return 0;
    }
    if (!sv_aligned16(e.x) || !sv_aligned16(e.codes) || !sv_aligned16(e.scales) ||
        !sv_aligned16(e.y) || (e.xo && (reinterpret_cast<uintptr_t>(e.xo) & 127u) != 0)) {
      *st = SV_ERR_ALIGN;
      return 0;
    }
    const int tiles = e.N / 16;
    const int per = tm * grid;
    nr += (tiles + per - 1) / per;
  }
  // Buffer rules (byte ranges): an x that meets an earlier xo is exactly that
  // xo; no xo meets the x of its own or an earlier link, another xo, or a y;
  // no y meets any x, xo or other y.
  for (int i = 0; i < count; ++i) {
    const sv_pass_link& e = links[i];
    const size_t xb = static_cast<size_t>(m) * e.K * 2, yb = static_cast<size_t>(m) * e.N * 4;
    for (int j = 0; j < count; ++j) {
      const sv_pass_link& f = links[j];
      const size_t fxo = static_cast<size_t>(m) * f.xo_cols * 2;
      const size_t fyb = static_cast<size_t>(m) * f.N * 4, fxb = static_cast<size_t>(m) * f.K * 2;
      if (overlap(e.x, xb, f.xo, fxo) &&
          (j >= i || e.x != f.xo || e.K != f.xo_cols)) {
        *st = SV_ERR_INVALID_ARG;
        return 0;
      }
      if (overlap(e.y, yb, f.x, fxb) || overlap(e.y, yb, f.xo, fxo) ||
          (j != i && overlap(e.y, yb, f.y, fyb))) {
        *st = SV_ERR_INVALID_ARG;
        return 0;
      }
      if (j != i && overlap(e.xo, static_cast<size_t>(m) * e.xo_cols * 2, f.xo, fxo)) {
        *st = SV_ERR_INVALID_ARG;
        return 0;
      }
    }
  }
  if (nr >= (1 << 24)) {
    *st = SV_ERR_UNSUPPORTED;
    return 0;
  }
  return static_cast<int>(nr);
}

int chain_grid(const sv_pass_link* links, int count, int cus) {
  int g = std::min(cus, kMaxGridC);
  for (int i = 0; i < count; ++i) g = std::min(g, links[i].N / 16);
  return std::max(g, 1);
}

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return cus;
}

// The plan image for a device of `cus` compute units (host only).
sv_status build_chain_image(int format, const sv_pass_link* links, int count, int m, int group,
                            int cus, std::vector<uint8_t>* image, int* grid_out, int* nr_out) {
  if (!links) return SV_ERR_NULL;
  if (cus < 1) return SV_ERR_INVALID_ARG;
  if (count < 1) return SV_ERR_INVALID_ARG;
  const int grid = chain_grid(links, count, cus);
  sv_status st;
  const int nr = chain_rounds(format, links, count, m, grid, &st);
  if (nr == 0) return st;
  if (group != 64) return SV_ERR_UNSUPPORTED;
  image->assign(chain_bytes(nr), 0);
  ChainHeader* hdr = reinterpret_cast<ChainHeader*>(image->data());
  ChainRound* rounds = reinterpret_cast<ChainRound*>(image->data() + kRoundsOff);
  // A link waits iff its x is an earlier link's xo; the link before a waiting
  // link raises the arrivals (a workgroup that arrives has finished every
  // earlier link: it runs the links in order).
  std::vector<int> waits(count, 0);
  for (int i = 0; i < count; ++i)
    for (int j = 0; j < i; ++j)
      if (links[j].xo && links[i].x == links[j].xo) waits[i] = 1;
  const int per = round_tiles(m > 16 ? 2 : 1) * grid;
  int nsig = 0, r = 0;
  for (int i = 0; i < count; ++i) {
    const sv_pass_link& e = links[i];
    if (waits[i]) ++nsig;
    const bool signal = i + 1 < count && waits[i + 1];
    const int tiles = e.N / 16;
    const int nround = (tiles + per - 1) / per;
    const int each = (tiles + nround - 1) / nround;
    for (int k = 0; k < nround; ++k) {
      ChainRound& rd = rounds[r++];
      rd.codes = e.codes;
      rd.sz = e.scales;
      rd.x = e.x;
      rd.y = e.y;
      rd.xo = e.xo;
      rd.alpha = e.alpha;
      rd.K = e.K;
      rd.N = e.N;
      rd.xo_cols = e.xo_cols;
      rd.tile0 = k * each;
      rd.ntiles = std::min(each, tiles - k * each);
      rd.signal_index = nsig;
      rd.flags = (k == 0 && waits[i] ? kFlagWait : 0u) |
                 (k + 1 == nround && signal ? kFlagSignal : 0u);
      if (rd.ntiles < grid) return SV_ERR_UNSUPPORTED;   // every workgroup owns a tile
    }
  }
  hdr->magic = kChainMagic;
  hdr->version = kChainVersion;
  hdr->format = format;
  hdr->m = m;
  hdr->grid = grid;
  hdr->nrounds = nr;
  hdr->nlinks = count;
  hdr->nsignals = nsig;
  hdr->spin_limit = kSpinLimit;
  for (int g = 0; g < kNG; ++g) hdr->group_size[g] = grid / kNG + (g < grid % kNG ? 1 : 0);
  *grid_out = grid;
  *nr_out = nr;
  return SV_OK;
}

}  // namespace

uint32_t sv_register_plan(const void* plan);   // pass.hip

extern "C" size_t sv_pass_chain_bytes(int format, const sv_pass_link* links, int count, int m) {
  const int cus = device_cus();
  if (cus < 1 || !links || count < 1) return 0;
  sv_status st;
  const int nr = chain_rounds(format, links, count, m, chain_grid(links, count, cus), &st);
  return nr > 0 ? chain_bytes(nr) : 0;
}

extern "C" sv_status sv_pass_chain_image(int format, const sv_pass_link* links, int count, int m,
                                         int group, int cus, void* image, size_t image_bytes,
                                         int* grid) {
  if (!image || !grid) return SV_ERR_NULL;
  std::vector<uint8_t> img;
  int g = 0, nr = 0;
  const sv_status st = build_chain_image(format, links, count, m, group, cus, &img, &g, &nr);
  if (st != SV_OK) return st;
  if (image_bytes < img.size()) return SV_ERR_WORKSPACE;
  std::copy(img.begin(), img.end(), static_cast<uint8_t*>(image));
  *grid = g;
  return SV_OK;
}

extern "C" sv_status sv_pass_chain_plan(int format, const sv_pass_link* links, int count, int m,
                                        int group, void* plan, size_t plan_bytes, sv_pass* pass,
                                        hipStream_t stream) {
  const int cus = device_cus();
  if (cus < 1) return SV_ERR_HIP;
  std::vector<uint8_t> image;
  int grid = 0, nr = 0;
  const sv_status st = build_chain_image(format, links, count, m, group, cus, &image, &grid, &nr);
  if (st != SV_OK) return st;
  if (!plan || !pass) return SV_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(plan) & 255u) != 0) return SV_ERR_ALIGN;
  if (plan_bytes < image.size()) return SV_ERR_WORKSPACE;
  if (hipMemcpyAsync(plan, image.data(), image.size(), hipMemcpyHostToDevice, stream) !=
          hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return SV_ERR_HIP;
  pass->plan = plan;
  pass->format = format;
  pass->m = m;
  pass->count = count;
  pass->grid = grid;
  pass->items = nr;
  pass->max_steps = 0;
  pass->stats = 0;
  pass->chain = 1;
  pass->id = sv_register_plan(plan);
  return SV_OK;
}

// Called by sv_pass_run for chain plans.
sv_status sv_chain_run(const sv_pass* pass, hipStream_t stream) {
  if (pass->format != SV_PASS_W4 && pass->format != SV_PASS_W8) return SV_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(pass->plan) & 255u) != 0) return SV_ERR_ALIGN;
  if (pass->grid < 1 || pass->grid > kMaxGridC || pass->grid > device_cus())
    return SV_ERR_INVALID_ARG;
  if (pass->items < 1) return SV_ERR_INVALID_ARG;
  void* const pl = pass->plan;
  if (pass->format == SV_PASS_W8)
    return pass->m > 16 ? launch_chain<2, SV_PASS_W8>(pl, pass->items, pass->m, pass->grid, stream)
                        : launch_chain<1, SV_PASS_W8>(pl, pass->items, pass->m, pass->grid, stream);
  return pass->m > 16 ? launch_chain<2, SV_PASS_W4>(pl, pass->items, pass->m, pass->grid, stream)
                      : launch_chain<1, SV_PASS_W4>(pl, pass->items, pass->m, pass->grid, stream);
}

// Byte offset of a chain plan's status word (sv_pass_status).
size_t sv_chain_status_offset(const sv_pass* pass) { return sync_off(pass->items) + kStatusOff; }
