// Verify-pass executor: every GEMM of one verify pass in a single persistent
// launch, for the three weight paths of the method:
//   SV_PASS_W4     bf16 activations x 4-bit asymmetric group-64 weights
//   SV_PASS_W8     bf16 activations x 8-bit symmetric per-channel weights
//   SV_PASS_W4_I8  int8 activations (per-row scale) x 4-bit weights, exact
//                  int32 group partials
//
// Source: Karpathy's Trick for Faster Local LLMs, "Why batch-one decoding is
// memory-bound" (a pass streams every weight once, so its speed is bandwidth
// divided by the weight bytes) and "How Uzu optimizes bytes and tokens per
// pass" (the 4-bit asymmetric and 8-bit symmetric checkpoint tiers; activations
// quantized to 8 bits so both operands are integers; format and kernels
// designed together); Local LLM 4x Faster (the int8 matrix path); Speculative
// Decoding Clearly Explained, "Check the guesses together" (all draft
// positions scored in one pass).
//
// Why one launch: a pass of a 9B-class stack is ~128 GEMMs of 9-57 MB.
// Launched one by one, each pays the ramp-up and drain of a kernel over 256
// compute units and the HBM stream stops at every boundary.  Here each
// workgroup owns a fixed list of work items from all GEMMs and streams them
// back to back through one software pipeline.
//
// Work item = one GEMM x 32 row tiles (512 output channels) x all of K.  Each
// of the 8 waves owns 4 row tiles for the whole K (no cross-wave reduction).
// The item advances in chunks of two 1 KiB weight blocks per tile (256 k for
// 4-bit codes, 128 k for 8-bit codes).  Per step a wave issues:
//   * 8 weight loads of 1 KiB (one fully contiguous 16-byte-per-lane load each,
//     already in MFMA operand order: the packed layouts of sv_w4_pack and
//     sv_w8_pack) into registers;
//   * for 4-bit weights one 1 KiB buffer -> LDS load of its tiles' scale/zero
//     records; for W8 / W4_I8 one small buffer -> LDS load of the channel
//     scales / row scales needed when an item ends;
//   * its share of the activation chunk (16 or 32 rows), copied once per
//     workgroup into LDS by buffer -> LDS loads and shared by the 32 tiles.
// Activation rows sit in LDS with XOR-swizzled 16-byte columns (column j of
// row r at j ^ (r % 16)), so the 16 lanes reading one MFMA operand hit 16
// different bank groups.  Chunks flow through a ring of P slots (P - 1 chunks
// in flight while one computes).  Every step issues the same number of vector
// memory instructions (out-of-range per-lane offsets where a tile, block or
// row does not exist; the item's output stores every step, out of range except
// on its last chunk), so one compile-time vmcnt wait is exact: vector memory
// operations of a wave complete in issue order.
//
// Arithmetic:
//   W4:    bf16 128 + c from a mask and a byte permute against 0x43;
//          v_mfma_f32_16x16x32_bf16 gives acc = sum x (128 + c) per group and
//          tile, folded as y += s acc (one VALU per output).  The bias and the
//          zero point leave once per 4 groups through one rank-4 binary32
//          update y -= sum_g xsum[r, g] s[n, g] (128 + z[n, g])
//          (v_mfma_f32_16x16x4_f32), whose row-sum operand comes straight
//          out of an all-ones-A MFMA in the required lane layout.  For a
//          one-hot row and integer z both terms are exact, so is
//          (c - z) s.
//   W8:    bf16 128 + c from the biased byte (v_cvt_f32_ubyte, upper half);
//          the MFMA accumulates over all of K; at the item end
//          y = s (acc - 128 xsum).
//   W4_I8: v_mfma_i32_16x16x64_i8 (K depth = one group) gives the exact int32
//          partial I = sum c xq, folded as y += s I; the zero point leaves
//          through the same rank-4 update with the exact int32 group sums
//          Xg = sum xq; at the item end y *= xscale[row].
//
// Optional softmax-statistics epilogue (any format, per GEMM): with a stats
// buffer, the item end also writes, for each row and each 64 output channels
// (one wave's share), the maximum of y and the sum of exp(y - max) -- the
// online-softmax pieces of a vocabulary projection, so a following accept
// step need not read the logits back to normalize them (Speculative Decoding
// Clearly Explained, "Check the guesses together": the target scores every
// draft position in the pass; "Accept from left to right" needs p = softmax).
#include <algorithm>
#include <cstddef>
#include <functional>
#include <mutex>
#include <queue>
#include <unordered_map>
#include <vector>

#include "w4_packed_dev.h"

namespace {

constexpr uint32_t kPlanMagic = 0x50565653u;   // "SVVP"
constexpr uint32_t kPlanVersion = 3;
constexpr int kMaxGrid = 2048;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kNB = 2;                          // 1 KiB weight blocks per tile per step
constexpr int kTW = 4;                          // row tiles per wave
constexpr int kItemTiles = kWaves * kTW;        // row tiles per item (512 channels)
constexpr int kGroup = 64;
// Cache policy of the streams touched once per pass (weights, scale/zero
// records, outputs): non-temporal, so they do not displace the activations
// that every workgroup re-reads from L2.  Measured: ~5% faster passes.
constexpr int kStream = 2;

template <int F>
struct Fmt;
template <>
struct Fmt<SV_PASS_W4> {
  static constexpr int KPB = 128;   // k per 1 KiB weight block (16 rows)
  static constexpr int XE = 2;      // activation bytes per element (bf16)
  static constexpr int SZD = 1;     // per-step scale/zero load
  static constexpr int AUXD = 0;    // per-step item-end data load
};
template <>
struct Fmt<SV_PASS_W8> {
  static constexpr int KPB = 64;
  static constexpr int XE = 2;
  static constexpr int SZD = 0;
  static constexpr int AUXD = 1;    // channel scales
};
template <>
struct Fmt<SV_PASS_W4_I8> {
  static constexpr int KPB = 128;
  static constexpr int XE = 1;      // int8 activations
  static constexpr int SZD = 1;
  static constexpr int AUXD = 1;    // row scales
};

inline int fmt_kpb(int f) { return f == SV_PASS_W8 ? 64 : 128; }
inline int fmt_xe(int f) { return f == SV_PASS_W4_I8 ? 1 : 2; }

struct PlanHeader {                             // 64 bytes
  uint32_t magic, version;
  int32_t format, m, count, grid, items, max_steps, stats;   // stats: some GEMM has a stats buffer
  uint32_t status;                              // SV_PASS_STATUS_* bits set by the kernel
  uint64_t reserved[3];
};
struct PlanItem {                               // 64 bytes
  const void* x;
  const float* xscale;
  const uint8_t* codes;
  const void* sz;
  float* y;
  int32_t K, N, tile0, nchunk;
  float* stats;                                 // [m, ceil(N / 64)] (max, sum) pairs, or null
};
static_assert(sizeof(PlanHeader) == 64, "plan header layout");
static_assert(sizeof(PlanItem) == 64, "plan item layout");
static_assert(offsetof(PlanHeader, status) == SV_PASS_STATUS_OFFSET, "status word offset");

// Plan image: header | wg_begin[kMaxGrid + 1] | wg_steps[kMaxGrid] | items.
constexpr size_t kBeginOff = sizeof(PlanHeader);
constexpr size_t kStepsOff = kBeginOff + sizeof(int32_t) * (kMaxGrid + 1);
constexpr size_t kItemsOff = (kStepsOff + sizeof(int32_t) * kMaxGrid + 63) / 64 * 64;

__host__ __device__ constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }

template <int F, int MT>
struct Geo {
  static constexpr int KC = kNB * Fmt<F>::KPB;                 // k per chunk
  static constexpr int XROW = KC * Fmt<F>::XE;                 // LDS bytes per activation row
  static constexpr int CPR = XROW / 16;                        // 16-byte columns per row
  static constexpr int RPP = 1024 / XROW;                      // rows per 1 KiB load
  static constexpr int XPIECES = 16 * MT * XROW / 1024;        // 1 KiB loads per chunk
  static constexpr int XD = XPIECES >= kWaves ? XPIECES / kWaves : 1;   // per wave
  static constexpr int XBUF = kWaves * XD * 1024;              // bytes per activation slot
  static constexpr int SZBUF = Fmt<F>::SZD ? kWaves * 1024 : 0;
  static constexpr int AUXBUF = Fmt<F>::AUXD ? kWaves * 1024 : 0;
  static constexpr int SLOT = XBUF + SZBUF + AUXBUF;
  static_assert(XPIECES % kWaves == 0 || XPIECES < kWaves, "uneven activation split");
  static_assert(CPR == 16 || CPR == 32, "activation row of 16 or 32 columns");
};

// W4: group row sums of each slot's activation chunk (MT row tiles x 4
// groups x 16 rows, binary32), written once per workgroup and shared by the
// waves.
template <int F, int MT>
constexpr int xsum_bytes() {
  return F == SV_PASS_W4 ? MT * 4 * 16 * 4 : 0;
}

template <int F, int MT, int P>
constexpr int pass_lds_bytes() {
  // slots + per-wave output transpose + per-slot row sums
  return P * Geo<F, MT>::SLOT + kWaves * 4096 + P * xsum_bytes<F, MT>();
}

// 4 int8 codes (one dword) -> 2 dwords of bf16 pairs holding 128 + c.
__device__ __forceinline__ sv_u32x2 w8_cvt4(unsigned int d) {
  const unsigned int u = d ^ 0x80808080u;
  const unsigned int f0 = __float_as_uint(static_cast<float>(u & 0xFFu));
  const unsigned int f1 = __float_as_uint(static_cast<float>((u >> 8) & 0xFFu));
  const unsigned int f2 = __float_as_uint(static_cast<float>((u >> 16) & 0xFFu));
  const unsigned int f3 = __float_as_uint(static_cast<float>(u >> 24));
  sv_u32x2 r;
  r.x = __builtin_amdgcn_perm(f1, f0, 0x07060302u);
  r.y = __builtin_amdgcn_perm(f3, f2, 0x07060302u);
  return r;
}

// ST: the plan has GEMMs with a softmax-statistics buffer.  Plans without
// any run the ST = false kernel, which holds no trace of the epilogue.
template <int F, int MT, int P, bool ST>
__global__ __launch_bounds__(kThreads) void pass_kernel(const uint8_t* __restrict__ plan, int m) {
  using G = Geo<F, MT>;
  constexpr int L = kTW * kNB + Fmt<F>::SZD + Fmt<F>::AUXD + G::XD;   // loads per wave per step
  // Waits count only loads.  Vector memory operations of a wave complete in
  // issue order, and the output stores (4 MT per wave, on an item's last
  // chunk only) come on top of the counted ones, so each wait is exact
  // except after an item end, where it is stricter than needed.  (A store
  // issued every step to keep the count exact costs as much address
  // processing as a real one.)
  // Chunk c's loads go out in two parts: its weights (LW loads, into the
  // registers chunk c - P has just freed) at the end of step c - P, its LDS
  // loads (activations first) at the start of step c - P + 1, after the
  // barrier that frees their slot.  So the weights run a full step further
  // ahead than the LDS data without more registers.  At the wait before
  // computing chunk c, the loads issued after chunk c's are the weights of
  // chunk c + 1 and the loads of the P - 2 steps after.
  constexpr int LW = kTW * kNB;
  constexpr int WAITN = LW + (P - 2) * L;
  // W4 also needs the activations of chunk c + 1 (the first XD loads of its
  // LDS part) at that wait: after them come the rest of that part, the
  // weights of chunk c + 2 and the loads of the P - 3 steps after.
  constexpr int WAITX = (L - G::XD) + (P - 3) * L;
  constexpr int WAITS = F == SV_PASS_W4 ? WAITX : WAITN;
  // Before the first step (W4): the activations of chunk 0 (the prologue
  // issues weights, then LDS loads, chunk by chunk, and the weights of chunk
  // P - 1 last).
  constexpr int WAIT0 = (L - G::XD) + (P - 2) * L;
  static_assert(P >= 3, "row sums of chunk c + 1 are formed while chunk c computes");
  static_assert(WAITN < 64 && WAIT0 < 64, "too many memory operations in flight for vmcnt");
  static_assert(kTW * kNB * 128 == 1024, "one 1 KiB scale/zero load per wave per step");
  static_assert(kTW == 4, "the output transpose covers a wave's 4 tiles = 64 channels");
  extern __shared__ __align__(16) uint8_t lds[];

  // A plan buffer that does not hold the plan this launch was made for:
  // compute nothing.  (sv_pass_run has already refused a plan that was made
  // again into the same buffer; this check covers a buffer the caller
  // overwrote.)
  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(plan);
  if (hdr->magic != kPlanMagic || hdr->format != F || hdr->m != m || (hdr->stats != 0) != ST ||
      hdr->grid != static_cast<int>(gridDim.x))
    return;
  const int32_t* wg_begin = reinterpret_cast<const int32_t*>(plan + kBeginOff);
  const int32_t* wg_steps = reinterpret_cast<const int32_t*>(plan + kStepsOff);
  const PlanItem* items = reinterpret_cast<const PlanItem*>(plan + kItemsOff);
  const int ib = wg_begin[blockIdx.x];
  const int ie = wg_begin[blockIdx.x + 1];
  const int steps = wg_steps[blockIdx.x];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;
  const int q = lane >> 4;
  const unsigned int magic = sv_opaque_u32(0x43434343u);
  const sv_u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const sv_u32x4 ones8 = {0x01010101u, 0x01010101u, 0x01010101u, 0x01010101u};
  const sv_f32x4 fz = {0.f, 0.f, 0.f, 0.f};
  const sv_i32x4 iz = {0, 0, 0, 0};
  float* const tpose = reinterpret_cast<float*>(lds + P * G::SLOT) + wave * 1024;
  float* const xsb = reinterpret_cast<float*>(lds + P * G::SLOT + kWaves * 4096);

  // ---- weight cursor: the item and chunk whose weight loads go out next ----
  int w_item = ib, w_c = 0;
  int w_K = 128, w_N = 16, w_t0 = 0, w_nchunk = 1;
  __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(nullptr, 0, 0, 0x00020000);
  auto load_w_item = [&](int idx) {
    const PlanItem it = items[idx];
    w_K = it.K;
    w_N = it.N;
    w_t0 = it.tile0;
    w_nchunk = it.nchunk;
    wrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(it.codes), 0,
                                            F == SV_PASS_W8 ? it.N * it.K : it.N * (it.K / 2),
                                            0x00020000);
  };
  // ---- LDS cursor: the item and chunk whose activation / record loads go
  // out next (one chunk behind the weight cursor in steady state) ----
  int i_item = ib, i_c = 0;
  int i_K = 128, i_N = 16, i_t0 = 0, i_nchunk = 1;
  __amdgpu_buffer_rsrc_t srs = wrs, xrs = wrs, ars = wrs;
  auto load_issue_item = [&](int idx) {
    const PlanItem it = items[idx];
    i_K = it.K;
    i_N = it.N;
    i_t0 = it.tile0;
    i_nchunk = it.nchunk;
    if constexpr (Fmt<F>::SZD)
      srs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(it.sz), 0,
                                              it.N * (it.K / kGroup) * 4, 0x00020000);
    if constexpr (F == SV_PASS_W8)
      ars = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(it.sz), 0, it.N * 2, 0x00020000);
    if constexpr (F == SV_PASS_W4_I8)
      ars = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(it.xscale), 0, m * 4,
                                              0x00020000);
    xrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(it.x), 0, m * it.K * Fmt<F>::XE,
                                            0x00020000);
  };
  // ---- compute cursor: the item and chunk computed next ----
  int c_item = ib, c_c = 0;
  int c_K = 128, c_N = 16, c_t0 = 0, c_nchunk = 1;
  bool c_stats = false;
  __amdgpu_buffer_rsrc_t yrs = wrs, zrs = wrs;
  auto load_compute_item = [&](int idx) {
    const PlanItem it = items[idx];
    c_K = it.K;
    c_N = it.N;
    c_t0 = it.tile0;
    c_nchunk = it.nchunk;
    yrs = __builtin_amdgcn_make_buffer_rsrc(it.y, 0, m * it.N * 4, 0x00020000);
    if constexpr (ST) {
      c_stats = it.stats != nullptr;
      zrs = __builtin_amdgcn_make_buffer_rsrc(it.stats, 0, m * ceil_div(it.N, 64) * 8,
                                              0x00020000);
    }
  };
  if (ib < ie) {
    load_w_item(ib);
    load_issue_item(ib);
    load_compute_item(ib);
  }

  sv_u32x4 wb[P][kTW][kNB];
  sv_f32x4 yacc[kTW][MT];
  sv_f32x4 xacc[MT];                            // W8: running activation row sums
#pragma unroll
  for (int a = 0; a < MT; ++a) {
    xacc[a] = fz;
#pragma unroll
    for (int t = 0; t < kTW; ++t) yacc[t][a] = fz;
  }

  // The activation, record and item-end loads of the LDS cursor's chunk into
  // `slot` (out-of-range offsets once the cursor has run past the last
  // item), activations first.
  int nvalid[P];                                // weight blocks of the chunk in each slot within K
#pragma unroll
  for (int i = 0; i < P; ++i) nvalid[i] = 0;
  auto issue_lds = [&](const int slot) {
    const bool live = i_item < ie;
    const int KB = i_K / Fmt<F>::KPB;           // weight blocks per tile row
    const int jb = i_c * kNB;
    const int ntile = i_N >> 4;
    uint8_t* const sl = lds + slot * G::SLOT;
    nvalid[slot] = live ? (KB - jb < kNB ? KB - jb : kNB) : 0;
    // activations first: W4 waits for them one step ahead of the rest
    const int k0 = i_c * G::KC;
#pragma unroll
    for (int i = 0; i < G::XD; ++i) {
      // rows RPP p .. RPP p + RPP - 1 of the chunk; lane -> row RPP p +
      // lane / CPR, stored column lane % CPR, read from column
      // (lane % CPR) ^ (row % 16).  Rows >= m are not read (they only feed
      // discarded output rows); columns past K land in the next row (never
      // read) or fail the range check.
      const int piece = wave + kWaves * i;
      const int r = G::RPP * piece + lane / G::CPR;
      const int jj = (lane % G::CPR) ^ (r & 15);
      const unsigned int off = live && r < m && r < 16 * MT
                                   ? (r * i_K + k0) * Fmt<F>::XE + jj * 16
                                   : kSvOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (sv_lds_void*)(sl + piece * 1024), 16, off,
                                               0, 0, 0);
    }
    if constexpr (Fmt<F>::SZD) {
      // scale/zero records of this wave's tiles, one 128-byte record per
      // (tile, 128-wide k block): lane -> tile lane / 16, block (lane / 8) % 2,
      // 16-byte piece lane % 8
      const int tw = lane >> 4, bb = (lane >> 3) & 1;
      const int tile = i_t0 + wave * kTW + tw;
      const bool ok = live && tile < ntile && jb + bb < KB;
      const unsigned int off =
          ok ? sv_pk_block(tile, jb + bb, KB, ntile) * 128 + (lane & 7) * 16 : kSvOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          srs, (sv_lds_void*)(sl + G::XBUF + wave * 1024), 16, off, 0, 0, kStream);
    }
    if constexpr (F == SV_PASS_W8) {
      // the 64 channel scales of this wave's tiles (lanes 0-7, 16 bytes each)
      const bool ok = live && lane < 8 && i_t0 + wave * kTW + (lane >> 1) < ntile;
      const unsigned int off = ok ? (i_t0 + wave * kTW) * 32 + lane * 16 : kSvOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ars, (sv_lds_void*)(sl + G::XBUF + G::SZBUF + wave * 1024), 16, off, 0, 0, 0);
    }
    if constexpr (F == SV_PASS_W4_I8) {
      // the row scales (lanes 0 .. 4 MT - 1, four rows each)
      const bool ok = live && lane < 4 * MT;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ars, (sv_lds_void*)(sl + G::XBUF + G::SZBUF + wave * 1024), 16,
          ok ? lane * 16 : kSvOutOfRange, 0, 0, 0);
    }
  };
  // The weight loads of the weight cursor's chunk into `slot`'s registers:
  // one 1 KiB block per tile and k block, already in MFMA operand order.
  auto issue_w = [&](const int slot) {
    const bool live = w_item < ie;
    const int KB = w_K / Fmt<F>::KPB;           // weight blocks per tile row
    const int jb = w_c * kNB;
    const int ntile = w_N >> 4;
#pragma unroll
    for (int tw = 0; tw < kTW; ++tw) {
      const int tile = w_t0 + wave * kTW + tw;
#pragma unroll
      for (int b = 0; b < kNB; ++b) {
        const bool ok = live && tile < ntile && jb + b < KB;
        wb[slot][tw][b] = __builtin_amdgcn_raw_buffer_load_b128(
            wrs, ok ? lane * 16 : kSvOutOfRange,
            ok ? sv_pk_block(tile, jb + b, KB, ntile) * 1024 : 0, kStream);
      }
    }
  };
  auto advance_w = [&]() {
    if (++w_c == w_nchunk) {
      w_c = 0;
      if (++w_item < ie) load_w_item(w_item);
    }
  };
  auto advance_issue = [&]() {
    if (++i_c == i_nchunk) {
      i_c = 0;
      if (++i_item < ie) load_issue_item(i_item);
    }
  };

  // Byte offset of this lane's 16-byte A operand for logical column j of
  // row col (+ 16 a rows): swizzled column j ^ col.
  auto aaddr = [&](const int j) { return col * G::XROW + ((j ^ col) << 4); };

  // W4: the group row sums of the activation chunk in `slot`, formed once per
  // workgroup: wave w < 4 MT takes row tile w / 4 and group w % 4 of the
  // chunk (two MFMAs with an all-ones A operand put the sum of row col on
  // lane (col, q)) and writes 16 binary32 sums; groups past K are 0.  Read
  // by every wave after the next barrier.
  auto row_sums = [&](const int slot) {
    if constexpr (F == SV_PASS_W4) {
      if (wave < 4 * MT) {
        const int a = wave >> 2, g = wave & 3, b = g >> 1, h = g & 1;
        const uint8_t* ap = lds + slot * G::SLOT + a * 16 * G::XROW;
        const sv_u32x4 x0 =
            *reinterpret_cast<const sv_u32x4*>(ap + aaddr(16 * b + 8 * h + 2 * q));
        const sv_u32x4 x1 =
            *reinterpret_cast<const sv_u32x4*>(ap + aaddr(16 * b + 8 * h + 2 * q + 1));
        sv_f32x4 xt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sv_as_bf16x8(ones),
                                                              sv_as_bf16x8(x0), fz, 0, 0, 0);
        xt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sv_as_bf16x8(ones), sv_as_bf16x8(x1), xt, 0,
                                                     0, 0);
        const float v = b < nvalid[slot] ? xt[0] : 0.0f;
        if (q == 0) xsb[slot * MT * 64 + (a * 4 + g) * 16 + col] = v;
      }
    }
  };

  auto compute = [&](const int slot) {
    const int KB = c_K / Fmt<F>::KPB;
    const int jb = c_c * kNB;
    const uint8_t* const sl = lds + slot * G::SLOT;
    // W4_I8: row sums of the step's 4 groups, lane (col, q) holding row col
    // of group q (the A operand layout of v_mfma_f32_16x16x4_f32)
    float xsum[MT];
#pragma unroll
    for (int a = 0; a < MT; ++a) xsum[a] = 0.f;
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      if (jb + b >= KB) break;
      if constexpr (F == SV_PASS_W4) {
        const uint8_t* sp = sl + G::XBUF + wave * 1024 + col * 8;
#pragma unroll
        for (int h = 0; h < 2; ++h) {           // the two groups of the block
          sv_u32x4 a0[MT], a1[MT];
#pragma unroll
          for (int a = 0; a < MT; ++a) {
            const uint8_t* ap = sl + a * 16 * G::XROW;
            a0[a] = *reinterpret_cast<const sv_u32x4*>(ap + aaddr(16 * b + 8 * h + 2 * q));
            a1[a] = *reinterpret_cast<const sv_u32x4*>(ap + aaddr(16 * b + 8 * h + 2 * q + 1));
          }
#pragma unroll
          for (int tw = 0; tw < kTW; ++tw) {
            const sv_u32x4 w = wb[slot][tw][b];
            const sv_u32x4 b0 = sv_w4_dequant8(h ? w.z : w.x, magic);
            const sv_u32x4 b1 = sv_w4_dequant8(h ? w.w : w.y, magic);
            const sv_u32x2 sbt =
                *reinterpret_cast<const sv_u32x2*>(sp + (tw * kNB + b) * 128);
            const float sc = sv_materialize(sv_half_lo(h ? sbt.y : sbt.x));
#pragma unroll
            for (int a = 0; a < MT; ++a) {
              sv_f32x4 acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  sv_as_bf16x8(a0[a]), sv_as_bf16x8(b0), fz, 0, 0, 0);
              acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sv_as_bf16x8(a1[a]),
                                                            sv_as_bf16x8(b1), acc, 0, 0, 0);
              // acc = sum x (128 + c): the bias and zero point leave through
              // the correction below
#pragma unroll
              for (int i = 0; i < 4; ++i) yacc[tw][a][i] = fmaf(sc, acc[i], yacc[tw][a][i]);
            }
          }
        }
      } else if constexpr (F == SV_PASS_W8) {
        sv_u32x4 a0[MT], a1[MT];
#pragma unroll
        for (int a = 0; a < MT; ++a) {
          const uint8_t* ap = sl + a * 16 * G::XROW;
          a0[a] = *reinterpret_cast<const sv_u32x4*>(ap + aaddr(8 * b + 2 * q));
          a1[a] = *reinterpret_cast<const sv_u32x4*>(ap + aaddr(8 * b + 2 * q + 1));
          xacc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sv_as_bf16x8(a0[a]),
                                                            sv_as_bf16x8(ones), xacc[a], 0, 0, 0);
          xacc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sv_as_bf16x8(a1[a]),
                                                            sv_as_bf16x8(ones), xacc[a], 0, 0, 0);
        }
#pragma unroll
        for (int tw = 0; tw < kTW; ++tw) {
          const sv_u32x4 w = wb[slot][tw][b];
          const sv_u32x2 l0 = w8_cvt4(w.x), l1 = w8_cvt4(w.y);
          const sv_u32x2 h0 = w8_cvt4(w.z), h1 = w8_cvt4(w.w);
          const sv_u32x4 b0 = {l0.x, l0.y, l1.x, l1.y};
          const sv_u32x4 b1 = {h0.x, h0.y, h1.x, h1.y};
#pragma unroll
          for (int a = 0; a < MT; ++a) {
            yacc[tw][a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                sv_as_bf16x8(a0[a]), sv_as_bf16x8(b0), yacc[tw][a], 0, 0, 0);
            yacc[tw][a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                sv_as_bf16x8(a1[a]), sv_as_bf16x8(b1), yacc[tw][a], 0, 0, 0);
          }
        }
      } else {                                  // SV_PASS_W4_I8
        const uint8_t* sp = sl + G::XBUF + wave * 1024 + col * 8;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          sv_u32x4 a8[MT];
#pragma unroll
          for (int a = 0; a < MT; ++a) {
            a8[a] = *reinterpret_cast<const sv_u32x4*>(sl + a * 16 * G::XROW +
                                                       aaddr(8 * b + 4 * h + q));
            // exact group sums Xg with the rows along N (all-ones A operand):
            // lane (col, q) receives row col; the lanes with q = group index
            // of the step keep it for the correction below
            const sv_i32x4 g = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                sv_as_i32x4(ones8), sv_as_i32x4(a8[a]), iz, 0, 0, 0);
            if (q == 2 * b + h) xsum[a] = static_cast<float>(g[0]);
          }
#pragma unroll
          for (int tw = 0; tw < kTW; ++tw) {
            const sv_u32x4 w = wb[slot][tw][b];
            const unsigned int wx = h ? w.z : w.x, wy = h ? w.w : w.y;
            // packed word (byte b = codes b | b+4 << 4): low nibbles are codes
            // 0..3, high nibbles 4..7, as bytes in natural order
            const sv_u32x4 bw = {wx & 0x0F0F0F0Fu, (wx >> 4) & 0x0F0F0F0Fu, wy & 0x0F0F0F0Fu,
                                 (wy >> 4) & 0x0F0F0F0Fu};
            const sv_u32x2 sbt =
                *reinterpret_cast<const sv_u32x2*>(sp + (tw * kNB + b) * 128);
            const float sc = sv_materialize(sv_half_lo(h ? sbt.y : sbt.x));
#pragma unroll
            for (int a = 0; a < MT; ++a) {
              const sv_i32x4 I = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                  sv_as_i32x4(a8[a]), sv_as_i32x4(bw), iz, 0, 0, 0);
              // I = sum c xq exactly; the zero point leaves through the
              // correction below
#pragma unroll
              for (int i = 0; i < 4; ++i)
                yacc[tw][a][i] = fmaf(sc, static_cast<float>(I[i]), yacc[tw][a][i]);
            }
          }
        }
      }
    }
    if constexpr (F != SV_PASS_W8) {
      // Zero point (and, for bf16 codes, the 128 bias) of the step's 4
      // groups in one rank-4 update: yacc -= sum_g xsum[row, g] * s[n, g]
      // (bias + z[n, g]), with lane (col, q) supplying channel col of group q
      // as the B operand.  Binary32 products and sums; for a one-hot row
      // both terms are exact and so is their difference (c - z) s.
      constexpr float kBias = F == SV_PASS_W4 ? 128.0f : 0.0f;
      const int bq = q >> 1;
      const uint8_t* sp = sl + G::XBUF + wave * 1024 + col * 8 + (q & 1) * 4;
      // all records are read (the slot always holds them, stale past K) and
      // groups past K select 0, so no lane-dependent branch splits the reads
      const float gmask = jb + bq < KB ? 1.0f : 0.0f;
      if constexpr (F == SV_PASS_W4) {
        // the shared group row sums of this chunk (zero past K): lane
        // (col, q) takes row col of group q
#pragma unroll
        for (int a = 0; a < MT; ++a) xsum[a] = xsb[slot * MT * 64 + (a * 4 + q) * 16 + col];
      }
      unsigned int szq[kTW];
#pragma unroll
      for (int tw = 0; tw < kTW; ++tw)
        szq[tw] = *reinterpret_cast<const unsigned int*>(sp + (tw * kNB + bq) * 128);
#pragma unroll
      for (int tw = 0; tw < kTW; ++tw) {
        const float v = -(sv_half_lo(szq[tw]) * (kBias + sv_half_hi(szq[tw])));
        const float nsz = gmask != 0.0f ? v : 0.0f;   // not v * 0: stale bits may be inf/NaN
#pragma unroll
        for (int a = 0; a < MT; ++a)
          yacc[tw][a] = __builtin_amdgcn_mfma_f32_16x16x4f32(xsum[a], nsz, yacc[tw][a], 0, 0, 0);
      }
    }
  };

  // On an item's last chunk: the epilogue of the format, then the wave's
  // 16 rows x 64 channels (its 4 tiles; lane (col, q) of an MFMA output holds
  // rows 4q .. 4q+3 of channel col) go through the wave's LDS transpose area
  // and come back into yacc so that each of the 4 MT stores writes 4 whole
  // rows of 256 contiguous bytes (lane l: row l / 16, channels 4 (l % 16) ..
  // +3), i.e. full cache lines.
  auto store = [&](const int slot) {
    const int ch = 4 * (lane & 15);             // this lane's 4 channels in the wave's 64
    const uint8_t* aux = lds + slot * G::SLOT + G::XBUF + G::SZBUF + wave * 1024;
#pragma unroll
    for (int a = 0; a < MT; ++a) {
#pragma unroll
      for (int tw = 0; tw < kTW; ++tw) {
        sv_f32x4 v = yacc[tw][a];
        if constexpr (F == SV_PASS_W8) {
          const float sc = __half2float(
              *reinterpret_cast<const __half*>(aux + (tw * 16 + col) * 2));
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = sc * fmaf(-128.0f, xacc[a][i], v[i]);
        }
        if constexpr (F == SV_PASS_W4_I8) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            v[i] *= *reinterpret_cast<const float*>(aux + (16 * a + 4 * q + i) * 4);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) tpose[(4 * q + i) * 64 + tw * 16 + col] = v[i];
      }
      // Lanes read what other lanes wrote: LDS operations of a wave execute
      // in order, so it is enough that the compiler keeps program order
      // (it may not move these accesses across the fence).
      sv_compiler_fence();
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        yacc[rr][a] = *reinterpret_cast<const sv_f32x4*>(tpose + (4 * rr + (lane >> 4)) * 64 + ch);
      sv_compiler_fence();                    // before the next 16 rows overwrite the area
    }
    const bool ch_ok = c_t0 + wave * kTW + (ch >> 4) < (c_N >> 4);
#pragma unroll
    for (int a = 0; a < MT; ++a) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int r = 16 * a + 4 * rr + (lane >> 4);
        const unsigned int off = ch_ok && r < m
                                     ? (r * c_N + 16 * (c_t0 + wave * kTW) + ch) * 4
                                     : kSvOutOfRange;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(sv_u32x4, yacc[rr][a]), yrs,
                                               off, 0, kStream);
      }
    }
    if (ST && c_stats) {
      // Row r's 64 channels of this wave sit in the 16 lanes of lane >> 4 ==
      // (r % 16) / 4 ... (4 each): max, then sum of exp(y - max) over the
      // 16 lanes.  A NaN or +inf makes the sum NaN (the row is invalid);
      // missing channels count as -inf.
      const int grp = (c_t0 + wave * kTW) >> 2;
      const int ngrp = ceil_div(c_N, 64);
#pragma unroll
      for (int a = 0; a < MT; ++a) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int r = 16 * a + 4 * rr + (lane >> 4);
          sv_f32x4 v = yacc[rr][a];
          bool bad = false;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            bad |= (v[i] != v[i]) | (v[i] == INFINITY);
            v[i] = ch_ok ? v[i] : -INFINITY;
          }
          float mx = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
          float sm = 0.f;
          if (mx != -INFINITY) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              sm += __builtin_amdgcn_exp2f((v[i] - mx) * 1.4426950408889634f);
          }
          sm = ch_ok && bad ? __builtin_nanf("") : sm;
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) sm += __shfl_xor(sm, o);
          const unsigned int off = (lane & 15) == 0 && r < m && grp < ngrp
                                       ? static_cast<unsigned int>(r * ngrp + grp) * 8
                                       : kSvOutOfRange;
          sv_u32x2 pr;
          pr.x = __float_as_uint(mx);
          pr.y = __float_as_uint(sm);
          __builtin_amdgcn_raw_buffer_store_b64(pr, zrs, off, 0, kStream);
        }
      }
    }
#pragma unroll
    for (int a = 0; a < MT; ++a) {
      xacc[a] = fz;
#pragma unroll
      for (int t = 0; t < kTW; ++t) yacc[t][a] = fz;
    }
  };
  auto advance_compute = [&]() {
    if (++c_c == c_nchunk) {
      c_c = 0;
      if (++c_item < ie) load_compute_item(c_item);
    }
  };

  // Prologue: chunks 0 .. P - 2 in flight, and the weights of chunk P - 1.
#pragma unroll
  for (int i = 0; i < P - 1; ++i) {
    issue_w(i);
    advance_w();
    issue_lds(i);
    advance_issue();
    sv_compiler_fence();
  }
  issue_w(P - 1);
  advance_w();
  sv_compiler_fence();
  if constexpr (F == SV_PASS_W4) {
    sv_wait_vmcnt<WAIT0>();                     // activations of chunk 0, every wave
    sv_barrier_no_fence();
    row_sums(0);
  }
  for (int s0 = 0; s0 < steps; s0 += P) {
#pragma unroll
    for (int s = 0; s < P; ++s) {
      // chunk s0 + s has landed in slot s (registers and LDS) for every wave,
      // and every wave has finished the chunk that last used the LDS of
      // slot s + P - 1;
      // W4: the activations of chunk s0 + s + 1 have landed too, and the
      // row sums of chunk s0 + s (formed in the previous step) are visible
      sv_wait_vmcnt<WAITS>();
      sv_barrier_no_fence();
      issue_lds((s + P - 1) % P);
      advance_issue();
      sv_compiler_fence();
      row_sums((s + 1) % P);                    // W4: activations of chunk s0 + s + 1 have landed
      const bool run = s0 + s < steps;
      const bool at_end = run && c_c == c_nchunk - 1;
      if (run) compute(s);
      sv_compiler_fence();
      issue_w(s);                               // chunk s0 + s + P into the registers just freed
      advance_w();
      sv_compiler_fence();
      if (at_end) store(s);
      if (run) advance_compute();
    }
  }
  // Drain every outstanding load (including buffer -> LDS copies) before the
  // workgroup's LDS can be handed to another workgroup.
  sv_wait_vmcnt<0>();
  sv_barrier_no_fence();
}

template <int F, int MT, int P, bool ST>
sv_status launch_pass(const void* plan, int m, int grid, hipStream_t st) {
  auto kern = pass_kernel<F, MT, P, ST>;
  constexpr int kLds = pass_lds_bytes<F, MT, P>();
  static_assert(kLds <= 160 * 1024, "LDS budget of a gfx950 workgroup");
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kLds) != hipSuccess)
    return SV_ERR_HIP;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), kLds, st,
                     static_cast<const uint8_t*>(plan), m);
  SV_LAUNCH_CHECK();
  return SV_OK;
}

// Plans made by this library, by buffer: the id of the last plan written into
// each plan buffer.  sv_pass_run refuses an sv_pass whose plan buffer has
// since been planned again (its id is no longer the buffer's).
std::mutex g_plan_mu;
std::unordered_map<const void*, uint32_t> g_plan_ids;
uint32_t g_plan_next = 0;

sv_status check_gemms(int format, const sv_pass_gemm* gemms, int count, int m,
                      long long* n_items) {
  if (format != SV_PASS_W4 && format != SV_PASS_W8 && format != SV_PASS_W4_I8)
    return SV_ERR_INVALID_ARG;
  if (!gemms) return SV_ERR_NULL;
  if (count < 1 || m < 1 || m > SV_MAX_ROWS) return SV_ERR_INVALID_ARG;
  const int kpb = fmt_kpb(format), xe = fmt_xe(format);
  long long items = 0;
  for (int g = 0; g < count; ++g) {
    const sv_pass_gemm& e = gemms[g];
    if (!e.x || !e.codes || !e.scales || !e.y) return SV_ERR_NULL;
    if ((format == SV_PASS_W4_I8) != (e.xscale != nullptr))
      return e.xscale ? SV_ERR_INVALID_ARG : SV_ERR_NULL;
    if (e.N < 16 || e.N % 16 != 0 || e.K < kpb || e.K % kpb != 0) return SV_ERR_INVALID_ARG;
    // buffer ranges are 32-bit: codes, activations and outputs below 2 GiB
    const long long code_bytes = static_cast<long long>(e.N) * e.K / (format == SV_PASS_W8 ? 1 : 2);
    if (code_bytes >= (1LL << 31) || static_cast<long long>(m) * e.K * xe >= (1LL << 31) ||
        static_cast<long long>(m) * e.N * 4 >= (1LL << 31))
      return SV_ERR_UNSUPPORTED;
    if (e.stats && static_cast<long long>(m) * ceil_div(e.N, 64) * 8 >= (1LL << 31))
      return SV_ERR_UNSUPPORTED;
    if (!sv_aligned16(e.x) || !sv_aligned16(e.codes) || !sv_aligned16(e.scales) ||
        !sv_aligned16(e.y) || (e.xscale && !sv_aligned16(e.xscale)) ||
        (e.stats && !sv_aligned16(e.stats)))
      return SV_ERR_ALIGN;
    items += ceil_div(e.N / 16, kItemTiles);
  }
  if (items >= (1LL << 30)) return SV_ERR_UNSUPPORTED;
  *n_items = items;
  return SV_OK;
}

}  // namespace

uint32_t sv_register_plan(const void* plan);

extern "C" size_t sv_pass_plan_bytes(int format, const sv_pass_gemm* gemms, int count, int m) {
  long long items = 0;
  if (check_gemms(format, gemms, count, m, &items) != SV_OK) return 0;
  return kItemsOff + static_cast<size_t>(items) * sizeof(PlanItem);
}

extern "C" sv_status sv_pass_plan(int format, const sv_pass_gemm* gemms, int count, int m,
                                  int group, void* plan, size_t plan_bytes, sv_pass* pass,
                                  hipStream_t stream) {
  long long n_items = 0;
  const sv_status st = check_gemms(format, gemms, count, m, &n_items);
  if (st != SV_OK) return st;
  if (!plan || !pass) return SV_ERR_NULL;
  if (format != SV_PASS_W8 && group != kGroup) return SV_ERR_UNSUPPORTED;
  if (!sv_aligned16(plan)) return SV_ERR_ALIGN;
  const size_t need = kItemsOff + static_cast<size_t>(n_items) * sizeof(PlanItem);
  if (plan_bytes < need) return SV_ERR_WORKSPACE;

  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    return SV_ERR_HIP;
  // One workgroup of 8 waves per compute unit; never more workgroups than items.
  const int grid = static_cast<int>(std::min<long long>({cus, kMaxGrid, n_items}));
  const int kc = kNB * fmt_kpb(format);

  int any_stats = 0;
  for (int g = 0; g < count; ++g) any_stats |= gemms[g].stats != nullptr;
  // Items in pass order.
  std::vector<PlanItem> items;
  items.reserve(static_cast<size_t>(n_items));
  for (int g = 0; g < count; ++g) {
    const sv_pass_gemm& e = gemms[g];
    const int tiles = e.N / 16;
    for (int t0 = 0; t0 < tiles; t0 += kItemTiles)
      items.push_back(PlanItem{e.x, e.xscale, e.codes, e.scales, e.y, e.K, e.N, t0,
                               ceil_div(e.K, kc), e.stats});
  }
  // Longest-first greedy: each item (by chunk count, ties in pass order) goes
  // to the workgroup with the fewest chunks so far (ties: lowest index).
  std::vector<int> order(items.size());
  for (size_t i = 0; i < order.size(); ++i) order[i] = static_cast<int>(i);
  std::stable_sort(order.begin(), order.end(),
                   [&](int a, int b) { return items[a].nchunk > items[b].nchunk; });
  typedef std::pair<long long, int> Load;
  std::priority_queue<Load, std::vector<Load>, std::greater<Load>> heap;
  for (int w = 0; w < grid; ++w) heap.push(Load(0, w));
  std::vector<std::vector<int>> owned(grid);
  for (int i : order) {
    Load l = heap.top();
    heap.pop();
    owned[l.second].push_back(i);
    l.first += items[i].nchunk;
    heap.push(l);
  }

  std::vector<uint8_t> image(need, 0);
  PlanHeader* hdr = reinterpret_cast<PlanHeader*>(image.data());
  int32_t* wg_begin = reinterpret_cast<int32_t*>(image.data() + kBeginOff);
  int32_t* wg_steps = reinterpret_cast<int32_t*>(image.data() + kStepsOff);
  PlanItem* out = reinterpret_cast<PlanItem*>(image.data() + kItemsOff);
  int pos = 0, max_steps = 0;
  for (int w = 0; w < grid; ++w) {
    std::sort(owned[w].begin(), owned[w].end());   // pass order inside a workgroup
    wg_begin[w] = pos;
    long long s = 0;
    for (int i : owned[w]) {
      out[pos++] = items[i];
      s += items[i].nchunk;
    }
    if (s >= (1LL << 30)) return SV_ERR_UNSUPPORTED;
    wg_steps[w] = static_cast<int32_t>(s);
    max_steps = std::max(max_steps, static_cast<int>(s));
  }
  wg_begin[grid] = pos;
  hdr->magic = kPlanMagic;
  hdr->version = kPlanVersion;
  hdr->format = format;
  hdr->m = m;
  hdr->count = count;
  hdr->grid = grid;
  hdr->items = static_cast<int32_t>(n_items);
  hdr->max_steps = max_steps;
  hdr->stats = any_stats;

  // Plan upload: a setup step (like packing the weights), synchronous so the
  // host image can be released.
  if (hipMemcpyAsync(plan, image.data(), need, hipMemcpyHostToDevice, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return SV_ERR_HIP;
  pass->plan = plan;
  pass->format = format;
  pass->m = m;
  pass->count = count;
  pass->grid = grid;
  pass->items = static_cast<int>(n_items);
  pass->max_steps = max_steps;
  pass->stats = any_stats;
  pass->chain = 0;
  pass->id = sv_register_plan(plan);
  return SV_OK;
}

namespace {
template <bool ST>
sv_status dispatch_pass(const sv_pass* pass, hipStream_t stream) {
  // Two activation tiles for m > 16.  The ring keeps three chunks in flight
  // (two for the 4-bit bf16 path at m > 16, whose registers would not hold a
  // third).
  const bool two = pass->m > 16;
  switch (pass->format) {
    case SV_PASS_W4:
      return two ? launch_pass<SV_PASS_W4, 2, 3, ST>(pass->plan, pass->m, pass->grid, stream)
                 : launch_pass<SV_PASS_W4, 1, 4, ST>(pass->plan, pass->m, pass->grid, stream);
    case SV_PASS_W8:
      return two ? launch_pass<SV_PASS_W8, 2, 4, ST>(pass->plan, pass->m, pass->grid, stream)
                 : launch_pass<SV_PASS_W8, 1, 4, ST>(pass->plan, pass->m, pass->grid, stream);
    case SV_PASS_W4_I8:
      return two ? launch_pass<SV_PASS_W4_I8, 2, 4, ST>(pass->plan, pass->m, pass->grid, stream)
                 : launch_pass<SV_PASS_W4_I8, 1, 4, ST>(pass->plan, pass->m, pass->grid, stream);
    default:
      return SV_ERR_INVALID_ARG;
  }
}
}  // namespace

sv_status sv_chain_run(const sv_pass* pass, hipStream_t stream);   // pass_chain.hip
size_t sv_chain_status_offset(const sv_pass* pass);                 // pass_chain.hip

uint32_t sv_register_plan(const void* plan) {
  std::lock_guard<std::mutex> lock(g_plan_mu);
  if (++g_plan_next == 0) ++g_plan_next;        // ids are never 0
  g_plan_ids[plan] = g_plan_next;
  return g_plan_next;
}

static bool plan_is_current(const sv_pass* pass) {
  std::lock_guard<std::mutex> lock(g_plan_mu);
  const auto it = g_plan_ids.find(pass->plan);
  return it != g_plan_ids.end() && it->second == pass->id;
}

extern "C" sv_status sv_pass_run(const sv_pass* pass, hipStream_t stream) {
  if (!pass || !pass->plan) return SV_ERR_NULL;
  if (!sv_aligned16(pass->plan)) return SV_ERR_ALIGN;
  if (!plan_is_current(pass)) return SV_ERR_INVALID_ARG;   // stale: the buffer was re-planned
  if (pass->chain) {
    if (pass->m < 1 || pass->m > SV_MAX_ROWS) return SV_ERR_INVALID_ARG;
    return sv_chain_run(pass, stream);
  }
  if (pass->m < 1 || pass->m > SV_MAX_ROWS || pass->grid < 1 || pass->grid > kMaxGrid)
    return SV_ERR_INVALID_ARG;
  return pass->stats ? dispatch_pass<true>(pass, stream) : dispatch_pass<false>(pass, stream);
}

extern "C" sv_status sv_pass_status(const sv_pass* pass, uint32_t* status, hipStream_t stream) {
  if (!pass || !pass->plan || !status) return SV_ERR_NULL;
  if (!sv_aligned16(pass->plan)) return SV_ERR_ALIGN;
  uint32_t v = 0;
  const size_t off = pass->chain ? sv_chain_status_offset(pass) : SV_PASS_STATUS_OFFSET;
  if (hipMemcpyAsync(&v, static_cast<const uint8_t*>(pass->plan) + off,
                     sizeof(v), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return SV_ERR_HIP;
  *status = v;
  return SV_OK;
}

// ---- W8 packing -------------------------------------------------------------
namespace {
// One 16-byte piece per thread: block (t, j), lane l of the wave that reads it.
__global__ void pack_w8_kernel(const int8_t* __restrict__ codes, int N, int K,
                               uint8_t* __restrict__ out) {
  const size_t piece = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int KB = K / 64;
  const size_t total = static_cast<size_t>(N / 16) * KB * 64;
  if (piece >= total) return;
  const int l = static_cast<int>(piece & 63);
  const size_t blk = piece >> 6;
  const int j = static_cast<int>(blk % KB);
  const int t = static_cast<int>(blk / KB);
  const int n = 16 * t + (l & 15), q = l >> 4;
  const sv_u32x4 v = sv_ld16(codes + static_cast<size_t>(n) * K + 64 * j + 16 * q);
  const size_t dst = static_cast<size_t>(sv_pk_block(t, j, KB, N / 16)) * 1024 + l * 16;
  *reinterpret_cast<sv_u32x4*>(out + dst) = v;
}
}  // namespace

extern "C" sv_status sv_w8_pack(const int8_t* codes, int N, int K, uint8_t* packed_codes,
                                hipStream_t stream) {
  if (!codes || !packed_codes) return SV_ERR_NULL;
  if (N < 16 || N % 16 != 0 || K < 64 || K % 64 != 0) return SV_ERR_INVALID_ARG;
  if (!sv_aligned16(codes) || !sv_aligned16(packed_codes)) return SV_ERR_ALIGN;
  const size_t pieces = static_cast<size_t>(N / 16) * (K / 64) * 64;
  hipLaunchKernelGGL(pack_w8_kernel, dim3(static_cast<unsigned>((pieces + 255) / 256)),
                     dim3(256), 0, stream, codes, N, K, packed_codes);
  SV_LAUNCH_CHECK();
  return SV_OK;
}
