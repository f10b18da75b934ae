// sv_w4_pass_plan + sv_qgemm_w4_pass: every W4 GEMM of one verify pass in a
// single persistent launch.
//
// Source: Karpathy's Trick for Faster Local LLMs, "Why batch-one decoding is
// memory-bound" (a pass streams every weight once, so its speed is bandwidth
// divided by the bytes of the weights) and "How Uzu optimizes bytes and tokens
// per pass" (4-bit asymmetric group quantization; kernels and checkpoint
// format designed together); Speculative Decoding Clearly Explained, "Check
// the guesses together" (all draft positions scored in one pass).
//
// Why one launch: a pass of a 9B-class stack is ~128 GEMMs of 9-57 MB each.
// Launched one by one, each pays the ramp-up and drain of a kernel over 256
// compute units (several microseconds apiece), and the HBM stream stops at
// every boundary.  Here each workgroup owns a fixed list of work items from
// all GEMMs and streams them back to back through one software pipeline, so
// the weight stream never stops between GEMMs.
//
// Work item = one GEMM x 16 row tiles (256 output channels) x all of K.
// Inside an item each of the 8 waves owns 2 row tiles for the whole K, so no
// cross-wave reduction is needed; the item advances in chunks of 512 k:
//   * activations of the chunk (16 or 32 rows x 1 KiB) are copied once per
//     workgroup into LDS by buffer -> LDS loads and shared by the 16 tiles
//     (activation bytes per weight byte: 4m / (16 * 16));
//   * each wave loads its 2 tiles x 4 k blocks of codes (1 KiB per block, one
//     fully contiguous 16-byte-per-lane load each) into registers, and its
//     tiles' scales/zeros (1 KiB) into its own LDS region;
//   * dequantization and MFMA as in sv_qgemm_w4_packed: bf16 128 + c from a
//     mask and a byte permute, v_mfma_f32_16x16x32_bf16 with A = draft rows,
//     an all-ones MFMA for the per-group row sums, and the fold
//     y += s * (acc - (128 + z) * xsum) in binary32.
// Chunks flow through a ring of P slots: while chunk c computes, chunks
// c+1 .. c+P-1 are in flight.  Every step issues the same number of vector
// memory instructions (loads with out-of-range offsets where a tile, block or
// row does not exist; the item's output stores on every step, out of range
// except on an item's last chunk), so one compile-time vmcnt wait is exact.
//
// The plan (built on the host once, like the packed weights) lists the items
// of every workgroup, balanced by chunk count with a longest-first greedy
// assignment and kept in pass order inside each workgroup.
#include <algorithm>
#include <functional>
#include <queue>
#include <vector>

#include "w4_packed_dev.h"

namespace {

constexpr uint32_t kPlanMagic = 0x50575653u;   // "SVWP"
constexpr uint32_t kPlanVersion = 1;
constexpr int kMaxGrid = 2048;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kNB = 2;                          // 128-wide k blocks per chunk
constexpr int kKC = 128 * kNB;                  // k per chunk
constexpr int kRowBytes = 2 * kKC;              // bytes of one activation row of a chunk
constexpr int kTW = 4;                          // row tiles per wave
constexpr int kItemTiles = kWaves * kTW;        // row tiles per item (512 channels)
constexpr int kGroup = 64;

struct PlanHeader {                             // 64 bytes
  uint32_t magic, version;
  int32_t m, count, grid, items, max_steps, reserved0;
  uint64_t reserved[4];
};
struct PlanItem {                               // 48 bytes
  const uint16_t* x;
  const uint8_t* pc;
  const uint16_t* psz;
  float* y;
  int32_t K, N, tile0, nchunk;
};
static_assert(sizeof(PlanHeader) == 64, "plan header layout");
static_assert(sizeof(PlanItem) == 48, "plan item layout");

// Plan image: header | wg_begin[kMaxGrid + 1] | wg_steps[kMaxGrid] | items.
constexpr size_t kBeginOff = sizeof(PlanHeader);
constexpr size_t kStepsOff = kBeginOff + sizeof(int32_t) * (kMaxGrid + 1);
constexpr size_t kItemsOff = (kStepsOff + sizeof(int32_t) * kMaxGrid + 63) / 64 * 64;

__host__ __device__ constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }

// LDS bytes of one instantiation: P activation slots, P scale/zero slots of
// 1 KiB per wave, and a 1 KiB output-transpose area per wave.
template <int MT, int P>
constexpr int pass_lds_bytes() {
  return P * 16 * MT * kRowBytes + P * kWaves * 1024 + kWaves * 1024;
}

template <int MT, int P>
__global__ __launch_bounds__(kThreads) void w4_pass_kernel(const uint8_t* __restrict__ plan,
                                                            int m) {
  constexpr int XBUF = 16 * MT * kRowBytes;     // bytes per activation slot
  constexpr int SZBUF = kWaves * 1024;          // bytes per scale/zero slot
  constexpr int XD = MT;                        // activation pieces (1 KiB = 2 rows) per wave
  constexpr int L = kTW * kNB + XD + 1;         // loads per wave per step
  constexpr int NS = kTW * MT;                  // 16-byte stores per wave per step
  // At the wait before computing chunk c, the operations issued after chunk
  // c's loads are the stores of that same step and the loads and stores of
  // the P - 2 steps after it.
  constexpr int WAITN = NS + (P - 2) * (L + NS);
  static_assert(WAITN < 64, "too many memory operations in flight for vmcnt");
  static_assert(kTW * kNB * 128 == 1024 && kRowBytes == 512,
                "one 1 KiB scale/zero load per wave; two activation rows per 1 KiB piece");
  extern __shared__ __align__(16) uint8_t lds[];

  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(plan);
  if (hdr->magic != kPlanMagic || hdr->m != m || hdr->grid != static_cast<int>(gridDim.x))
    return;                                     // stale or foreign plan: touch nothing
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
  const sv_f32x4 fz = {0.f, 0.f, 0.f, 0.f};
  uint8_t* const szl = lds + P * XBUF;
  float* const tpose = reinterpret_cast<float*>(lds + P * XBUF + P * SZBUF) + wave * 256;

  // Activation rows sit in LDS at 512-byte pitch with their 16-byte columns
  // permuted: column j of row r is stored at column j ^ (r & 15).  The 16
  // lanes that read one MFMA operand (rows r..r+15, same column) then hit 16
  // different bank groups.  Byte offset of this lane's A operand for group
  // half h and k-octet e inside a 128-wide block:
  int aoff[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 2; ++e) aoff[h][e] = col * kRowBytes + (((8 * h + 2 * q + e) ^ col) << 4);

  // ---- issue cursor: the item and chunk whose loads go out next ----
  int i_item = ib, i_c = 0;
  int i_K = 128, i_N = 16, i_t0 = 0, i_nchunk = 1;
  __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(nullptr, 0, 0, 0x00020000);
  __amdgpu_buffer_rsrc_t srs = wrs, xrs = wrs;
  auto load_issue_item = [&](int idx) {
    const PlanItem it = items[idx];
    i_K = it.K;
    i_N = it.N;
    i_t0 = it.tile0;
    i_nchunk = it.nchunk;
    wrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(it.pc), 0, it.N * (it.K / 2),
                                            0x00020000);
    srs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(it.psz), 0,
                                            it.N * (it.K / kGroup) * 4, 0x00020000);
    xrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(it.x), 0, m * it.K * 2,
                                            0x00020000);
  };
  // ---- compute cursor: the item and chunk computed next ----
  int c_item = ib, c_c = 0;
  int c_K = 128, c_N = 16, c_t0 = 0, c_nchunk = 1;
  __amdgpu_buffer_rsrc_t yrs = wrs;
  auto load_compute_item = [&](int idx) {
    const PlanItem it = items[idx];
    c_K = it.K;
    c_N = it.N;
    c_t0 = it.tile0;
    c_nchunk = it.nchunk;
    yrs = __builtin_amdgcn_make_buffer_rsrc(it.y, 0, m * it.N * 4, 0x00020000);
  };
  if (ib < ie) {
    load_issue_item(ib);
    load_compute_item(ib);
  }

  sv_u32x4 wb[P][kTW][kNB];
  sv_f32x4 yacc[kTW][MT];
#pragma unroll
  for (int t = 0; t < kTW; ++t)
#pragma unroll
    for (int a = 0; a < MT; ++a) yacc[t][a] = fz;

  // All L loads of the issue cursor's chunk into `slot` (out-of-range
  // offsets once the cursor has run past the last item).
  auto issue = [&](const int slot) {
    const bool live = i_item < ie;
    const int KB = i_K >> 7;
    const int jb = i_c * kNB;
    const int ntile = i_N >> 4;
#pragma unroll
    for (int tw = 0; tw < kTW; ++tw) {
      const int tile = i_t0 + wave * kTW + tw;
#pragma unroll
      for (int b = 0; b < kNB; ++b) {
        const bool ok = live && tile < ntile && jb + b < KB;
        wb[slot][tw][b] = __builtin_amdgcn_raw_buffer_load_b128(
            wrs, ok ? lane * 16 : kSvOutOfRange, ok ? (tile * KB + jb + b) * 1024 : 0, 0);
      }
    }
    {
      // scales/zeros of this wave's tiles for the chunk, one 128-byte record
      // per (tile, k block): lane -> tile lane / 16, block (lane / 8) % 2,
      // 16-byte piece lane % 8
      const int tw = lane >> 4, bb = (lane >> 3) & 1;
      const int tile = i_t0 + wave * kTW + tw;
      const bool ok = live && tile < ntile && jb + bb < KB;
      const unsigned int off =
          ok ? (tile * KB + jb + bb) * 128 + (lane & 7) * 16 : kSvOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          srs, (sv_lds_void*)(szl + slot * SZBUF + wave * 1024), 16, off, 0, 0, 0);
    }
    const int k0 = i_c * kKC;
#pragma unroll
    for (int i = 0; i < XD; ++i) {
      // rows 2p and 2p + 1 of the chunk; lane -> row 2p + lane / 32, stored
      // column lane % 32, read from column (lane % 32) ^ (row % 16).  Rows
      // >= m are not read (they only feed discarded output rows); columns
      // past K land in the next row (never read) or fail the range check.
      const int piece = wave + kWaves * i;
      const int r = 2 * piece + (lane >> 5);
      const int jj = (lane & 31) ^ (r & 15);
      const unsigned int off =
          live && r < m ? (r * i_K + k0) * 2 + jj * 16 : kSvOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xrs, (sv_lds_void*)(lds + slot * XBUF + piece * 1024), 16, off, 0, 0, 0);
    }
  };
  auto advance_issue = [&]() {
    if (++i_c == i_nchunk) {
      i_c = 0;
      if (++i_item < ie) load_issue_item(i_item);
    }
  };

  auto compute = [&](const int slot) {
    const int KB = c_K >> 7;
    const int jb = c_c * kNB;
    const uint8_t* xb = lds + slot * XBUF;
    const uint8_t* sp = szl + slot * SZBUF + wave * 1024 + col * 8;
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      if (jb + b >= KB) break;
#pragma unroll
      for (int h = 0; h < 2; ++h) {             // the two groups of the block
        sv_u32x4 a0[MT], a1[MT];
        sv_f32x4 xs[MT];
#pragma unroll
        for (int a = 0; a < MT; ++a) {
          const uint8_t* ap = xb + a * 16 * kRowBytes + b * 256;
          a0[a] = *reinterpret_cast<const sv_u32x4*>(ap + aoff[h][0]);
          a1[a] = *reinterpret_cast<const sv_u32x4*>(ap + aoff[h][1]);
          xs[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sv_as_bf16x8(a0[a]),
                                                          sv_as_bf16x8(ones), fz, 0, 0, 0);
          xs[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sv_as_bf16x8(a1[a]),
                                                          sv_as_bf16x8(ones), xs[a], 0, 0, 0);
        }
#pragma unroll
        for (int tw = 0; tw < kTW; ++tw) {
          const sv_u32x4 w = wb[slot][tw][b];
          const sv_u32x4 b0 = sv_w4_dequant8(h ? w.z : w.x, magic);
          const sv_u32x4 b1 = sv_w4_dequant8(h ? w.w : w.y, magic);
          const sv_u32x2 sbt = *reinterpret_cast<const sv_u32x2*>(sp + (tw * kNB + b) * 128);
          const unsigned int sz = h ? sbt.y : sbt.x;
          const float s = sv_half_lo(sz);
          const float zb = 128.0f + sv_half_hi(sz);
#pragma unroll
          for (int a = 0; a < MT; ++a) {
            sv_f32x4 acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                sv_as_bf16x8(a0[a]), sv_as_bf16x8(b0), fz, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sv_as_bf16x8(a1[a]),
                                                          sv_as_bf16x8(b1), acc, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i)
              yacc[tw][a][i] = fmaf(s, fmaf(-zb, xs[a][i], acc[i]), yacc[tw][a][i]);
          }
        }
      }
    }
  };

  // NS stores every step.  On an item's last chunk: each 16x16 output tile
  // goes through the wave's LDS transpose area (lane (col, q) of an MFMA
  // output holds rows 4q .. 4q+3 of channel col) so that lane l stores
  // channels 4 (l % 4) .. +3 of row l / 4 as one 16-byte write.  Otherwise
  // the same number of stores with out-of-range offsets.
  auto store = [&](const bool at_end) {
    if (at_end) {
#pragma unroll
      for (int tw = 0; tw < kTW; ++tw) {
        const int tile = c_t0 + wave * kTW + tw;
#pragma unroll
        for (int a = 0; a < MT; ++a) {
#pragma unroll
          for (int i = 0; i < 4; ++i) tpose[(4 * q + i) * 16 + col] = yacc[tw][a][i];
          const sv_u32x4 v =
              *reinterpret_cast<const sv_u32x4*>(tpose + (lane >> 2) * 16 + 4 * (lane & 3));
          const int r = 16 * a + (lane >> 2);
          const bool ok = tile < (c_N >> 4) && r < m;
          const unsigned int off =
              ok ? (r * c_N + 16 * tile + 4 * (lane & 3)) * 4 : kSvOutOfRange;
          __builtin_amdgcn_raw_buffer_store_b128(v, yrs, off, 0, 0);
        }
      }
#pragma unroll
      for (int t = 0; t < kTW; ++t)
#pragma unroll
        for (int a = 0; a < MT; ++a) yacc[t][a] = fz;
    } else {
#pragma unroll
      for (int tw = 0; tw < kTW; ++tw)
#pragma unroll
        for (int a = 0; a < MT; ++a)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(sv_u32x4, yacc[tw][a]), yrs,
                                                 kSvOutOfRange, 0, 0);
    }
  };
  auto advance_compute = [&]() {
    if (++c_c == c_nchunk) {
      c_c = 0;
      if (++c_item < ie) load_compute_item(c_item);
    }
  };

  // Prologue: P - 1 chunks in flight, each followed by a step's worth of
  // (out-of-range) stores so every step sees the same operation pattern.
#pragma unroll
  for (int i = 0; i < P - 1; ++i) {
    issue(i);
    advance_issue();
    sv_compiler_fence();
    store(false);
  }
  for (int s0 = 0; s0 < steps; s0 += P) {
#pragma unroll
    for (int s = 0; s < P; ++s) {
      // chunk s0 + s has landed in slot s (registers and LDS) for every wave,
      // and every wave has finished the chunk that last used slot s + P - 1
      sv_wait_vmcnt<WAITN>();
      sv_barrier_no_fence();
      issue((s + P - 1) % P);
      advance_issue();
      sv_compiler_fence();
      const bool run = s0 + s < steps;
      const bool at_end = run && c_c == c_nchunk - 1;
      if (run) compute(s);
      store(at_end);
      if (run) advance_compute();
    }
  }
  // Drain every outstanding load (including buffer -> LDS copies) before the
  // workgroup's LDS can be handed to another workgroup.
  sv_wait_vmcnt<0>();
  sv_barrier_no_fence();
}

template <int MT, int P>
sv_status launch_pass(const void* plan, int m, int grid, hipStream_t st) {
  auto kern = w4_pass_kernel<MT, P>;
  constexpr int kLds = pass_lds_bytes<MT, P>();
  static_assert(kLds <= 160 * 1024, "LDS budget of a gfx950 workgroup");
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kLds) != hipSuccess)
    return SV_ERR_HIP;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), kLds, st,
                     static_cast<const uint8_t*>(plan), m);
  SV_LAUNCH_CHECK();
  return SV_OK;
}

sv_status check_gemms(const sv_w4_gemm* gemms, int count, int m, long long* n_items) {
  if (!gemms) return SV_ERR_NULL;
  if (count < 1 || m < 1 || m > SV_MAX_ROWS) return SV_ERR_INVALID_ARG;
  long long items = 0;
  for (int g = 0; g < count; ++g) {
    const sv_w4_gemm& e = gemms[g];
    if (!e.x || !e.packed_codes || !e.packed_sz || !e.y) return SV_ERR_NULL;
    if (e.N < 16 || e.N % 16 != 0 || e.K < 128 || e.K % 128 != 0) return SV_ERR_INVALID_ARG;
    // buffer ranges are 32-bit: codes, activations and outputs below 2 GiB
    if (static_cast<long long>(e.N) * e.K / 2 >= (1LL << 31) ||
        static_cast<long long>(m) * e.K * 2 >= (1LL << 31) ||
        static_cast<long long>(m) * e.N * 4 >= (1LL << 31))
      return SV_ERR_UNSUPPORTED;
    if (!sv_aligned16(e.x) || !sv_aligned16(e.packed_codes) || !sv_aligned16(e.packed_sz) ||
        !sv_aligned16(e.y))
      return SV_ERR_ALIGN;
    items += ceil_div(e.N / 16, kItemTiles);
  }
  if (items >= (1LL << 30)) return SV_ERR_UNSUPPORTED;
  *n_items = items;
  return SV_OK;
}

}  // namespace

extern "C" size_t sv_w4_pass_plan_bytes(const sv_w4_gemm* gemms, int count, int m) {
  long long items = 0;
  if (check_gemms(gemms, count, m, &items) != SV_OK) return 0;
  return kItemsOff + static_cast<size_t>(items) * sizeof(PlanItem);
}

extern "C" sv_status sv_w4_pass_plan(const sv_w4_gemm* gemms, int count, int m, int group,
                                     void* plan, size_t plan_bytes, sv_w4_pass* pass,
                                     hipStream_t stream) {
  long long n_items = 0;
  const sv_status st = check_gemms(gemms, count, m, &n_items);
  if (st != SV_OK) return st;
  if (!plan || !pass) return SV_ERR_NULL;
  if (group != kGroup) return SV_ERR_UNSUPPORTED;
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

  // Items in pass order.
  std::vector<PlanItem> items;
  items.reserve(static_cast<size_t>(n_items));
  for (int g = 0; g < count; ++g) {
    const sv_w4_gemm& e = gemms[g];
    const int tiles = e.N / 16;
    for (int t0 = 0; t0 < tiles; t0 += kItemTiles)
      items.push_back(PlanItem{static_cast<const uint16_t*>(e.x), e.packed_codes,
                               static_cast<const uint16_t*>(e.packed_sz), e.y, e.K, e.N, t0,
                               ceil_div(e.K, kKC)});
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
  hdr->m = m;
  hdr->count = count;
  hdr->grid = grid;
  hdr->items = static_cast<int32_t>(n_items);
  hdr->max_steps = max_steps;

  // Plan upload: a setup step (like packing the weights), synchronous so the
  // host image can be released.
  if (hipMemcpyAsync(plan, image.data(), need, hipMemcpyHostToDevice, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return SV_ERR_HIP;
  pass->plan = plan;
  pass->m = m;
  pass->count = count;
  pass->grid = grid;
  pass->items = static_cast<int>(n_items);
  pass->max_steps = max_steps;
  pass->reserved = 0;
  return SV_OK;
}

extern "C" sv_status sv_qgemm_w4_pass(const sv_w4_pass* pass, hipStream_t stream) {
  if (!pass || !pass->plan) return SV_ERR_NULL;
  if (!sv_aligned16(pass->plan)) return SV_ERR_ALIGN;
  if (pass->m < 1 || pass->m > SV_MAX_ROWS || pass->grid < 1 || pass->grid > kMaxGrid)
    return SV_ERR_INVALID_ARG;
  // Two activation tiles for m > 16; the ring keeps two chunks in flight.
  if (pass->m <= 16) return launch_pass<1, 4>(pass->plan, pass->m, pass->grid, stream);
  return launch_pass<2, 4>(pass->plan, pass->m, pass->grid, stream);
}
