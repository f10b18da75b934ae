// sv_verify_accept: fused vocabulary softmax for target and draft rows, the
// left-to-right accept scan, and the residual / bonus resample.
//
// Source: Speculative Decoding Clearly Explained, "Accept from left to right"
// (accept with probability min(1, p/q), stop at the first rejection) and
// "Correct and continue" (resample from max(0, p - q) normalized; if every
// draft is accepted the target supplies one more token); Karpathy's Trick for
// Faster Local LLMs, "Producing several tokens from one model pass".
//
// Two launches on the caller's stream:
//  1. stats   one wave per (trial, row, vocabulary span): max and sum of exp
//             over a span, with all loads of a 2048-float batch in flight
//             before any is used; the workgroup's 4 spans are merged into one
//             partial (max, sum, invalid flag, and the row's logit at its
//             draft token when the token lies in those spans).  It also
//             zeroes the per-trial completion counters of launch 2.
//             sv_verify_accept_stats: for the target rows the wave merges the
//             (max, sum) pairs of 64 logits that the vocabulary projection's
//             epilogue wrote, instead of reading the logits.
//  2. decide  one workgroup per (trial, residual share): merges the trial's
//             partials into log-sum-exp values (all loads in flight at once,
//             staged in LDS, 4 lanes per row -- 2 past 64 rows -- in a fixed
//             order), evaluates p_i(d_i), q_i(d_i) from the recorded token
//             logits, draws the Philox uniforms and takes the accept
//             decisions with one wave ballot (first rejection = first zero
//             bit), then sums the residual weights max(0, p_r - q_r) (or p_k
//             for the bonus) of its 2048-float blocks in binary64: 16 groups
//             of 16 threads of 8 consecutive entries each (loaded straight
//             from memory), always in the same order.  Every workgroup of a
//             trial reaches the same decision; workgroup 0 writes the
//             per-trial outputs but the drawn token.  The last workgroup of
//             the trial to finish (a device-scope counter) runs the
//             inverse-CDF selection over the running sums of the block
//             totals (formed by a wave in one fixed association, searched by
//             a wave ballot) and replays the same sums inside the chosen
//             block, so the chosen bin always exists.
#include "sv_common.h"
#include "sv_philox.h"

#include <math.h>

#include <mutex>
#include <type_traits>

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kStatsWaves = 4;
constexpr int kThreads = 256;

struct StatPartial {
  float m;
  float s;
  int bad;
  float tok_logit;   // the row's logit at its draft token if the token lies in
                     // this span, else 0 (no draft token: the bonus row)
};

struct Decision {
  int status;
  int n_acc;
  float lse_t;
  float lse_d;
  double u2;
  double pad;
};

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions over the 4 lanes of a quad, in VALU latency (a lane shuffle
// goes through the LDS pipe): the DPP quad permutes [1,0,3,2] and [2,3,0,1].
// Every lane of the quad ends with the same bits (binary32 max and add are
// commutative, and each step pairs the same two values).
template <int CTRL>
__device__ __forceinline__ int dpp_quad(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E;
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, __int_as_float(dpp_quad<kDppXor1>(__float_as_int(v))));
  return fmaxf(v, __int_as_float(dpp_quad<kDppXor2>(__float_as_int(v))));
}
__device__ __forceinline__ float quad_sum(float v) {
  v += __int_as_float(dpp_quad<kDppXor1>(__float_as_int(v)));
  return v + __int_as_float(dpp_quad<kDppXor2>(__float_as_int(v)));
}
__device__ __forceinline__ int quad_or(int v) {
  v |= dpp_quad<kDppXor1>(v);
  return v | dpp_quad<kDppXor2>(v);
}
// The same over the 2 lanes of a pair (the permute [1,0,3,2] alone).
__device__ __forceinline__ float pair_max(float v) {
  return fmaxf(v, __int_as_float(dpp_quad<kDppXor1>(__float_as_int(v))));
}
__device__ __forceinline__ float pair_sum(float v) {
  return v + __int_as_float(dpp_quad<kDppXor1>(__float_as_int(v)));
}
__device__ __forceinline__ int pair_or(int v) { return v | dpp_quad<kDppXor1>(v); }

// Online softmax statistics: running max m and sum s of exp(v - m).
__device__ __forceinline__ void stat_add4(float& m, float& s, int& bad, float4 v) {
  bad |= (v.x != v.x) | (v.y != v.y) | (v.z != v.z) | (v.w != v.w);
  bad |= (v.x == INFINITY) | (v.y == INFINITY) | (v.z == INFINITY) | (v.w == INFINITY);
  const float vm = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
  if (vm > m) {
    s *= exp2_fast((m - vm) * kLog2e);
    m = vm;
  }
  if (m != -INFINITY) {
    s += exp2_fast((v.x - m) * kLog2e) + exp2_fast((v.y - m) * kLog2e) +
         exp2_fast((v.z - m) * kLog2e) + exp2_fast((v.w - m) * kLog2e);
  }
}

__device__ __forceinline__ void stat_add1(float& m, float& s, int& bad, float v) {
  bad |= (v != v) | (v == INFINITY);
  if (v > m) {
    s *= exp2_fast((m - v) * kLog2e);
    m = v;
  }
  if (m != -INFINITY) s += exp2_fast((v - m) * kLog2e);
}

__device__ __forceinline__ void stat_merge(float& m, float& s, float m2, float s2) {
  const float mm = fmaxf(m, m2);
  if (mm == -INFINITY) {
    m = -INFINITY;
    s = 0.f;
    return;
  }
  s = s * exp2_fast((m - mm) * kLog2e) + s2 * exp2_fast((m2 - mm) * kLog2e);
  m = mm;
}

// Vocabulary tiling shared by the kernels.
//  * Statistics: each row is cut into C1 <= kMaxC1 spans of whole 2048-float
//    batches; one wave reduces one (trial, row, span), and a workgroup of
//    kStatsWaves waves merges its spans into one partial (CG per row).
//  * Residual: the vocabulary is cut into blocks of kBlk floats; block
//    totals, and inside a block 16 groups of 16 thread ranges of 8 floats,
//    are summed in one fixed order everywhere, so the inverse-CDF search of
//    the selection walks exactly the sums that kernel 2 produced.
constexpr int kBatch = 2048;                    // floats per wave per statistics batch
constexpr int kMaxC1 = 80;                      // statistics spans per row
// partials per row: one per statistics workgroup of kStatsWaves spans
constexpr int kMaxCG = (kMaxC1 + kStatsWaves - 1) / kStatsWaves;
__host__ __device__ inline int stat_groups(int C1) { return (C1 + kStatsWaves - 1) / kStatsWaves; }
constexpr int kBlk = 2048;                      // floats per residual block
constexpr int kPerThread = kBlk / kThreads;     // 8
constexpr int kGroups = 16;                     // thread groups per block
constexpr int kGroupThreads = kThreads / kGroups;

__host__ __device__ inline int stat_spans(int V) {
  const int batches = (V + kBatch - 1) / kBatch;
  return batches < kMaxC1 ? batches : kMaxC1;
}
__host__ __device__ inline int stat_span_len(int V, int C1) {
  const int batches = (V + kBatch - 1) / kBatch;
  return ((batches + C1 - 1) / C1) * kBatch;
}
__host__ __device__ inline int resid_blocks(int V) { return (V + kBlk - 1) / kBlk; }
// Workgroups of kernel 2 per trial: enough for about 256 in total, 1024 from
// 32 trials on (measured: B = 64 466 -> 451 us; at B = 8 more cost 2 us).
__host__ __device__ inline int resid_wgs(int B, int V) {
  const long long target = B >= 32 ? 1024 : 256;
  long long c = (target + static_cast<long long>(B) - 1) / B;
  const long long nb = resid_blocks(V);
  if (c > nb) c = nb;
  return static_cast<int>(c < 1 ? 1 : c);
}

struct WsLayout {
  size_t partial_off, decision_off, total_off, done_off, bytes;
};

__host__ inline WsLayout ws_layout(int B, int k, int V) {
  auto up = [](size_t v) { return (v + 255) & ~static_cast<size_t>(255); };
  WsLayout L;
  const size_t R = 2 * static_cast<size_t>(k) + 1;
  L.partial_off = 0;
  L.decision_off =
      up(static_cast<size_t>(B) * R * stat_groups(stat_spans(V)) * sizeof(StatPartial));
  L.total_off = L.decision_off + up(static_cast<size_t>(B) * sizeof(Decision));
  L.done_off = L.total_off + up(static_cast<size_t>(B) * resid_blocks(V) * sizeof(double));
  L.bytes = L.done_off + up(static_cast<size_t>(B) * sizeof(int));
  return L;
}

__device__ __forceinline__ const float* row_ptr(const float* tgt, const float* dft, int b, int j,
                                                int k, int V) {
  if (j <= k) return tgt + (static_cast<size_t>(b) * (k + 1) + j) * V;
  return dft + (static_cast<size_t>(b) * k + (j - k - 1)) * V;
}

// ---- kernel 1: per-span softmax statistics ---------------------------------
// All loads of a 2048-float batch are issued before any is used (8 float4 or
// 32 floats per lane), so a wave pays one memory latency per batch.
template <bool VEC, bool PRE>
__global__ __launch_bounds__(64 * kStatsWaves) void stats_kernel(
    const float* __restrict__ tgt, const float* __restrict__ dft,
    const float2* __restrict__ tstats, const int32_t* __restrict__ toks, int B, int k, int V,
    int CG, int span, StatPartial* __restrict__ part, int* __restrict__ done) {
  // the per-trial completion counters of kernel 2 start at zero every call
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < B; i += blockDim.x) done[i] = 0;
  __shared__ StatPartial wp[kStatsWaves];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  // workgroup = (trial, row, group of kStatsWaves spans); the grid is exact,
  // and a span past the row's last (c >= C1) is empty
  const int R = 2 * k + 1;
  const int g = static_cast<int>(blockIdx.x % CG);
  const long long br = blockIdx.x / CG;
  const int j = static_cast<int>(br % R);
  const int b = static_cast<int>(br / R);
  const int c = g * kStatsWaves + w;
  const float* row = row_ptr(tgt, dft, b, j, k, V);
  const int lo = min(V, c * span);
  const int hi = min(V, lo + span);
  // the draft token of this row (target row i < k and draft row i share d_i;
  // the bonus row k has none); its logit is recorded by the wave whose span
  // holds it, so the decide launch reads it with the statistics
  const int ti = j < k ? j : j - k - 1;
  const int tok = j == k ? -1 : toks[static_cast<size_t>(b) * k + ti];
  const bool tok_here = tok >= lo && tok < hi;
  float tok_logit = 0.f;
  float m = -INFINITY, s = 0.f;
  int bad = 0;
  if (PRE && j <= k) {
    if (tok_here) tok_logit = row[tok];
    // the span's pairs of 64 logits (span and lo are multiples of 64; an
    // empty span past the row's end has lo = hi = V and reads none)
    const int G = (V + 63) / 64;
    const float2* st = tstats + (static_cast<size_t>(b) * (k + 1) + j) * G;
    const int g_end = lo < hi ? (hi + 63) / 64 : 0;
    for (int g = lo / 64 + lane; g < g_end; g += 64) {
      const float2 pr = st[g];
      bad |= pr.y != pr.y;
      if (pr.y == pr.y) stat_merge(m, s, pr.x, pr.y);
    }
  } else
  for (int base = lo; base < hi; base += kBatch) {
    constexpr int NV = VEC ? kBatch / 256 : kBatch / 64;
    float v[VEC ? 4 * NV : NV];
    if (VEC) {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int e = base + 256 * i + 4 * lane;
        float4 t = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        if (e < hi) t = *reinterpret_cast<const float4*>(row + e);
        v[4 * i] = t.x;
        v[4 * i + 1] = t.y;
        v[4 * i + 2] = t.z;
        v[4 * i + 3] = t.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int e = base + 64 * i + lane;
        v[i] = e < hi ? row[e] : -INFINITY;
      }
    }
    if (tok_here && tok >= base && tok < base + kBatch) {
      // lane and register holding the token's logit (wave-uniform branch)
      const int off = tok - base;
      const int want = VEC ? 4 * (off >> 8) + (off & 3) : off >> 6;
      const int src = VEC ? (off >> 2) & 63 : off & 63;
      float val = v[0];
#pragma unroll
      for (int i = 1; i < (VEC ? 4 * NV : NV); ++i) val = i == want ? v[i] : val;
      tok_logit = __shfl(val, src);
    }
    float vm = -INFINITY;
#pragma unroll
    for (int i = 0; i < (VEC ? 4 * NV : NV); ++i) {
      bad |= (v[i] != v[i]) | (v[i] == INFINITY);
      vm = fmaxf(vm, v[i]);
    }
    if (vm > m) {
      s *= exp2_fast((m - vm) * kLog2e);
      m = vm;
    }
    if (m != -INFINITY) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < (VEC ? 4 * NV : NV); ++i) acc += exp2_fast((v[i] - m) * kLog2e);
      s += acc;
    }
  }
  for (int off = 32; off > 0; off >>= 1) {
    const float m2 = __shfl_xor(m, off);
    const float s2 = __shfl_xor(s, off);
    bad |= __shfl_xor(bad, off);
    stat_merge(m, s, m2, s2);
  }
  // the workgroup's kStatsWaves partials merged in wave order; the token
  // logit is the one of the wave whose span holds the token
  if (lane == 0) wp[w] = StatPartial{m, s, bad, tok_logit};
  __syncthreads();
  if (threadIdx.x == 0) {
    float M = wp[0].m, S = wp[0].s;
    int bd = wp[0].bad;
#pragma unroll
    for (int u = 1; u < kStatsWaves; ++u) {
      stat_merge(M, S, wp[u].m, wp[u].s);
      bd |= wp[u].bad;
    }
    const int ut = tok >= 0 ? tok / span - g * kStatsWaves : -1;
    const float tl = ut >= 0 && ut < kStatsWaves ? wp[ut].tok_logit : 0.f;
    part[static_cast<size_t>(blockIdx.x)] = StatPartial{M, S, bd, tl};
  }
}

// Residual / bonus weight of one vocabulary entry from its two logits
// (binary32).  The residual sums and the selection's replay evaluate it with
// the same IEEE operations in the same order, so both see bit-identical
// weights; inlined, a thread's 8 evaluations overlap.
__device__ __forceinline__ float resid_weight(float tl, float lt, float dl, float ld, bool bonus) {
  const float p = expf(tl - lt);
  if (bonus) return p;
  const float q = expf(dl - ld);
  return fmaxf(0.f, p - q);
}

// One thread's kPerThread consecutive entries a .. a+7 of the residual rows
// (target row pt, draft row pd): two 16-byte loads per row when the entries
// are whole and aligned, else one guarded load each; entries past V read as
// -inf (weight 0) and are never counted.
__device__ __forceinline__ void load_entries(const float* pt, const float* pd, int V, int a,
                                             float* t, float* d) {
  if ((V & 3) == 0 && a + kPerThread <= V) {
    const float4* t4 = reinterpret_cast<const float4*>(pt + a);
    const float4 t0 = t4[0], t1 = t4[1];
    t[0] = t0.x; t[1] = t0.y; t[2] = t0.z; t[3] = t0.w;
    t[4] = t1.x; t[5] = t1.y; t[6] = t1.z; t[7] = t1.w;
    if (pd != nullptr) {
      const float4* d4 = reinterpret_cast<const float4*>(pd + a);
      const float4 d0 = d4[0], d1 = d4[1];
      d[0] = d0.x; d[1] = d0.y; d[2] = d0.z; d[3] = d0.w;
      d[4] = d1.x; d[5] = d1.y; d[6] = d1.z; d[7] = d1.w;
    } else {
#pragma unroll
      for (int i = 0; i < kPerThread; ++i) d[i] = -INFINITY;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int e = a + i;
      t[i] = e < V ? pt[e] : -INFINITY;
      d[i] = (pd != nullptr && e < V) ? pd[e] : -INFINITY;
    }
  }
}

// Sum of this thread's 8 consecutive weights w of block blk, in order
// (entries past V not counted).
__device__ __forceinline__ double thread_sum(const float* pt, const float* pd, int V, int blk,
                                             float lt, float ld, bool bonus, float* w) {
  const int a = blk * kBlk + threadIdx.x * kPerThread;
  float t[kPerThread], d[kPerThread];
  load_entries(pt, pd, V, a, t, d);
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) w[i] = resid_weight(t[i], lt, d[i], ld, bonus);
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i)
    if (a + i < V) acc += static_cast<double>(w[i]);
  return acc;
}
__device__ __forceinline__ double thread_sum(const float* pt, const float* pd, int V, int blk,
                                             float lt, float ld, bool bonus) {
  float w[kPerThread];
  return thread_sum(pt, pd, V, blk, lt, ld, bonus, w);
}

// Group sums (16 consecutive threads, in order) and the block total (groups
// in order) from the per-thread sums in tsum; gsum receives the group sums.
__device__ __forceinline__ void block_sums(const double* tsum, double* gsum, double* total) {
  if (threadIdx.x < kGroups) {
    double g = 0.0;
    for (int t = 0; t < kGroupThreads; ++t) g += tsum[threadIdx.x * kGroupThreads + t];
    gsum[threadIdx.x] = g;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double T = 0.0;
    for (int g = 0; g < kGroups; ++g) T += gsum[g];
    *total = T;
  }
  __syncthreads();
}

__device__ void select_trial(const float* __restrict__ tgt, const float* __restrict__ dft, int k,
                             int V, int b, const Decision dec,
                             const double* __restrict__ totals,
                             int32_t* __restrict__ out_tokens, double* tsum, double* gsum,
                             double* btot_p, double* dyn_tot);

// ---- kernel 2: decide + residual block totals + select-----------------------------
// Every workgroup of a trial merges the trial's statistics and takes the same
// decisions (identical inputs and order); workgroup 0 writes the per-trial
// outputs.  Then each workgroup sums its share of the residual blocks.
__global__ __launch_bounds__(kThreads) void decide_kernel(
    const float* __restrict__ tgt, const float* __restrict__ dft, const int32_t* __restrict__ toks,
    int B, int k, int V, int CG, int span, int C2, unsigned int key0, unsigned int key1,
    unsigned int offset,
    const StatPartial* __restrict__ part, Decision* __restrict__ decs, double* __restrict__ totals,
    int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_n_acc,
    int32_t* __restrict__ out_status, float* __restrict__ p_at, float* __restrict__ q_at,
    float* __restrict__ lse_out, int* __restrict__ done) {
  __shared__ float pm[(2 * SV_MAX_ROWS + 1) * kMaxCG];
  __shared__ float ps[(2 * SV_MAX_ROWS + 1) * kMaxCG];
  __shared__ int pb[(2 * SV_MAX_ROWS + 1) * kMaxCG];
  __shared__ float pl[(2 * SV_MAX_ROWS + 1) * kMaxCG];
  __shared__ float lse_sh[2 * SV_MAX_ROWS + 1];
  __shared__ int bad_sh[2 * SV_MAX_ROWS + 1];
  __shared__ Decision dec;
  __shared__ double tsum[kThreads];
  __shared__ double gsum[kGroups];
  __shared__ double btot;
  const int b = blockIdx.x / C2;
  const int c = blockIdx.x % C2;
  const int R = 2 * k + 1;
  const int tid = threadIdx.x;

  // 1. The trial's R x CG statistics partials -> LDS (coalesced), each
  //    thread's loads all issued before its first store (one memory
  //    latency); wave 0 also loads the draft tokens.  The tokens' logits come
  //    with the partials (the statistics launch recorded them).
  const bool has_draft = tid < k;
  int tok = 0;
  if (has_draft) tok = toks[static_cast<size_t>(b) * k + tid];
  {
    constexpr int kPer = ((2 * SV_MAX_ROWS + 1) * kMaxCG + kThreads - 1) / kThreads;
    const int4* pp = reinterpret_cast<const int4*>(part + static_cast<size_t>(b) * R * CG);
    const int n = R * CG;
    int4 q[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = tid + u * kThreads;
      if (e < n) q[u] = pp[e];
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = tid + u * kThreads;
      if (e < n) {
        pm[e] = __int_as_float(q[u].x);
        ps[e] = __int_as_float(q[u].y);
        pb[e] = q[u].z;
        pl[e] = __int_as_float(q[u].w);
      }
    }
  }
  const bool tok_bad = has_draft && (tok < 0 || tok >= V);
  __syncthreads();
  // 2. merge each row's partials: 4 lanes (one quad) per row, 64 rows per
  //    round of the workgroup, lane sub taking partials sub, sub + 4, ..; the
  //    row maximum first, then the sum rescaled to it, each combined over the
  //    quad in a fixed order
  // (2 lanes per row when there are more rows than quads, so that every row
  // is merged in one round)
  auto merge_rows = [&](auto lanes_c) {
    constexpr int kL = decltype(lanes_c)::value;
    const int sub = tid & (kL - 1);
    for (int j0 = 0; j0 < R; j0 += kThreads / kL) {
      const int j = j0 + tid / kL;
      const bool own = j < R;
      float m = -INFINITY;
      int bad = 0;
      if (own) {
#pragma unroll 5
        for (int i = sub; i < CG; i += kL) {
          m = fmaxf(m, pm[j * CG + i]);
          bad |= pb[j * CG + i];
        }
      }
      m = kL == 4 ? quad_max(m) : pair_max(m);
      bad = kL == 4 ? quad_or(bad) : pair_or(bad);
      float sum = 0.f;
      if (own && m != -INFINITY) {
#pragma unroll 5
        for (int i = sub; i < CG; i += kL)
          sum += ps[j * CG + i] * exp2_fast((pm[j * CG + i] - m) * kLog2e);
      }
      sum = kL == 4 ? quad_sum(sum) : pair_sum(sum);
      if (own && sub == 0) {
        const int bd = bad | (m == -INFINITY) | !(sum > 0.f);
        lse_sh[j] = bd ? NAN : m + logf(sum);
        bad_sh[j] = bd;
      }
    }
  };
  if (R <= kThreads / 4)
    merge_rows(std::integral_constant<int, 4>{});
  else
    merge_rows(std::integral_constant<int, 2>{});
  __syncthreads();

  // 3. decisions (wave 0): accept iff u_i q_i(d_i) < p_i(d_i), first rejection
  if (tid < 64) {
    const int i = tid;
    const bool row_bad = (i < R && bad_sh[i]) || (i + 64 < R && bad_sh[i + 64]);
    const bool any_tok_bad = __any(tok_bad);
    const bool any_row_bad = __any(row_bad);
    const int status = any_tok_bad ? 1 : (any_row_bad ? 2 : 0);

    float p = NAN, q = NAN, u2 = 0.f;
    bool accepted = true;
    if (i <= k) {
      unsigned int ctr[4] = {static_cast<unsigned int>(i), static_cast<unsigned int>(b), offset, 0u};
      sv_philox_rounds(ctr, key0, key1);
      const float u = sv_u24(ctr[0]);
      u2 = sv_u24(ctr[1]);
      if (has_draft && status == 0) {
        const int ct = tok / span / kStatsWaves;   // the partial whose spans hold the token
        const float tl = pl[i * CG + ct];
        const float dl = pl[(k + 1 + i) * CG + ct];
        p = expf(tl - lse_sh[i]);
        q = expf(dl - lse_sh[k + 1 + i]);
        accepted = u * q < p;
      }
    }
    const unsigned long long rej = __ballot(has_draft && !accepted);
    const int n_acc = rej ? (__ffsll(static_cast<long long>(rej)) - 1) : k;
    const float u2r = __shfl(u2, n_acc);
    if (i == 0) {
      dec.status = status;
      dec.n_acc = status == 0 ? n_acc : -1;
      dec.lse_t = lse_sh[n_acc];
      dec.lse_d = n_acc < k ? lse_sh[k + 1 + n_acc] : 0.f;
      dec.u2 = static_cast<double>(u2r);
      dec.pad = 0.0;
    }
    if (c == 0) {
      if (has_draft) {
        if (p_at) p_at[static_cast<size_t>(b) * k + i] = status == 0 ? p : NAN;
        if (q_at) q_at[static_cast<size_t>(b) * k + i] = status == 0 ? q : NAN;
      }
      if (i <= k && !(status == 0 && i == n_acc)) {
        // accepted drafts, -1 after them; position n_acc is left to the
        // selection (two workgroups writing one word would race: their
        // caches are written back in either order)
        const bool keep = status == 0 && i < n_acc;
        out_tokens[static_cast<size_t>(b) * (k + 1) + i] = keep ? tok : -1;
      }
      if (lse_out) {
        for (int j = i; j < R; j += 64) lse_out[static_cast<size_t>(b) * R + j] = lse_sh[j];
      }
      if (i == 0) {
        out_status[b] = status;
        out_n_acc[b] = status == 0 ? n_acc : -1;
      }
    }
  }
  __syncthreads();
  if (c == 0 && tid == 0) decs[b] = dec;

  // 4. residual block totals of this workgroup's blocks
  const int nb = resid_blocks(V);
  const int b0 = static_cast<int>(static_cast<long long>(nb) * c / C2);
  const int b1 = static_cast<int>(static_cast<long long>(nb) * (c + 1) / C2);
  double* tot = totals + static_cast<size_t>(b) * nb;
  if (dec.status != 0) return;
  const int r = dec.n_acc;
  const bool bonus = r == k;
  const float* pt = tgt + (static_cast<size_t>(b) * (k + 1) + r) * V;
  const float* pd = bonus ? nullptr : dft + (static_cast<size_t>(b) * k + r) * V;
  for (int blk = b0; blk < b1; ++blk) {
    tsum[tid] = thread_sum(pt, pd, V, blk, dec.lse_t, dec.lse_d, bonus);
    __syncthreads();
    block_sums(tsum, gsum, &btot);
    if (tid == 0)
      __hip_atomic_store(reinterpret_cast<unsigned long long*>(tot + blk),
                         static_cast<unsigned long long>(__double_as_longlong(btot)),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // The last workgroup of the trial to finish (device-scope counter, zeroed
  // by kernel 1 of this call) selects the token.  The block totals go
  // through device-scope stores and loads, which bypass the compute units'
  // non-coherent caches: each wave waits for its own to complete, then the
  // barrier, then the count.
  __shared__ int is_last;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) is_last = atomicAdd(&done[b], 1) == C2 - 1;
  __syncthreads();
  if (!is_last) return;
  extern __shared__ double dyn_tot[];   // resid_blocks(V) doubles
  select_trial(tgt, dft, k, V, b, dec, totals, out_tokens, tsum, gsum, &btot, dyn_tot);
}

// ---- select the replacement / bonus token ------------------------------------
// Run by the last workgroup of kernel 2 to finish a trial, on the LDS arrays
// of that workgroup: inverse CDF over the block totals, then inside the
// chosen block over groups, threads and a thread's 8 entries, replaying the
// exact sums kernel 2 formed.
__device__ void select_trial(const float* __restrict__ tgt, const float* __restrict__ dft, int k,
                             int V, int b, const Decision dec,
                             const double* __restrict__ totals,
                             int32_t* __restrict__ out_tokens, double* tsum, double* gsum,
                             double* btot_p, double* dyn_tot) {
  __shared__ double sh_S, sh_pc, sh_thr, sh_q[2];
  __shared__ int sh_blk, sh_ts;
  double& btot = *btot_p;
  const int tid = threadIdx.x;
  const int r = dec.n_acc;
  const float* pt = tgt + (static_cast<size_t>(b) * (k + 1) + r) * V;
  const float* pd = r < k ? dft + (static_cast<size_t>(b) * k + r) * V : nullptr;
  bool bonus = r == k;
  const int nb = resid_blocks(V);
  const unsigned long long* T =
      reinterpret_cast<const unsigned long long*>(totals + static_cast<size_t>(b) * nb);

  // Block totals -> LDS (dyn_tot), then replaced in place by their running
  // sums in vocabulary order: wave 0, lane l adding a contiguous range of
  // blocks after the exclusive running sum of the ranges before it (one
  // fixed association).
  auto running_sums = [&]() {
    if (tid < 64) {
      const int per = (nb + 63) / 64;
      const int i0 = min(nb, tid * per), i1 = min(nb, i0 + per);
      double c = 0.0;
      for (int i = i0; i < i1; ++i) c += dyn_tot[i];
      double incl = c;
      for (int o = 1; o < 64; o <<= 1) {
        const double y = __shfl_up(incl, o, 64);
        if (tid >= o) incl += y;
      }
      double run = __shfl_up(incl, 1, 64);
      if (tid == 0) run = 0.0;
      for (int i = i0; i < i1; ++i) {
        run += dyn_tot[i];
        dyn_tot[i] = run;
      }
      const double S = __shfl(incl, 63, 64);
      if (tid == 0) sh_S = S;
    }
    __syncthreads();
  };
  for (int i = tid; i < nb; i += kThreads)
    dyn_tot[i] = __longlong_as_double(static_cast<long long>(
        __hip_atomic_load(T + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)));
  __syncthreads();
  running_sums();
  // Rounding left no residual mass: sample from p_r instead, with block
  // totals recomputed here (a rare path, so one block at a time).
  const bool usep = !(sh_S > 0.0);
  if (usep) {
    bonus = true;
    pd = nullptr;
    for (int blk = 0; blk < nb; ++blk) {
      tsum[tid] = thread_sum(pt, pd, V, blk, dec.lse_t, dec.lse_d, true);
      __syncthreads();
      block_sums(tsum, gsum, &btot);
      if (tid == 0) dyn_tot[blk] = btot;
      __syncthreads();
    }
    running_sums();
  }
  // The first block whose running sum exceeds thr = u' S (wave 0 ballots over
  // 64 blocks at a time); pc = the running sum before it.  None: the last
  // block, with pc = S.
  if (tid < 64) {
    const double S = sh_S;
    const double thr_w = dec.u2 * S;
    int bs = -1;
    for (int c0 = 0; c0 < nb; c0 += 64) {
      const int i = c0 + tid;
      const unsigned long long hit = __ballot(i < nb && dyn_tot[i] > thr_w);
      if (hit) {
        bs = c0 + __ffsll(static_cast<long long>(hit)) - 1;
        break;
      }
    }
    if (tid == 0) {
      sh_thr = thr_w;
      sh_blk = bs < 0 ? nb - 1 : bs;
      sh_pc = bs < 0 ? S : (bs > 0 ? dyn_tot[bs - 1] : 0.0);
    }
  }
  __syncthreads();
  const double thr = sh_thr, pc = sh_pc;
  const int blk = sh_blk;
  float w[kPerThread];                          // kept for the replay below
  tsum[tid] = thread_sum(pt, pd, V, blk, dec.lse_t, dec.lse_d, bonus, w);
  __syncthreads();
  block_sums(tsum, gsum, &btot);
  // groups, then threads inside the group (thread 0, on sums held in
  // registers); every comparison is pc + (group prefix + (thread prefix +
  // run)), the association under which the block total was formed
  double qg = 0.0, qt = 0.0;
  if (tid == 0) {
    int gs = kGroups - 1;
    {
      double gv[kGroups];
#pragma unroll
      for (int g = 0; g < kGroups; ++g) gv[g] = gsum[g];
      double Q = 0.0;
      bool found = false;
#pragma unroll
      for (int g = 0; g < kGroups; ++g) {
        const double nxt = Q + gv[g];
        if (!found && pc + nxt > thr) {
          gs = g;
          qg = Q;
          found = true;
        }
        if (!found) {
          Q = nxt;
          qg = Q;
        }
      }
    }
    int ts = gs * kGroupThreads + kGroupThreads - 1;
    {
      double tv[kGroupThreads];
#pragma unroll
      for (int t = 0; t < kGroupThreads; ++t) tv[t] = tsum[gs * kGroupThreads + t];
      double Q = 0.0;
      bool found = false;
#pragma unroll
      for (int t = 0; t < kGroupThreads; ++t) {
        const double nxt = Q + tv[t];
        if (!found && pc + (qg + nxt) > thr) {
          ts = gs * kGroupThreads + t;
          qt = Q;
          found = true;
        }
        if (!found) {
          Q = nxt;
          qt = Q;
        }
      }
    }
    sh_ts = ts;
    sh_q[0] = qg;
    sh_q[1] = qt;
  }
  __syncthreads();
  // the chosen thread runs through its own 8 weights in order (the values
  // its sum was formed from)
  if (tid == sh_ts) {
    const int a = blk * kBlk + tid * kPerThread;
    const double qg2 = sh_q[0], qt2 = sh_q[1];
    int tok = -1, last_pos = -1;
    double run = 0.0;
    for (int i = 0; i < kPerThread && a + i < V; ++i) {
      const double wi = static_cast<double>(w[i]);
      run += wi;
      if (wi > 0.0) last_pos = a + i;
      if (pc + (qg2 + (qt2 + run)) > thr) {
        tok = a + i;
        break;
      }
    }
    if (tok < 0) tok = last_pos >= 0 ? last_pos : min(a, V - 1);
    out_tokens[static_cast<size_t>(b) * (k + 1) + r] = tok;
  }
}

// ---- Philox known-answer hook ------------------------------------------------
__global__ void philox_kernel(const unsigned int* __restrict__ ctr,
                              const unsigned int* __restrict__ key, unsigned int* __restrict__ out,
                              int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  unsigned int c[4] = {ctr[4 * i], ctr[4 * i + 1], ctr[4 * i + 2], ctr[4 * i + 3]};
  sv_philox_rounds(c, key[2 * i], key[2 * i + 1]);
  for (int j = 0; j < 4; ++j) out[4 * i + j] = c[j];
}

}  // namespace

extern "C" size_t sv_verify_accept_workspace_bytes(int B, int k, int V) {
  if (B < 1 || k < 1 || k > SV_MAX_ROWS || V < 1) return 0;
  return ws_layout(B, k, V).bytes;
}

namespace {
sv_status verify_accept(const float* target_logits, const float* target_stats,
                        const float* draft_logits, const int32_t* draft_tokens, int B, int k,
                        int V, uint64_t seed, uint32_t offset, int32_t* out_tokens,
                        int32_t* out_n_acc, int32_t* out_status, float* p_at, float* q_at,
                        float* lse, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  if (!target_logits || !draft_logits || !draft_tokens || !out_tokens || !out_n_acc ||
      !out_status)
    return SV_ERR_NULL;
  if (target_stats && !sv_aligned16(target_stats)) return SV_ERR_ALIGN;
  if (B < 1 || k < 1 || k > SV_MAX_ROWS || V < 1) return SV_ERR_INVALID_ARG;
  if (static_cast<long long>(k + 1) * V >= (1LL << 31)) return SV_ERR_INVALID_ARG;
  if (!sv_aligned16(target_logits) || !sv_aligned16(draft_logits) ||
      !sv_aligned16(draft_tokens) || !sv_aligned16(out_tokens) || !sv_aligned16(out_n_acc) ||
      !sv_aligned16(out_status) || (p_at && !sv_aligned16(p_at)) ||
      (q_at && !sv_aligned16(q_at)) || (lse && !sv_aligned16(lse)))
    return SV_ERR_ALIGN;
  const WsLayout L = ws_layout(B, k, V);
  if (!workspace || workspace_bytes < L.bytes) return SV_ERR_WORKSPACE;
  if (!sv_aligned16(workspace)) return SV_ERR_ALIGN;

  char* ws = static_cast<char*>(workspace);
  StatPartial* part = reinterpret_cast<StatPartial*>(ws + L.partial_off);
  Decision* decs = reinterpret_cast<Decision*>(ws + L.decision_off);
  double* totals = reinterpret_cast<double*>(ws + L.total_off);
  int* done = reinterpret_cast<int*>(ws + L.done_off);
  const int C1 = stat_spans(V);
  const int span = stat_span_len(V, C1);
  const int CG = stat_groups(C1);
  const int C2 = resid_wgs(B, V);
  const long long blocks1 = static_cast<long long>(B) * (2 * k + 1) * CG;
  if (blocks1 >= (1LL << 31) || static_cast<long long>(B) * C2 >= (1LL << 31))
    return SV_ERR_INVALID_ARG;
  // dynamic LDS of kernel 2: block totals of the selecting workgroup
  const size_t dyn = static_cast<size_t>(resid_blocks(V)) * sizeof(double);
  if (dyn > 32 * 1024) return SV_ERR_UNSUPPORTED;

  const float2* tst = reinterpret_cast<const float2*>(target_stats);
  if (tst && V % 4 == 0)
    hipLaunchKernelGGL((stats_kernel<true, true>), dim3(static_cast<unsigned>(blocks1)),
                       dim3(64 * kStatsWaves), 0, stream, target_logits, draft_logits, tst,
                       draft_tokens, B, k, V, CG, span, part, done);
  else if (tst)
    hipLaunchKernelGGL((stats_kernel<false, true>), dim3(static_cast<unsigned>(blocks1)),
                       dim3(64 * kStatsWaves), 0, stream, target_logits, draft_logits, tst,
                       draft_tokens, B, k, V, CG, span, part, done);
  else if (V % 4 == 0)
    hipLaunchKernelGGL((stats_kernel<true, false>), dim3(static_cast<unsigned>(blocks1)),
                       dim3(64 * kStatsWaves), 0, stream, target_logits, draft_logits, tst,
                       draft_tokens, B, k, V, CG, span, part, done);
  else
    hipLaunchKernelGGL((stats_kernel<false, false>), dim3(static_cast<unsigned>(blocks1)),
                       dim3(64 * kStatsWaves), 0, stream, target_logits, draft_logits, tst,
                       draft_tokens, B, k, V, CG, span, part, done);
  SV_LAUNCH_CHECK();
  hipLaunchKernelGGL(decide_kernel, dim3(static_cast<unsigned>(B) * C2), dim3(kThreads), dyn,
                     stream, target_logits, draft_logits, draft_tokens, B, k, V, CG, span, C2,
                     static_cast<unsigned int>(seed & 0xFFFFFFFFu),
                     static_cast<unsigned int>(seed >> 32), offset, part, decs, totals,
                     out_tokens, out_n_acc, out_status, p_at, q_at, lse, done);
  SV_LAUNCH_CHECK();
  return SV_OK;
}
}  // namespace

extern "C" sv_status sv_verify_accept(const float* target_logits, const float* draft_logits,
                                      const int32_t* draft_tokens, int B, int k, int V,
                                      uint64_t seed, uint32_t offset, int32_t* out_tokens,
                                      int32_t* out_n_acc, int32_t* out_status, float* p_at,
                                      float* q_at, float* lse, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  return verify_accept(target_logits, nullptr, draft_logits, draft_tokens, B, k, V, seed, offset,
                       out_tokens, out_n_acc, out_status, p_at, q_at, lse, workspace,
                       workspace_bytes, stream);
}

extern "C" sv_status sv_verify_accept_stats(const float* target_logits, const float* target_stats,
                                            const float* draft_logits,
                                            const int32_t* draft_tokens, int B, int k, int V,
                                            uint64_t seed, uint32_t offset, int32_t* out_tokens,
                                            int32_t* out_n_acc, int32_t* out_status, float* p_at,
                                            float* q_at, float* lse, void* workspace,
                                            size_t workspace_bytes, hipStream_t stream) {
  if (!target_stats) return SV_ERR_NULL;
  return verify_accept(target_logits, target_stats, draft_logits, draft_tokens, B, k, V, seed,
                       offset, out_tokens, out_n_acc, out_status, p_at, q_at, lse, workspace,
                       workspace_bytes, stream);
}

extern "C" sv_status sv_philox4x32_10(const uint32_t* ctr, const uint32_t* key, uint32_t* out,
                                      int n, hipStream_t stream) {
  if (!ctr || !key || !out) return SV_ERR_NULL;
  if (n < 1) return SV_ERR_INVALID_ARG;
  hipLaunchKernelGGL(philox_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, ctr, key, out,
                     n);
  SV_LAUNCH_CHECK();
  return SV_OK;
}

// ---- no-allocation variant -----------------------------------------------
// The workspace of sv_verify_accept_noalloc: one fixed array per device,
// held until the process ends.  Host code never passes `scratch` itself (in
// host code the name is a stand-in, not a device address): it looks up each
// device's address once, with that device current, and passes that.
namespace {
__device__ __align__(256) unsigned char scratch[SV_ACCEPT_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];               // per device, set on first use

// Device address of this device's scratch array (nullptr on a HIP error).
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" size_t sv_verify_accept_noalloc_max_bytes(void) { return SV_ACCEPT_SCRATCH_BYTES; }

extern "C" sv_status sv_verify_accept_noalloc(const float* target_logits,
                                              const float* draft_logits,
                                              const int32_t* draft_tokens, int B, int k, int V,
                                              uint64_t seed, uint32_t offset,
                                              int32_t* out_tokens, int32_t* out_n_acc,
                                              int32_t* out_status, float* p_at, float* q_at,
                                              float* lse, hipStream_t stream) {
  if (B < 1 || k < 1 || k > SV_MAX_ROWS || V < 1) return SV_ERR_INVALID_ARG;
  if (static_cast<long long>(k + 1) * V >= (1LL << 31)) return SV_ERR_INVALID_ARG;
  const size_t need = ws_layout(B, k, V).bytes;
  if (need > SV_ACCEPT_SCRATCH_BYTES) return SV_ERR_WORKSPACE;   // beyond the fixed array
  if (!target_logits || !draft_logits || !draft_tokens || !out_tokens || !out_n_acc ||
      !out_status)
    return SV_ERR_NULL;
  void* ws = scratch_address();
  if (!ws) return SV_ERR_HIP;
  return verify_accept(target_logits, nullptr, draft_logits, draft_tokens, B, k, V, seed, offset,
                       out_tokens, out_n_acc, out_status, p_at, q_at, lse, ws, need, stream);
}
