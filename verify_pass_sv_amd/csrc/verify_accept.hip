// sv_verify_accept: fused vocabulary softmax for target and draft rows, the
// left-to-right accept scan, and the residual / bonus resample.
//
// Source: Speculative Decoding Clearly Explained, "Accept from left to right"
// (accept with probability min(1, p/q), stop at the first rejection) and
// "Correct and continue" (resample from max(0, p - q) normalized; if every
// draft is accepted the target supplies one more token); Karpathy's Trick for
// Faster Local LLMs, "Producing several tokens from one model pass".
//
// Three launches on the caller's stream:
//  1. stats   one wave per (trial, row, vocab chunk): online max / sum of
//             exp over 128-bit loads -> partial (max, sum, invalid flag).
//  2. decide  one workgroup per (trial, residual chunk): combines the
//             partials into log-sum-exp values, evaluates p_i(d_i), q_i(d_i),
//             draws Philox uniforms, takes the accept decisions with one
//             wave ballot (first rejection = first zero bit), then sums the
//             residual weights max(0, p_r - q_r) (or p_k for the bonus) of
//             its chunk in binary64.  Every workgroup of a trial reaches the
//             same decision; workgroup 0 writes the per-trial outputs.
//  3. select  one workgroup per trial: prefix over chunk totals, then inside
//             the chosen chunk over per-thread sums, then a walk inside one
//             thread's range.  Totals, prefixes and the walk use the same
//             binary64 addition order, so the chosen bin always exists.
#include "sv_common.h"

#include <math.h>

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kStatsWaves = 4;
constexpr int kThreads = 256;

struct StatPartial {
  float m;
  float s;
  int bad;
  int pad;
};

struct Decision {
  int status;
  int n_acc;
  float lse_t;
  float lse_d;
  double u2;
  double pad;
};

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two 32x32
// multiplies with the published multipliers, key bumped by the published
// Weyl constants between rounds.
__device__ __forceinline__ void philox4x32_10(unsigned int c[4], unsigned int k0,
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

__device__ __forceinline__ float u24(unsigned int w) {
  return static_cast<float>(w >> 8) * (1.0f / 16777216.0f);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

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

__host__ __device__ inline int stat_chunks(int B, int k, int V) {
  const long long rows = static_cast<long long>(B) * (2 * k + 1);
  long long c = (2048 + rows - 1) / rows;
  long long cmax = V / 2048;
  if (cmax < 1) cmax = 1;
  if (cmax > 64) cmax = 64;
  if (c > cmax) c = cmax;
  return static_cast<int>(c < 1 ? 1 : c);
}

__host__ __device__ inline int resid_chunks(int B, int V) {
  long long c = (256 + static_cast<long long>(B) - 1) / B;
  long long cmax = V / 2048;
  if (cmax < 1) cmax = 1;
  if (cmax > 64) cmax = 64;
  if (c > cmax) c = cmax;
  return static_cast<int>(c < 1 ? 1 : c);
}

struct WsLayout {
  size_t partial_off, decision_off, total_off, bytes;
};

__host__ inline WsLayout ws_layout(int B, int k, int V) {
  auto up = [](size_t v) { return (v + 255) & ~static_cast<size_t>(255); };
  WsLayout L;
  const size_t R = 2 * static_cast<size_t>(k) + 1;
  L.partial_off = 0;
  L.decision_off = up(static_cast<size_t>(B) * R * stat_chunks(B, k, V) * sizeof(StatPartial));
  L.total_off = L.decision_off + up(static_cast<size_t>(B) * sizeof(Decision));
  L.bytes = L.total_off + up(static_cast<size_t>(B) * resid_chunks(B, V) * sizeof(double));
  return L;
}

__device__ __forceinline__ const float* row_ptr(const float* tgt, const float* dft, int b, int j,
                                                int k, int V) {
  if (j <= k) return tgt + (static_cast<size_t>(b) * (k + 1) + j) * V;
  return dft + (static_cast<size_t>(b) * k + (j - k - 1)) * V;
}

// ---- kernel 1: per-chunk softmax statistics --------------------------------
template <bool VEC>
__global__ __launch_bounds__(64 * kStatsWaves) void stats_kernel(
    const float* __restrict__ tgt, const float* __restrict__ dft, int B, int k, int V, int C1,
    StatPartial* __restrict__ part) {
  const int lane = threadIdx.x & 63;
  const long long item = static_cast<long long>(blockIdx.x) * kStatsWaves + (threadIdx.x >> 6);
  const int R = 2 * k + 1;
  if (item >= static_cast<long long>(B) * R * C1) return;
  const int c = static_cast<int>(item % C1);
  const long long br = item / C1;
  const int j = static_cast<int>(br % R);
  const int b = static_cast<int>(br / R);
  const float* row = row_ptr(tgt, dft, b, j, k, V);
  int L = (V + C1 - 1) / C1;
  L = (L + 3) & ~3;
  const int lo = min(V, c * L);
  const int hi = min(V, lo + L);
  float m = -INFINITY, s = 0.f;
  int bad = 0;
  if (VEC) {
    for (int i = lo + lane * 4; i < hi; i += 256)
      stat_add4(m, s, bad, *reinterpret_cast<const float4*>(row + i));
  } else {
    for (int i = lo + lane; i < hi; i += 64) stat_add1(m, s, bad, row[i]);
  }
  for (int off = 32; off > 0; off >>= 1) {
    const float m2 = __shfl_xor(m, off);
    const float s2 = __shfl_xor(s, off);
    bad |= __shfl_xor(bad, off);
    stat_merge(m, s, m2, s2);
  }
  if (lane == 0) part[item] = StatPartial{m, s, bad, 0};
}

// Residual / bonus weight of vocab entry v (binary32), shared by kernels 2
// and 3 so that both see bit-identical weights.
__device__ __noinline__ float resid_weight(const float* pt, float lt, const float* pd, float ld,
                                           int v) {
  const float p = expf(pt[v] - lt);
  if (pd == nullptr) return p;
  const float q = expf(pd[v] - ld);
  return fmaxf(0.f, p - q);
}

__device__ __noinline__ double range_sum(const float* pt, float lt, const float* pd, float ld,
                                         int a, int e) {
  double acc = 0.0;
  for (int v = a; v < e; ++v) acc += static_cast<double>(resid_weight(pt, lt, pd, ld, v));
  return acc;
}

__device__ __forceinline__ void chunk_range(int V, int C2, int c, int& lo, int& hi) {
  const int L = (V + C2 - 1) / C2;
  lo = min(V, c * L);
  hi = min(V, lo + L);
}

__device__ __forceinline__ void thread_range(int lo, int hi, int t, int& a, int& e) {
  const long long len = hi - lo;
  a = lo + static_cast<int>(len * t / kThreads);
  e = lo + static_cast<int>(len * (t + 1) / kThreads);
}

// ---- kernel 2: decide + residual chunk totals ------------------------------
__global__ __launch_bounds__(kThreads) void decide_kernel(
    const float* __restrict__ tgt, const float* __restrict__ dft, const int32_t* __restrict__ toks,
    int B, int k, int V, int C1, int C2, unsigned int key0, unsigned int key1, unsigned int offset,
    const StatPartial* __restrict__ part, Decision* __restrict__ decs, double* __restrict__ totals,
    int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_n_acc,
    int32_t* __restrict__ out_status, float* __restrict__ p_at, float* __restrict__ q_at,
    float* __restrict__ lse_out) {
  __shared__ float lse_sh[2 * SV_MAX_ROWS + 1];
  __shared__ int bad_sh[2 * SV_MAX_ROWS + 1];
  __shared__ Decision dec;
  __shared__ double tsum[kThreads];
  const int b = blockIdx.x / C2;
  const int c = blockIdx.x % C2;
  const int R = 2 * k + 1;
  const int tid = threadIdx.x;

  if (tid < R) {
    const StatPartial* pp = part + (static_cast<size_t>(b) * R + tid) * C1;
    float m = -INFINITY, s = 0.f;
    int bad = 0;
    for (int i = 0; i < C1; ++i) {
      bad |= pp[i].bad;
      stat_merge(m, s, pp[i].m, pp[i].s);
    }
    bad |= (m == -INFINITY) || !(s > 0.f);
    lse_sh[tid] = bad ? NAN : m + logf(s);
    bad_sh[tid] = bad;
  }
  __syncthreads();

  if (tid < 64) {
    const int i = tid;
    const bool has_draft = i < k;
    int tok = 0;
    bool tok_bad = false;
    if (has_draft) {
      tok = toks[static_cast<size_t>(b) * k + i];
      tok_bad = tok < 0 || tok >= V;
    }
    const bool row_bad = (i < R && bad_sh[i]) || (i + 64 < R && bad_sh[i + 64]);
    const bool any_tok_bad = __any(tok_bad);
    const bool any_row_bad = __any(row_bad);
    const int status = any_tok_bad ? 1 : (any_row_bad ? 2 : 0);

    float p = NAN, q = NAN, u2 = 0.f;
    bool accepted = true;
    if (i <= k) {
      unsigned int ctr[4] = {static_cast<unsigned int>(i), static_cast<unsigned int>(b), offset, 0u};
      philox4x32_10(ctr, key0, key1);
      const float u = u24(ctr[0]);
      u2 = u24(ctr[1]);
      if (has_draft && status == 0) {
        const float tl = tgt[(static_cast<size_t>(b) * (k + 1) + i) * V + tok];
        const float dl = dft[(static_cast<size_t>(b) * k + i) * V + tok];
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
      if (i <= k) {
        // accepted drafts; position n_acc is written by the select kernel
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

  double* tot = totals + static_cast<size_t>(b) * C2 + c;
  if (dec.status != 0) {
    if (tid == 0) *tot = 0.0;
    return;
  }
  const int r = dec.n_acc;
  const float* pt = tgt + (static_cast<size_t>(b) * (k + 1) + r) * V;
  const float* pd = r < k ? dft + (static_cast<size_t>(b) * k + r) * V : nullptr;
  int lo, hi, a, e;
  chunk_range(V, C2, c, lo, hi);
  thread_range(lo, hi, tid, a, e);
  tsum[tid] = range_sum(pt, dec.lse_t, pd, dec.lse_d, a, e);
  __syncthreads();
  if (tid == 0) {
    double acc = 0.0;
    for (int t = 0; t < kThreads; ++t) acc += tsum[t];
    *tot = acc;
  }
}

// ---- kernel 3: select the replacement / bonus token ------------------------
__global__ __launch_bounds__(kThreads) void select_kernel(
    const float* __restrict__ tgt, const float* __restrict__ dft, int k, int V, int C2,
    const Decision* __restrict__ decs, const double* __restrict__ totals,
    int32_t* __restrict__ out_tokens) {
  __shared__ double tsum[kThreads];
  __shared__ double sh_thr, sh_pc, sh_qt;
  __shared__ int sh_c, sh_t, sh_usep;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const Decision dec = decs[b];
  if (dec.status != 0) return;
  const int r = dec.n_acc;
  const float* pt = tgt + (static_cast<size_t>(b) * (k + 1) + r) * V;
  const float* pd = r < k ? dft + (static_cast<size_t>(b) * k + r) * V : nullptr;

  if (tid == 0) {
    const double* T = totals + static_cast<size_t>(b) * C2;
    double S = 0.0;
    for (int c = 0; c < C2; ++c) S += T[c];
    sh_usep = !(S > 0.0);
  }
  __syncthreads();
  const bool usep = sh_usep != 0;
  if (usep) pd = nullptr;  // rounding left no residual mass: sample from p_r

  // Chunk totals: from kernel 2, or recomputed here for the p_r fallback.
  double* ctot = nullptr;
  __shared__ double ctot_sh[64];
  if (usep) {
    for (int c = 0; c < C2; ++c) {
      int lo, hi, a, e;
      chunk_range(V, C2, c, lo, hi);
      thread_range(lo, hi, tid, a, e);
      tsum[tid] = range_sum(pt, dec.lse_t, pd, dec.lse_d, a, e);
      __syncthreads();
      if (tid == 0) {
        double acc = 0.0;
        for (int t = 0; t < kThreads; ++t) acc += tsum[t];
        ctot_sh[c] = acc;
      }
      __syncthreads();
    }
    ctot = ctot_sh;
  }
  if (tid == 0) {
    const double* T = usep ? ctot : totals + static_cast<size_t>(b) * C2;
    double S = 0.0;
    for (int c = 0; c < C2; ++c) S += T[c];
    const double thr = dec.u2 * S;
    double P = 0.0;
    int cs = C2 - 1;
    double pc = 0.0;
    for (int c = 0; c < C2; ++c) {
      const double nxt = P + T[c];
      if (nxt > thr) {
        cs = c;
        pc = P;
        break;
      }
      P = nxt;
      pc = P;
    }
    sh_thr = thr;
    sh_c = cs;
    sh_pc = pc;
  }
  __syncthreads();
  const double thr = sh_thr, pc = sh_pc;
  int lo, hi, a, e;
  chunk_range(V, C2, sh_c, lo, hi);
  thread_range(lo, hi, tid, a, e);
  tsum[tid] = range_sum(pt, dec.lse_t, pd, dec.lse_d, a, e);
  __syncthreads();
  if (tid == 0) {
    double Q = 0.0;
    int ts = kThreads - 1;
    double qt = 0.0;
    for (int t = 0; t < kThreads; ++t) {
      const double nxt = Q + tsum[t];
      if (pc + nxt > thr) {
        ts = t;
        qt = Q;
        break;
      }
      Q = nxt;
      qt = Q;
    }
    sh_t = ts;
    sh_qt = qt;
  }
  __syncthreads();
  if (tid == sh_t) {
    const double qt = sh_qt;
    int tok = -1, last_pos = -1;
    double run = 0.0;
    for (int v = a; v < e; ++v) {
      const float w = resid_weight(pt, dec.lse_t, pd, dec.lse_d, v);
      run += static_cast<double>(w);
      if (w > 0.f) last_pos = v;
      if (pc + (qt + run) > thr) {
        tok = v;
        break;
      }
    }
    if (tok < 0) tok = last_pos >= 0 ? last_pos : (e > a ? e - 1 : lo);
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
  philox4x32_10(c, key[2 * i], key[2 * i + 1]);
  for (int j = 0; j < 4; ++j) out[4 * i + j] = c[j];
}

}  // namespace

extern "C" size_t sv_verify_accept_workspace_bytes(int B, int k, int V) {
  if (B < 1 || k < 1 || k > SV_MAX_ROWS || V < 1) return 0;
  return ws_layout(B, k, V).bytes;
}

extern "C" sv_status sv_verify_accept(const float* target_logits, const float* draft_logits,
                                      const int32_t* draft_tokens, int B, int k, int V,
                                      uint64_t seed, uint32_t offset, int32_t* out_tokens,
                                      int32_t* out_n_acc, int32_t* out_status, float* p_at,
                                      float* q_at, float* lse, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  if (!target_logits || !draft_logits || !draft_tokens || !out_tokens || !out_n_acc ||
      !out_status)
    return SV_ERR_NULL;
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
  const int C1 = stat_chunks(B, k, V);
  const int C2 = resid_chunks(B, V);
  const long long items = static_cast<long long>(B) * (2 * k + 1) * C1;
  const long long blocks1 = (items + kStatsWaves - 1) / kStatsWaves;
  if (blocks1 >= (1LL << 31) || static_cast<long long>(B) * C2 >= (1LL << 31))
    return SV_ERR_INVALID_ARG;

  if (V % 4 == 0)
    hipLaunchKernelGGL((stats_kernel<true>), dim3(static_cast<unsigned>(blocks1)),
                       dim3(64 * kStatsWaves), 0, stream, target_logits, draft_logits, B, k, V,
                       C1, part);
  else
    hipLaunchKernelGGL((stats_kernel<false>), dim3(static_cast<unsigned>(blocks1)),
                       dim3(64 * kStatsWaves), 0, stream, target_logits, draft_logits, B, k, V,
                       C1, part);
  SV_LAUNCH_CHECK();
  hipLaunchKernelGGL(decide_kernel, dim3(static_cast<unsigned>(B) * C2), dim3(kThreads), 0,
                     stream, target_logits, draft_logits, draft_tokens, B, k, V, C1, C2,
                     static_cast<unsigned int>(seed & 0xFFFFFFFFu),
                     static_cast<unsigned int>(seed >> 32), offset, part, decs, totals,
                     out_tokens, out_n_acc, out_status, p_at, q_at, lse);
  SV_LAUNCH_CHECK();
  hipLaunchKernelGGL(select_kernel, dim3(static_cast<unsigned>(B)), dim3(kThreads), 0, stream,
                     target_logits, draft_logits, k, V, C2, decs, totals, out_tokens);
  SV_LAUNCH_CHECK();
  return SV_OK;
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
