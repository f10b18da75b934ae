// Verification by target choices: sv_verify_coupled (Gumbel-max coupled
// verification) and sv_verify_tree (greedy verification of a draft tree).
//
// Source: @trymirai timeline, the post on speculators that predict the
// distribution correctly and are still rejected: sample both the speculator
// and the LLM with the same seed through the Gumbel-max trick, so matching
// distributions give matching tokens; Speculative Decoding Clearly Explained,
// "Accept from left to right" and "Correct and continue" (keep the drafts up
// to the first disagreement, emit the target's token there, one more after k
// agreements).
//
// Tree source: Karpathy's Trick for Faster Local LLMs, "Issue with parallel
// draft generation" and "Verifying a draft tree without restoring model
// state" (the main model verifies the tree and accepts the longest valid
// path); Local LLM 4x Faster (the whole tree verified at once).
//
// Two launches on the caller's stream:
//  1. choose  one workgroup per (4096-entry vocabulary span, target row,
//             trial): the best score over the span -- l + g with the Gumbel
//             noise g = -log(-log u) in binary64 from the Philox uniform of
//             word v mod 4 of counter (v / 4, i, b, 3 + 256 offset) for
//             coupled verification, l alone for the tree; partial (score,
//             index, validity).
//  2. decide  one wave per trial: lane r merges the spans of target row r
//             (score down, index up), then the status checks and
//             coupled: the first disagreement (one ballot);
//             tree: the valid nodes and their depths by pointer jumping over
//             the parent links, the longest valid chain (a wave maximum) and
//             its bonus.
#include "sv_common.h"
#include "sv_philox.h"

#include <math.h>

namespace {

constexpr int kThreads = 256;
constexpr int kSpan = 4096;                     // vocabulary entries per span
constexpr unsigned int kTagCoupled = 3u;

struct CoupledPartial {
  double score;                                 // best l + g of the span (-inf if none)
  int index;                                    // its smallest index
  int flags;                                    // bit 0: NaN or +inf seen; bit 1: finite logit seen
};
static_assert(sizeof(CoupledPartial) == 16, "partial layout");

__host__ __device__ inline int coupled_spans(int V) { return (V + kSpan - 1) / kSpan; }

__device__ __forceinline__ bool better(double s, int v, double bs, int bv) {
  return s > bs || (s == bs && v < bv);
}

// Merges the span partials of one target row in span order (score down,
// index up), loading up to 40 partials at a time (every span of a vocabulary
// up to 163 840 entries) so that one memory latency covers them.
__device__ __forceinline__ void merge_spans(const CoupledPartial* __restrict__ p, int spans,
                                            double& best, int& bi, int& flags) {
  constexpr int kUnroll = 40;
  for (int s0 = 0; s0 < spans; s0 += kUnroll) {
    CoupledPartial q[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j)
      if (s0 + j < spans) q[j] = p[s0 + j];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      if (s0 + j < spans) {
        if (better(q[j].score, q[j].index, best, bi)) {
          best = q[j].score;
          bi = q[j].index;
        }
        flags |= q[j].flags;
      }
    }
  }
}

// Rows of [B, rows, V] logits: rows = k + 1 (coupled) or n + 1 (tree).
template <bool NOISE>
__global__ __launch_bounds__(kThreads) void choose_kernel(
    const float* __restrict__ tgt, int k, int V, unsigned int key0, unsigned int key1,
    unsigned int tagword, CoupledPartial* __restrict__ parts) {
  __shared__ double ssh[kThreads];
  __shared__ int ish[kThreads];
  __shared__ int fsh[kThreads];
  __shared__ double wmax[kThreads / 64];
  const int tid = threadIdx.x;
  const int span = blockIdx.x;
  const int i = blockIdx.y;
  const int b = blockIdx.z;
  const float* row = tgt + (static_cast<size_t>(b) * (k + 1) + i) * V;
  const int v0 = span * kSpan;
  const int v1 = min(V, v0 + kSpan);
  double best = -INFINITY;
  int bi = V;
  int flags = 0;
  // the thread's 16 entries are 4 runs of 4 consecutive ones (one Philox
  // counter each, its four words for the four entries); every load goes out
  // before any is used
  constexpr int kRuns = kSpan / (4 * kThreads);
  const bool vec = (V & 3) == 0;                // rows 16-byte aligned
  float xs[kRuns][4];
#pragma unroll
  for (int g = 0; g < kRuns; ++g) {
    const int vb = v0 + 4 * (tid + g * kThreads);
    if (vec) {
      // V % 4 == 0 makes v1 a multiple of 4: the whole run is in the span
      const float4 a = vb < v1 ? *reinterpret_cast<const float4*>(row + vb)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
      xs[g][0] = a.x;
      xs[g][1] = a.y;
      xs[g][2] = a.z;
      xs[g][3] = a.w;
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) xs[g][q] = vb + q < v1 ? row[vb + q] : 0.f;
    }
  }
  if constexpr (NOISE) {
    // Screen in binary32: g32 = -logf(-logf(u)) is within 4e-6 of the
    // binary64 noise for every 24-bit u (logf within 1 ulp; -log u in
    // [6e-8, 16.7]).  With M the workgroup's best screened score, the
    // binary64 winner's screened score is at least M - 2 margin, so only
    // entries at or above that take the binary64 logarithms.
    double ap[kRuns][4];
    unsigned int wd[kRuns][4];
    double m = -INFINITY;
#pragma unroll
    for (int g = 0; g < kRuns; ++g) {
      const int vb = v0 + 4 * (tid + g * kThreads);
      unsigned int c[4] = {static_cast<unsigned int>(vb >> 2), static_cast<unsigned int>(i),
                           static_cast<unsigned int>(b), tagword};
      sv_philox_rounds(c, key0, key1);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float x = xs[g][q];
        const bool in = vb + q < v1;
        wd[g][q] = c[q];
        const float g32 = -logf(-logf(sv_u24(c[q])));
        const double a = static_cast<double>(x) + static_cast<double>(g32);
        ap[g][q] = a;
        if (in) {
          flags |= ((x != x) | (x == INFINITY)) ? 1 : 0;
          flags |= (x > -INFINITY && x < INFINITY) ? 2 : 0;
          if (a > m) m = a;                       // NaN never
        }
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double t = __shfl_xor(m, o, 64);
      if (t > m) m = t;
    }
    if ((tid & 63) == 0) wmax[tid >> 6] = m;
    __syncthreads();
    double M = wmax[0];
    for (int w = 1; w < kThreads / 64; ++w)
      if (wmax[w] > M) M = wmax[w];
    const double thr = isinf(M) ? M : M - 2.0 * (1e-4 + fabs(M) * 0x1p-40);
#pragma unroll
    for (int g = 0; g < kRuns; ++g) {
      const int vb = v0 + 4 * (tid + g * kThreads);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int v = vb + q;
        if (v < v1 && ap[g][q] >= thr) {
          const double u = static_cast<double>(sv_u24(wd[g][q]));  // 24 bits: exact
          const double sc = static_cast<double>(xs[g][q]) - log(-log(u));   // u = 0: -inf
          if (better(sc, v, best, bi)) {
            best = sc;
            bi = v;
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int g = 0; g < kRuns; ++g) {
      const int vb = v0 + 4 * (tid + g * kThreads);
      if (vb >= v1) break;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int v = vb + q;
        if (v >= v1) break;
        const float x = xs[g][q];
        flags |= ((x != x) | (x == INFINITY)) ? 1 : 0;
        flags |= (x > -INFINITY && x < INFINITY) ? 2 : 0;
        const double sc = static_cast<double>(x);
        if (better(sc, v, best, bi)) {
          best = sc;
          bi = v;
        }
      }
    }
  }
  ssh[tid] = best;
  ish[tid] = bi;
  fsh[tid] = flags;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (tid < w) {
      if (better(ssh[tid + w], ish[tid + w], ssh[tid], ish[tid])) {
        ssh[tid] = ssh[tid + w];
        ish[tid] = ish[tid + w];
      }
      fsh[tid] |= fsh[tid + w];
    }
    __syncthreads();
  }
  if (tid == 0) {
    CoupledPartial p;
    p.score = ssh[0];
    p.index = ish[0];
    p.flags = fsh[0];
    parts[(static_cast<size_t>(b) * (k + 1) + i) * gridDim.x + span] = p;
  }
}

__global__ __launch_bounds__(64) void coupled_decide_kernel(
    const int32_t* __restrict__ toks, int k, int V, int spans,
    const CoupledPartial* __restrict__ parts, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ out_n_acc, int32_t* __restrict__ out_status,
    int32_t* __restrict__ choices) {
  const int lane = threadIdx.x;
  const int b = blockIdx.x;
  const bool is_row = lane <= k;
  double best = -INFINITY;
  int bi = V;
  int flags = 0;
  if (is_row)
    merge_spans(parts + (static_cast<size_t>(b) * (k + 1) + lane) * spans, spans, best, bi,
                flags);
  const bool row_bad = is_row && ((flags & 1) || !(flags & 2));
  int tok = 0;
  bool tok_bad = false;
  if (lane < k) {
    tok = toks[static_cast<size_t>(b) * k + lane];
    tok_bad = tok < 0 || tok >= V;
  }
  const int status = __any(tok_bad) ? 1 : (__any(row_bad) ? 2 : 0);
  const unsigned long long mism = __ballot(lane < k && tok != bi);
  const int n_acc = mism ? (__ffsll(static_cast<long long>(mism)) - 1) : k;
  const int pick = __shfl(bi, n_acc);
  int32_t* ot = out_tokens + static_cast<size_t>(b) * (k + 1);
  if (is_row) {
    ot[lane] = status != 0 ? -1 : (lane < n_acc ? tok : (lane == n_acc ? pick : -1));
    if (choices) choices[static_cast<size_t>(b) * (k + 1) + lane] = status != 0 ? -1 : bi;
  }
  if (lane == 0) {
    out_n_acc[b] = status == 0 ? n_acc : -1;
    out_status[b] = status;
  }
}

// pars == nullptr: a chain (node j's parent is node j - 1), which is greedy
// verification of n drafts; p_at / q_at (nullable) then receive 1 or 0 for
// d_j == argmax of target row j, and 1 (NaN for both when status != 0).
__global__ __launch_bounds__(64) void tree_decide_kernel(
    const int32_t* __restrict__ toks, const int32_t* __restrict__ pars, int n, int V, int spans,
    const CoupledPartial* __restrict__ parts, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ out_n_acc, int32_t* __restrict__ out_status,
    int32_t* __restrict__ out_path, float* __restrict__ p_at, float* __restrict__ q_at) {
  __shared__ int choice[SV_MAX_ROWS + 1];
  __shared__ int tok_sh[SV_MAX_ROWS], path[SV_MAX_ROWS];
  __shared__ int res[3];                        // status, path length, bonus row
  const int lane = threadIdx.x;
  const int b = blockIdx.x;
  const bool is_row = lane <= n;
  double best = -INFINITY;
  int bi = V;
  int flags = 0;
  if (is_row) {
    merge_spans(parts + (static_cast<size_t>(b) * (n + 1) + lane) * spans, spans, best, bi,
                flags);
    choice[lane] = bi;
  }
  const bool row_bad = is_row && ((flags & 1) || !(flags & 2));
  int tok = 0, par = -1;
  bool tok_bad = false, par_bad = false;
  if (lane < n) {
    tok = toks[static_cast<size_t>(b) * n + lane];
    par = pars ? pars[static_cast<size_t>(b) * n + lane] : lane - 1;
    tok_bad = tok < 0 || tok >= V;
    par_bad = par < -1 || par >= lane;
    tok_sh[lane] = tok;
  }
  const int status = __any(tok_bad) ? 1 : (__any(row_bad) ? 2 : (__any(par_bad) ? 3 : 0));
  // Node j on lane j.  It matches when its token is the target's choice at
  // its parent's row (lane p + 1 holds row p + 1's choice).  Pointer jumping
  // over the parent links (5 rounds cover depths up to 32): ok becomes the
  // AND of the matches from the root down to the node, d the node's depth,
  // and jmp[r] keeps each node's 2^r-th ancestor for the path below.
  static_assert(SV_MAX_ROWS <= 32, "5 jumping rounds cover trees of at most 32 nodes");
  const int pchoice = __shfl(bi, par + 1 < 0 ? 0 : par + 1);
  int ok = lane < n && status == 0 && tok == pchoice;
  if (lane < n) {
    if (p_at) p_at[static_cast<size_t>(b) * n + lane] = status == 0 ? (ok ? 1.f : 0.f) : NAN;
    if (q_at) q_at[static_cast<size_t>(b) * n + lane] = status == 0 ? 1.f : NAN;
  }
  int a = lane < n ? par : -1;
  int d = lane < n ? 1 : 0;
  int jmp[5];
#pragma unroll
  for (int r = 0; r < 5; ++r) {
    jmp[r] = a;
    const int src = a < 0 ? lane : a;
    const int ok_a = __shfl(ok, src);
    const int d_a = __shfl(d, src);
    const int a_a = __shfl(a, src);
    if (a >= 0) {
      ok &= ok_a;
      d += d_a;
      a = a_a;
    }
  }
  const int depth = ok ? d : 0;
  // the deepest valid node, the smallest index among equal depths
  int key = depth > 0 ? (depth << 6) | (63 - lane) : 0;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) key = max(key, __shfl_xor(key, off));
  const int end = key > 0 ? 63 - (key & 63) : -1;
  const int len_v = key >> 6;
  // node j lies on the chosen path iff it is end's ancestor at distance
  // len - depth (binary lifting with the jump pointers)
  {
    const int dist = len_v - depth;
    int x = end;
#pragma unroll
    for (int r = 0; r < 5; ++r) {
      const int nx = __shfl(jmp[r], x < 0 ? 0 : x);
      if (((dist >> r) & 1) && x >= 0) x = nx;
    }
    if (depth > 0 && dist >= 0 && x == lane) path[depth - 1] = lane;
  }
  if (lane == 0) {
    res[0] = status;
    res[1] = status == 0 ? len_v : -1;
    res[2] = end + 1;
  }
  __syncthreads();
  const int len = res[1];
  int32_t* ot = out_tokens + static_cast<size_t>(b) * (n + 1);
  if (lane <= n) {
    int v = -1;
    if (status == 0) v = lane < len ? tok_sh[path[lane]] : (lane == len ? choice[res[2]] : -1);
    ot[lane] = v;
  }
  if (out_path && lane < n)
    out_path[static_cast<size_t>(b) * n + lane] = status == 0 && lane < len ? path[lane] : -1;
  if (lane == 0) {
    out_n_acc[b] = len;
    out_status[b] = status;
  }
}

}  // namespace

extern "C" size_t sv_verify_coupled_workspace_bytes(int B, int k, int V) {
  if (B < 1 || k < 1 || k > SV_MAX_ROWS || V < 1) return 0;
  return static_cast<size_t>(B) * (k + 1) * coupled_spans(V) * sizeof(CoupledPartial);
}

extern "C" sv_status sv_verify_coupled(const float* target_logits, const int32_t* draft_tokens,
                                       int B, int k, int V, uint64_t seed, uint32_t offset,
                                       int32_t* out_tokens, int32_t* out_n_acc,
                                       int32_t* out_status, int32_t* choices, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
  if (!target_logits || !draft_tokens || !out_tokens || !out_n_acc || !out_status)
    return SV_ERR_NULL;
  if (B < 1 || B > 65535 || k < 1 || k > SV_MAX_ROWS || V < 1 || offset >= (1u << 24))
    return SV_ERR_INVALID_ARG;
  if (static_cast<long long>(k + 1) * V >= (1LL << 31)) return SV_ERR_INVALID_ARG;
  if (!sv_aligned16(target_logits) || !sv_aligned16(draft_tokens) || !sv_aligned16(out_tokens) ||
      !sv_aligned16(out_n_acc) || !sv_aligned16(out_status) ||
      (choices && !sv_aligned16(choices)))
    return SV_ERR_ALIGN;
  if (!workspace || workspace_bytes < sv_verify_coupled_workspace_bytes(B, k, V))
    return SV_ERR_WORKSPACE;
  if (!sv_aligned16(workspace)) return SV_ERR_ALIGN;
  const int spans = coupled_spans(V);
  CoupledPartial* parts = static_cast<CoupledPartial*>(workspace);
  hipLaunchKernelGGL(choose_kernel<true>, dim3(spans, k + 1, B), dim3(kThreads), 0, stream,
                     target_logits, k, V, static_cast<unsigned int>(seed & 0xFFFFFFFFu),
                     static_cast<unsigned int>(seed >> 32), kTagCoupled + (offset << 8), parts);
  SV_LAUNCH_CHECK();
  hipLaunchKernelGGL(coupled_decide_kernel, dim3(B), dim3(64), 0, stream, draft_tokens, k, V,
                     spans, parts, out_tokens, out_n_acc, out_status, choices);
  SV_LAUNCH_CHECK();
  return SV_OK;
}

extern "C" size_t sv_verify_tree_workspace_bytes(int B, int n, int V) {
  if (B < 1 || n < 1 || n > SV_MAX_ROWS || V < 1) return 0;
  return static_cast<size_t>(B) * (n + 1) * coupled_spans(V) * sizeof(CoupledPartial);
}

extern "C" sv_status sv_verify_tree(const float* target_logits, const int32_t* tokens,
                                    const int32_t* parents, int B, int n, int V,
                                    int32_t* out_tokens, int32_t* out_n_acc,
                                    int32_t* out_status, int32_t* out_path, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  if (!target_logits || !tokens || !parents || !out_tokens || !out_n_acc || !out_status)
    return SV_ERR_NULL;
  if (B < 1 || B > 65535 || n < 1 || n > SV_MAX_ROWS || V < 1) return SV_ERR_INVALID_ARG;
  if (static_cast<long long>(n + 1) * V >= (1LL << 31)) return SV_ERR_INVALID_ARG;
  if (!sv_aligned16(target_logits) || !sv_aligned16(tokens) || !sv_aligned16(parents) ||
      !sv_aligned16(out_tokens) || !sv_aligned16(out_n_acc) || !sv_aligned16(out_status) ||
      (out_path && !sv_aligned16(out_path)))
    return SV_ERR_ALIGN;
  if (!workspace || workspace_bytes < sv_verify_tree_workspace_bytes(B, n, V))
    return SV_ERR_WORKSPACE;
  if (!sv_aligned16(workspace)) return SV_ERR_ALIGN;
  const int spans = coupled_spans(V);
  CoupledPartial* parts = static_cast<CoupledPartial*>(workspace);
  hipLaunchKernelGGL(choose_kernel<false>, dim3(spans, n + 1, B), dim3(kThreads), 0, stream,
                     target_logits, n, V, 0u, 0u, 0u, parts);
  SV_LAUNCH_CHECK();
  hipLaunchKernelGGL(tree_decide_kernel, dim3(B), dim3(64), 0, stream, tokens, parents, n, V,
                     spans, parts, out_tokens, out_n_acc, out_status, out_path, nullptr,
                     nullptr);
  SV_LAUNCH_CHECK();
  return SV_OK;
}

// Greedy verification of k drafts (sv_verify_sampled at temperature 0) as the
// chain tree d_0 <- d_1 <- ..: the argmax of target row i is node i's parent
// choice, the longest valid chain is the matching prefix and the bonus is the
// argmax of the row after it.  Arguments are validated by the caller; the
// workspace holds sv_greedy_chain_workspace_bytes(B, k, V) bytes.
size_t sv_greedy_chain_workspace_bytes(int B, int k, int V) {
  return static_cast<size_t>(B) * (k + 1) * coupled_spans(V) * sizeof(CoupledPartial);
}
sv_status sv_greedy_chain(const float* target_logits, const int32_t* draft_tokens, int B, int k,
                          int V, int32_t* out_tokens, int32_t* out_n_acc, int32_t* out_status,
                          float* p_at, float* q_at, void* workspace, hipStream_t stream) {
  const int spans = coupled_spans(V);
  CoupledPartial* parts = static_cast<CoupledPartial*>(workspace);
  hipLaunchKernelGGL(choose_kernel<false>, dim3(spans, k + 1, B), dim3(kThreads), 0, stream,
                     target_logits, k, V, 0u, 0u, 0u, parts);
  SV_LAUNCH_CHECK();
  hipLaunchKernelGGL(tree_decide_kernel, dim3(B), dim3(64), 0, stream, draft_tokens, nullptr, k,
                     V, spans, parts, out_tokens, out_n_acc, out_status, nullptr, p_at, q_at);
  SV_LAUNCH_CHECK();
  return SV_OK;
}
