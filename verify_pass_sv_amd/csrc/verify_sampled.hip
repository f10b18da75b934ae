// sv_verify_sampled: verification under a request's sampling settings --
// temperature, top-k, top-p -- and greedy verification (temperature 0).
//
// Source: Karpathy's Trick for Faster Local LLMs, "Call Uzu through a local
// application endpoint" (the local server honours temperature, top_p and
// top_k) and "Use one client for Uzu, MLX, and llama.cpp" (temperature 0: the
// same answer on every run); Speculative Decoding Clearly Explained, "Accept
// from left to right" and "Correct and continue", applied to the truncated
// distributions.
//
// Two launches on the caller's stream:
//  1. rows    one workgroup per (trial, row), target rows 0..k then draft rows
//             0..k-1.  It checks the row and takes its maximum; for greedy
//             settings also the argmax (smallest index among equal maxima).
//             Otherwise it describes the kept set by a key threshold and a
//             tie cut: token v is kept iff key(l_v) > tau, or key(l_v) == tau
//             and v <= tie, where key() maps binary32 order to unsigned order.
//               top-k: radix selection of the top_k-th largest key (4 passes
//                 of 8-bit digits, integer histograms), then one ordered pass
//                 for the tie cut;
//               top-p: an 8-bit-digit search of the boundary key on binary64
//                 mass sums (4 passes), the number of tied tokens at the
//                 boundary from its mass, then an ordered pass.
//             Then the kept mass S (binary64, fixed order) and the kept
//             probability of the row's draft token.  Masses are exp((l - m)
//             / T) in binary64 throughout.
//  2. decide  one workgroup per trial: the accept scan on the kept
//             probabilities (binary64) with the Philox uniforms of
//             sv_verify_accept, then
//             the replacement/bonus draw over the kept rows: per-thread
//             contiguous chunks summed in binary64, an exclusive scan, and the
//             chosen chunk replayed in the same order.
#include "sv_common.h"
#include "sv_philox.h"

#include <math.h>

namespace {

constexpr int kThreads = 256;

struct SampledRow {                 // per (trial, row), written by launch 1
  float m;                          // row maximum
  float temp;                       // temperature
  unsigned int tau;                 // kept iff key > tau || (key == tau && v <= tie)
  int tie;
  double s;                         // kept mass: sum of exp((l - m) / T)
  double pd;                        // kept probability of the row's draft token
  int status;                       // 0 ok, 2 NaN / +inf / no finite logit
  int argmax;                       // smallest index of the maximum
};
static_assert(sizeof(SampledRow) == 40, "row record layout");

// Binary32 order as unsigned order (NaN excluded): negative values reversed.
__device__ __forceinline__ unsigned int order_key(float x) {
  const unsigned int b = __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_value(unsigned int key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}
__device__ __forceinline__ bool kept_by(unsigned int key, int v, unsigned int tau, int tie) {
  return key > tau || (key == tau && v <= tie);
}
// Unnormalised probability exp((x - m) / T) in binary64: the difference of two
// binary32 values is exact there, so the masses that place the top-p
// boundary and the probabilities of the accept test carry binary64 accuracy.
__device__ __forceinline__ double mass(float x, float m, float T) {
  return exp((static_cast<double>(x) - static_cast<double>(m)) / static_cast<double>(T));
}

// Fixed-order workgroup reductions (every thread gets the result).
__device__ double block_sum(double x, double* sh) {
  const int tid = threadIdx.x;
  sh[tid] = x;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (tid < w) sh[tid] += sh[tid + w];
    __syncthreads();
  }
  const double r = sh[0];
  __syncthreads();
  return r;
}
__device__ int block_sum_int(int x, int* sh) {
  const int tid = threadIdx.x;
  sh[tid] = x;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (tid < w) sh[tid] += sh[tid + w];
    __syncthreads();
  }
  const int r = sh[0];
  __syncthreads();
  return r;
}

// Index of the want-th (1-based) token, in vocabulary order, with key == tau
// among those kept by (tau0, tie0); V when there are fewer.  Threads own
// contiguous chunks; an exclusive scan of their counts finds the owner.
__device__ int ordered_tie(const float* row, int V, unsigned int tau, int want,
                           unsigned int tau0, int tie0, int* ish) {
  const int tid = threadIdx.x;
  const int chunk = (V + kThreads - 1) / kThreads;
  const int v0 = tid * chunk, v1 = min(V, v0 + chunk);
  int c = 0;
  for (int v = v0; v < v1; ++v) {
    const unsigned int key = order_key(row[v]);
    c += key == tau && kept_by(key, v, tau0, tie0);
  }
  ish[tid] = c;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int t = 0; t < kThreads; ++t) {
      const int n = ish[t];
      ish[t] = run;
      run += n;
    }
    ish[kThreads] = V;
  }
  __syncthreads();
  const int pre = ish[tid];
  if (pre < want && want <= pre + c) {
    int seen = pre;
    for (int v = v0; v < v1; ++v) {
      const unsigned int key = order_key(row[v]);
      if (key == tau && kept_by(key, v, tau0, tie0) && ++seen == want) {
        ish[kThreads] = v;
        break;
      }
    }
  }
  __syncthreads();
  const int r = ish[kThreads];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kThreads) void sampled_rows_kernel(
    const float* __restrict__ tgt, const float* __restrict__ dft, const int32_t* __restrict__ toks,
    int k, int V, float temperature, int top_k, float top_p, SampledRow* __restrict__ rows) {
  __shared__ double dsh[kThreads];
  __shared__ double above_sh;
  __shared__ int ish[kThreads + 1];
  __shared__ float fsh[kThreads];
  __shared__ int ash[kThreads];
  const int tid = threadIdx.x;
  const int rho = blockIdx.x;                   // 0..k target rows, k+1..2k draft rows
  const int b = blockIdx.y;
  const int R = 2 * k + 1;
  const bool is_t = rho <= k;
  const int i = is_t ? rho : rho - k - 1;
  const float* row = is_t ? tgt + (static_cast<size_t>(b) * (k + 1) + i) * V
                          : dft + (static_cast<size_t>(b) * k + i) * V;
  const int tok = i < k ? toks[static_cast<size_t>(b) * k + i] : -1;
  SampledRow out = {};

  // maximum, argmax (smallest index among equal maxima), validity
  float mx = -INFINITY;
  int am = V;
  int bad = 0;
  for (int v = tid; v < V; v += kThreads) {
    const float x = row[v];
    bad |= (x != x) | (x == INFINITY);
    if (x > mx) {
      mx = x;
      am = v;
    }
  }
  fsh[tid] = mx;
  ash[tid] = am;
  ish[tid] = bad;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (tid < w) {
      const float o = fsh[tid + w];
      const int oa = ash[tid + w];
      if (o > fsh[tid] || (o == fsh[tid] && oa < ash[tid])) {
        fsh[tid] = o;
        ash[tid] = oa;
      }
      ish[tid] |= ish[tid + w];
    }
    __syncthreads();
  }
  mx = fsh[0];
  am = ash[0];
  bad = ish[0] | (mx == -INFINITY);
  __syncthreads();
  out.m = mx;
  out.argmax = am;
  out.status = bad ? 2 : 0;
  out.tau = 0u;                                 // every non-NaN key exceeds 0
  out.tie = -1;
  out.temp = temperature;
  if (bad || temperature == 0.f) {
    if (tid == 0) rows[static_cast<size_t>(b) * R + rho] = out;
    return;
  }
  const float T = temperature;
  unsigned int tau = 0u;
  int tie = -1;

  // top-k: the top_k-th largest key, then the tie cut among equal keys
  if (top_k > 0 && top_k < V) {
    unsigned int prefix = 0u, pmask = 0u;
    int want = top_k;
    for (int shift = 24; shift >= 0; shift -= 8) {
      ish[tid] = 0;
      __syncthreads();
      for (int v = tid; v < V; v += kThreads) {
        const unsigned int key = order_key(row[v]);
        if ((key & pmask) == prefix) atomicAdd(&ish[(key >> shift) & 255u], 1);
      }
      __syncthreads();
      if (tid == 0) {
        int above = 0, d = 255;
        for (; d > 0; --d) {
          if (above + ish[d] >= want) break;
          above += ish[d];
        }
        ish[kThreads] = d | (above << 8);
      }
      __syncthreads();
      const int pick = ish[kThreads];
      __syncthreads();
      want -= pick >> 8;
      prefix |= static_cast<unsigned int>(pick & 255) << shift;
      pmask |= 255u << shift;
    }
    tie = ordered_tie(row, V, prefix, want, 0u, -1, ish);
    tau = prefix;
  }

  // top-p on the renormalised top-k row: the boundary key by 8-bit digits on
  // binary64 mass (digit bins summed with LDS atomics: their order moves a
  // sum only in its last bits), then the tied tokens it needs, then their
  // tie cut
  if (top_p < 1.f) {
    double s1 = 0.0;
    for (int v = tid; v < V; v += kThreads) {
      const float x = row[v];
      if (kept_by(order_key(x), v, tau, tie)) s1 += mass(x, mx, T);
    }
    s1 = block_sum(s1, dsh);
    const double need = static_cast<double>(top_p) * s1;
    unsigned int prefix = 0u, pmask = 0u;
    double above = 0.0;
    for (int shift = 24; shift >= 0; shift -= 8) {
      dsh[tid] = 0.0;
      __syncthreads();
      for (int v = tid; v < V; v += kThreads) {
        const float x = row[v];
        const unsigned int key = order_key(x);
        if ((key & pmask) == prefix && kept_by(key, v, tau, tie))
          atomicAdd(&dsh[(key >> shift) & 255u], mass(x, mx, T));
      }
      __syncthreads();
      if (tid == 0) {
        // highest digit whose mass brings the running sum to `need`; if
        // rounding leaves it short, the lowest digit holding any mass
        int pick = -1, last = -1;
        double run = above;
        for (int d = 255; d >= 0; --d) {
          const double md = dsh[d];
          if (md > 0.0) last = d;
          if (md > 0.0 && run + md >= need) {
            pick = d;
            break;
          }
          run += md;
        }
        if (pick < 0) {
          pick = last < 0 ? 0 : last;
          run = above;
          for (int d = 255; d > pick; --d) run += dsh[d];
        }
        ish[0] = pick;
        above_sh = run;                         // mass above the chosen digit
      }
      __syncthreads();
      const int pick = ish[0];
      above = above_sh;
      __syncthreads();
      prefix |= static_cast<unsigned int>(pick) << shift;
      pmask |= 255u << shift;
    }
    // tokens with key == prefix (all of equal mass): how many reach `need`
    const double e_tau = mass(key_value(prefix), mx, T);
    int n_tied = 0;
    for (int v = tid; v < V; v += kThreads) {
      const unsigned int key = order_key(row[v]);
      n_tied += key == prefix && kept_by(key, v, tau, tie);
    }
    n_tied = block_sum_int(n_tied, ish);
    const double jn = e_tau > 0.0 ? ceil((need - above) / e_tau) : 1.0;
    const int j = jn < 1.0 ? 1 : (jn > n_tied ? n_tied : static_cast<int>(jn));
    tie = ordered_tie(row, V, prefix, j < 1 ? 1 : j, tau, tie, ish);
    tau = prefix;
  }

  // kept mass and the kept probability of the row's draft token
  double s = 0.0;
  for (int v = tid; v < V; v += kThreads) {
    const float x = row[v];
    if (kept_by(order_key(x), v, tau, tie)) s += mass(x, mx, T);
  }
  s = block_sum(s, dsh);
  if (tid == 0) {
    out.tau = tau;
    out.tie = tie;
    out.s = s;
    double pd = 0.0;
    if (tok >= 0 && tok < V) {
      const float x = row[tok];
      pd = kept_by(order_key(x), tok, tau, tie) ? mass(x, mx, T) / s : 0.0;
    }
    out.pd = pd;
    rows[static_cast<size_t>(b) * R + rho] = out;
  }
}

// Kept probability of token v of a row described by its record (binary64).
__device__ __forceinline__ double kept_prob(const float* row, int v, const SampledRow& r) {
  const float x = row[v];
  return kept_by(order_key(x), v, r.tau, r.tie) ? mass(x, r.m, r.temp) / r.s : 0.0;
}

__global__ __launch_bounds__(kThreads) void sampled_decide_kernel(
    const float* __restrict__ tgt, const float* __restrict__ dft, const int32_t* __restrict__ toks,
    int k, int V, bool greedy, const SampledRow* __restrict__ rows, unsigned int key0,
    unsigned int key1, unsigned int offset, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ out_n_acc, int32_t* __restrict__ out_status, float* __restrict__ p_at,
    float* __restrict__ q_at) {
  __shared__ double wsh[kThreads];
  __shared__ double dsc[2];                     // threshold, running sum before the owner
  __shared__ int ish[4];
  __shared__ float u2sh;
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int R = 2 * k + 1;
  const SampledRow* rr = rows + static_cast<size_t>(b) * R;
  const int32_t* tk = toks + static_cast<size_t>(b) * k;

  // status, kept probabilities of the drafts, and the accept scan (thread 0)
  if (tid == 0) {
    int status = 0;
    for (int i = 0; i < k; ++i)
      if (tk[i] < 0 || tk[i] >= V) status = 1;
    if (status == 0) {
      // greedy settings read only the target rows
      for (int j = 0; j < (greedy ? k + 1 : R); ++j)
        if (rr[j].status != 0) status = 2;
    }
    int n_acc = k;
    float u2r = 0.f;
    for (int i = 0; i <= k; ++i) {
      unsigned int ctr[4] = {static_cast<unsigned int>(i), static_cast<unsigned int>(b), offset,
                             0u};
      sv_philox_rounds(ctr, key0, key1);
      if (i == k) {
        if (n_acc == k) u2r = sv_u24(ctr[1]);
        break;
      }
      double p = NAN, q = NAN;
      if (status == 0) {
        p = greedy ? (tk[i] == rr[i].argmax ? 1.0 : 0.0) : rr[i].pd;
        q = greedy ? 1.0 : rr[k + 1 + i].pd;
        if (n_acc == k) {
          // u carries 24 bits: exact in binary32 and binary64
          const bool acc = greedy ? p > 0.0 : static_cast<double>(sv_u24(ctr[0])) * q < p;
          if (!acc) {
            n_acc = i;
            u2r = sv_u24(ctr[1]);
          }
        }
      }
      if (p_at) p_at[static_cast<size_t>(b) * k + i] = static_cast<float>(p);
      if (q_at) q_at[static_cast<size_t>(b) * k + i] = static_cast<float>(q);
    }
    ish[0] = status;
    ish[1] = n_acc;
    ish[3] = -1;
    u2sh = u2r;
  }
  __syncthreads();
  const int status = ish[0];
  const int n_acc = ish[1];
  int32_t* ot = out_tokens + static_cast<size_t>(b) * (k + 1);
  if (status != 0) {
    for (int i = tid; i <= k; i += kThreads) ot[i] = -1;
    if (tid == 0) {
      out_n_acc[b] = -1;
      out_status[b] = status;
    }
    return;
  }
  for (int i = tid; i <= k; i += kThreads) ot[i] = i < n_acc ? tk[i] : -1;
  if (greedy) {
    if (tid == 0) {
      ot[n_acc] = rr[n_acc].argmax;
      out_n_acc[b] = n_acc;
      out_status[b] = 0;
    }
    return;
  }

  // replacement (r < k: max(0, p_r - q_r)) or bonus (r = k: p_k) draw
  const int r = n_acc;
  const float* trow = tgt + (static_cast<size_t>(b) * (k + 1) + r) * V;
  const float* drow = r < k ? dft + (static_cast<size_t>(b) * k + r) * V : trow;
  const SampledRow rt = rr[r];
  const SampledRow rd = r < k ? rr[k + 1 + r] : rt;
  const int chunk = (V + kThreads - 1) / kThreads;
  const int v0 = tid * chunk, v1 = min(V, v0 + chunk);
  auto weight = [&](int v, bool plain) {
    const double pv = kept_prob(trow, v, rt);
    return plain ? pv : fmax(0.0, pv - kept_prob(drow, v, rd));
  };
  bool plain = r == k;
  for (int pass = 0; pass < 2; ++pass) {
    double local = 0.0;
    for (int v = v0; v < v1; ++v) local += weight(v, plain);
    wsh[tid] = local;
    __syncthreads();
    if (tid == 0) {
      // S, the threshold u' S, and the chunk whose running sum crosses it
      double run = 0.0;
      for (int t = 0; t < kThreads; ++t) run += wsh[t];
      const double S = run;
      const double thr = static_cast<double>(u2sh) * S;
      int owner = -1, lastnz = -1;
      double pre = 0.0, lastnz_pre = 0.0;
      run = 0.0;
      for (int t = 0; t < kThreads; ++t) {
        const double w = wsh[t];
        if (w > 0.0) {
          lastnz = t;
          lastnz_pre = run;
        }
        if (owner < 0 && run + w > thr) {
          owner = t;
          pre = run;
        }
        run += w;
      }
      if (owner < 0) {                          // rounding left the threshold past the end
        owner = lastnz;
        pre = lastnz_pre;
      }
      ish[2] = S > 0.0 ? owner : -2;
      dsc[0] = thr;
      dsc[1] = pre;
    }
    __syncthreads();
    if (ish[2] != -2) break;
    plain = true;                               // S = 0 only through rounding: w = p_r
    __syncthreads();
  }
  if (tid == ish[2]) {
    // replay the owner's chunk with the same association as its sum
    const double thr = dsc[0], pre = dsc[1];
    double local = 0.0;
    int pick = -1, last = -1;
    for (int v = v0; v < v1; ++v) {
      const double w = weight(v, plain);
      if (w > 0.0) last = v;
      local += w;
      if (pre + local > thr) {
        pick = v;
        break;
      }
    }
    ish[3] = pick >= 0 ? pick : last;
  }
  __syncthreads();
  if (tid == 0) {
    ot[n_acc] = ish[3];
    out_n_acc[b] = n_acc;
    out_status[b] = 0;
  }
}

}  // namespace

extern "C" size_t sv_verify_sampled_workspace_bytes(int B, int k, int V) {
  if (B < 1 || k < 1 || k > SV_MAX_ROWS || V < 1) return 0;
  return static_cast<size_t>(B) * (2 * k + 1) * sizeof(SampledRow);
}

extern "C" sv_status sv_verify_sampled(const float* target_logits, const float* draft_logits,
                                       const int32_t* draft_tokens, int B, int k, int V,
                                       const sv_sampling* sampling, uint64_t seed,
                                       uint32_t offset, int32_t* out_tokens, int32_t* out_n_acc,
                                       int32_t* out_status, float* p_at, float* q_at,
                                       void* workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
  if (!target_logits || !draft_logits || !draft_tokens || !out_tokens || !out_n_acc ||
      !out_status || !sampling)
    return SV_ERR_NULL;
  if (B < 1 || k < 1 || k > SV_MAX_ROWS || V < 1) return SV_ERR_INVALID_ARG;
  if (static_cast<long long>(k + 1) * V >= (1LL << 31) || B > 65535) return SV_ERR_INVALID_ARG;
  const float T = sampling->temperature;
  if (!(T >= 0.f) || !(T < INFINITY) || sampling->top_k < 0 || !(sampling->top_p > 0.f) ||
      !(sampling->top_p <= 1.f))
    return SV_ERR_INVALID_ARG;
  if (!sv_aligned16(target_logits) || !sv_aligned16(draft_logits) ||
      !sv_aligned16(draft_tokens) || !sv_aligned16(out_tokens) || !sv_aligned16(out_n_acc) ||
      !sv_aligned16(out_status) || (p_at && !sv_aligned16(p_at)) ||
      (q_at && !sv_aligned16(q_at)))
    return SV_ERR_ALIGN;
  const size_t need = sv_verify_sampled_workspace_bytes(B, k, V);
  if (!workspace || workspace_bytes < need) return SV_ERR_WORKSPACE;
  if (!sv_aligned16(workspace)) return SV_ERR_ALIGN;
  SampledRow* rows = static_cast<SampledRow*>(workspace);
  const bool greedy = T == 0.f;
  // greedy settings need only the target rows' maxima
  hipLaunchKernelGGL(sampled_rows_kernel, dim3(greedy ? k + 1 : 2 * k + 1, B), dim3(kThreads), 0,
                     stream, target_logits, draft_logits, draft_tokens, k, V, T, sampling->top_k,
                     sampling->top_p, rows);
  SV_LAUNCH_CHECK();
  hipLaunchKernelGGL(sampled_decide_kernel, dim3(B), dim3(kThreads), 0, stream, target_logits,
                     draft_logits, draft_tokens, k, V, greedy, rows,
                     static_cast<unsigned int>(seed & 0xFFFFFFFFu),
                     static_cast<unsigned int>(seed >> 32), offset, out_tokens, out_n_acc,
                     out_status, p_at, q_at);
  SV_LAUNCH_CHECK();
  return SV_OK;
}
