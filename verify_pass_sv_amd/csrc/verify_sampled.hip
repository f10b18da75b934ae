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
// Temperature 0 (greedy verification) runs as the chain tree d_0 <- d_1 <- ..
// through the draft-tree kernels (sv_verify_tree's row maxima over many
// workgroups per row, then one wave per trial).  Other settings take three
// launches on the caller's stream (four in a large call, whose selection is
// a launch of its own).  A call with fewer rows than compute units
// first takes three more: a clear, a pass of W workgroups per row (each
// row's maximum, argmax, validity and bins or whole mass, merged in slice
// order, the boundary planned by the row's last slice) and a gather of the
// boundary tokens by the same slices:
//  1. rows    one workgroup per (trial, row), target rows 0..k then draft rows
//             0..k-1.  It checks the row and takes its maximum (and the
//             argmax, smallest index among equal maxima, into the record).
//             It describes the kept set by a key threshold and a
//             tie cut: token v is kept iff key(l_v) > tau, or key(l_v) == tau
//             and v <= tie, where key() maps binary32 order to unsigned order.
//             One pass reads the row once against a provisional reference
//             (the maximum of its first entries, raised) and bins it (1/32
//             logit): counts for top-k, binary64 masses for top-p alone,
//             the whole mass without truncation.  The top_k largest
//             tokens are sorted in LDS -- from a list the pass keeps of the
//             tokens above a bin predicted from the row's first entries, else
//             gathered by a second read -- and top-p on the renormalised
//             top-k row is resolved on their masses; top-p alone resolves its
//             boundary bin from its tokens, gathered and sorted in LDS.  A
//             boundary larger than the LDS list falls back to radix passes
//             over the whole row.  Then the kept mass S and the kept
//             probability of the row's draft token.  Masses are
//             exp((l - m) / T) in binary64 throughout.
//  2. decide  one workgroup per trial: the accept scan on the kept
//             probabilities (binary64) with the Philox uniforms of
//             sv_verify_accept; writes the outputs except the drawn token.
//  3. resid   one workgroup per (2048-entry vocabulary block, trial): block
//             totals of the residual weights max(0, p'_r - q'_r) (or p'_k for
//             the bonus), per-thread ranges of 4 entries added in order and
//             their running sums formed in one fixed association.  The last
//             workgroup of a trial to finish (a device-scope counter) selects:
//             S, the block whose running sum exceeds u' S, then the thread
//             range and the entry inside it, replaying the same sums in the
//             same order.
#include "sv_common.h"
#include "sv_philox.h"

// Greedy verification of k drafts as a chain tree (defined with the
// draft-tree kernels in verify_coupled.hip).  Arguments are validated by the
// caller.
size_t sv_greedy_chain_workspace_bytes(int B, int k, int V);
sv_status sv_greedy_chain(const float* target_logits, const int32_t* draft_tokens, int B, int k,
                          int V, int32_t* out_tokens, int32_t* out_n_acc, int32_t* out_status,
                          float* p_at, float* q_at, void* workspace, hipStream_t stream);

#include <math.h>

namespace {

constexpr int kThreads = 512;

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
// Unnormalised probability exp((x - m) / T), x <= m, in binary64, as
// 2^(y / 64) with y = 64 log2(e) (x - m) / T.  With n = rint(y), f = y - n
// (|f| <= 1/2, exact) and n = 64 i + j (0 <= j < 64):
//   2^(y / 64) = 2^i * 2^(j / 64) * e^(f ln2 / 64),
// the middle factor from a 64-entry table in LDS, the last one from its
// Taylor polynomial of degree 5 (|f ln2 / 64| <= 0.0055, remainder below
// 4e-17).  The difference of two binary32 values is exact in binary64; the
// product with the binary64 constant adds one rounding (an error of |y| 2^-53
// in y: relative 1e-14 in the mass at |x - m| / T = 50), the table entry, the
// polynomial and the product two ulps at most.  So the masses that place the
// top-p boundary and the probabilities of the accept test carry binary64
// accuracy, at about 17 vector operations and one LDS read per token.
constexpr int kExpTab = 64;
constexpr double kLog2e64 = 64.0 * 1.4426950408889634;     // 64 log2(e)
constexpr double kE1 = 0.6931471805599453 / 64.0;           // ln(2) / 64
constexpr double kE2 = kE1 * kE1 / 2.0;
constexpr double kE3 = kE2 * kE1 / 3.0;
constexpr double kE4 = kE3 * kE1 / 4.0;
constexpr double kE5 = kE4 * kE1 / 5.0;
// 2^(j / 64), j = 0..63, by threads 0..63 (a barrier before the first use).
__device__ __forceinline__ void exp_table_init(double* tab) {
  if (threadIdx.x < kExpTab) tab[threadIdx.x] = exp2(threadIdx.x * (1.0 / kExpTab));
}
struct Mass {
  const double* tab;                // 2^(j / 64) in LDS
  double m;                         // reference logit
  double c;                         // 64 log2(e) / T
  __device__ Mass(const double* t, float ref, float T)
      : tab(t), m(static_cast<double>(ref)), c(kLog2e64 / static_cast<double>(T)) {}
  __device__ __forceinline__ double operator()(float x) const {
    // clamped where the mass is below the smallest subnormal (and at x = -inf)
    const double y = fmax((static_cast<double>(x) - m) * c, -70000.0);
    const double n = rint(y);
    const double f = y - n;
    double p = fma(f, kE5, kE4);
    p = fma(f, p, kE3);
    p = fma(f, p, kE2);
    p = fma(f, p, kE1);
    p = fma(f, p, 1.0);
    const int ni = static_cast<int>(n);
    return ldexp(tab[ni & (kExpTab - 1)] * p, ni >> 6);
  }
};

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

// Binned selection: bins of 1/32 logit below the row maximum (the bin index
// is monotone in the logit), counted and massed in one pass; the boundary
// bin of a truncation is then resolved exactly from its tokens, gathered and
// sorted in LDS.
constexpr int kBins = 2048;
constexpr float kBinsPerUnit = 32.f;
constexpr int kCap = 2048;                      // tokens of one bin resolved in LDS
constexpr int kPeek = 4096;                     // entries that set a row's provisional maximum
constexpr int kPer = kBins / kThreads;          // bins (and candidate slots) per thread
static_assert(kCap / kThreads == kPer, "one range size for bins and candidates");
static_assert(kCap >= kBins, "the candidate arrays hold the fixed-point bins first");

// 0 for x >= mref (and for NaN), kBins - 1 from 64 logits below mref on
__device__ __forceinline__ int bin_of(float x, float mref) {
  const float d = (mref - x) * kBinsPerUnit;
  return static_cast<int>(fminf(fmaxf(d, 0.f), static_cast<float>(kBins - 1)));
}
// Candidate order: decreasing logit, then increasing index.
__device__ __forceinline__ unsigned long long cand_key(float x, int v) {
  return (static_cast<unsigned long long>(order_key(x)) << 32) | static_cast<unsigned int>(~v);
}

// Masses in [0, 1] summed by many threads at once (histogram bins, radix
// digits) go through 63-bit fixed point: m = (hi 2^32 + lo) 2^-63 with
// hi = floor(m 2^31) <= 2^31 and lo < 2^32, bits below 2^-63 dropped.  Chunk
// sums are integer additions, exact for up to 2^32 terms whatever their
// order, so every run (and every interleaving of the atomics) yields the same
// bin; one rounding turns a bin back into binary64.
typedef unsigned long long u64;
__device__ __forceinline__ void fx_split(double m, u64& hi, u64& lo) {
  const double t = fmin(m, 1.0) * 0x1p31;       // exact
  const double h = floor(t);
  hi = static_cast<unsigned int>(h);
  lo = static_cast<unsigned int>((t - h) * 0x1p32);   // t - h and the scaling are exact
}
__device__ __forceinline__ double fx_value(u64 hi, u64 lo) {
  // chunk sums stay below 2^53 for V < 2^21 (exact); beyond, one rounding each
  return static_cast<double>(hi) * 0x1p-31 + static_cast<double>(lo) * 0x1p-63;
}
__device__ __forceinline__ void fx_add(u64* hi, u64* lo, double m) {
  u64 h, l;
  fx_split(m, h, l);
  atomicAdd(hi, h);
  atomicAdd(lo, l);
}

// f(x, v) for the n tokens at p (v counted from p); each thread visits its
// tokens in ascending index order, with 32 values in flight when `vec` (p is
// 16-byte aligned and n a multiple of 4) allows 16-byte loads.
template <int U = 8, typename F>
__device__ __forceinline__ void scan_span(const float* p, int n, bool vec, F&& f) {
  const int tid = threadIdx.x;
  if (vec) {
    const float4* r4 = reinterpret_cast<const float4*>(p);
    const int V4 = n >> 2;
    // the ragged last round loads clamped indices (in bounds: V4 >= 1 inside
    // the loop), so its loads are in flight together, and skips them
    for (int v = tid; v < V4; v += U * kThreads) {
      float4 a[U];
#pragma unroll
      for (int u = 0; u < U; ++u) a[u] = r4[min(v + u * kThreads, V4 - 1)];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (v + u * kThreads < V4) {
          const int base = 4 * (v + u * kThreads);
          f(a[u].x, base);
          f(a[u].y, base + 1);
          f(a[u].z, base + 2);
          f(a[u].w, base + 3);
        }
      }
    }
  } else {
    for (int v = tid; v < n; v += kThreads) f(p[v], v);
  }
}
// The whole row (rows start 16-byte aligned when V is a multiple of 4).
template <int U = 8, typename F>
__device__ __forceinline__ void scan_row(const float* row, int V, F&& f) {
  scan_span<U>(row, V, (V & 3) == 0, f);
}

// Exclusive scan of one value per thread (thread order); returns this
// thread's prefix.  Lanes scan within their wave by shuffles, then each
// thread adds the totals of the waves before it, in wave order: one fixed
// association, the same on every call.
template <typename X>
__device__ X scan_excl(X c, X* sh) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  X x = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const X y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  X e = __shfl_up(x, 1, 64);                   // the lanes before this one
  if (lane == 0) e = 0;
  if (lane == 63) sh[wv] = x;
  __syncthreads();
  X base = 0;
  for (int w = 0; w < wv; ++w) base += sh[w];
  __syncthreads();
  return base + e;
}
__device__ int scan_int(int c, int* ish) { return scan_excl<int>(c, ish); }

// First bin where the count from the top reaches `want`; `above` = tokens in
// the bins before it.
__device__ int bins_cross_count(const int* hcnt, int want, int& above, int* ish) {
  const int tid = threadIdx.x;
  const int b0 = tid * kPer;
  int c = 0;
  for (int j = 0; j < kPer; ++j) c += hcnt[b0 + j];
  const int pre = scan_int(c, ish);
  if (tid == 0) ish[kThreads] = kBins;
  __syncthreads();
  if (pre < want && want <= pre + c) {
    int run = pre;
    for (int j = 0; j < kPer; ++j) {
      if (run + hcnt[b0 + j] >= want) {
        ish[kThreads] = b0 + j;
        ish[0] = run;
        break;
      }
      run += hcnt[b0 + j];
    }
  }
  __syncthreads();
  const int bn = ish[kThreads];
  above = ish[0];
  __syncthreads();
  return bn;
}

// Sum of m[0 .. n) (bins or candidates), in a fixed order.
__device__ double sum_before(const double* m, int n, double* dsh) {
  const int tid = threadIdx.x;
  double c = 0.0;
  for (int j = 0; j < kPer; ++j) {
    const int i = tid * kPer + j;
    if (i < n) c += m[i];
  }
  return block_sum(c, dsh);
}

// First index j < n (with mass > 0) where the running sum of m[0..j] reaches
// `need`; n if none.  `above` = running sum before it (or of all n).  Each
// thread replays its range after the scan, so the decision uses one
// association of the sums.
__device__ int cross_mass(const double* m, int n, double need, double& above, double* dsh,
                          int* ish) {
  const int tid = threadIdx.x;
  const int j0 = tid * kPer;
  double c = 0.0;
  for (int j = 0; j < kPer; ++j)
    if (j0 + j < n) c += m[j0 + j];
  const double pre = scan_excl<double>(c, dsh);
  if (tid == 0) ish[kThreads] = n;
  __syncthreads();
  double run = pre;
  int found = -1;
  double before = 0.0;
  for (int j = 0; j < kPer && j0 + j < n; ++j) {
    const double mj = m[j0 + j];
    if (mj > 0.0 && run + mj >= need) {
      found = j0 + j;
      before = run;
      break;
    }
    run += mj;
  }
  if (found >= 0) atomicMin(&ish[kThreads], found);
  __syncthreads();
  const int r = ish[kThreads];
  if (r < n && found == r) dsh[0] = before;
  if (r == n && tid == kThreads - 1) dsh[0] = run;   // all of them: the last running sum
  __syncthreads();
  above = dsh[0];
  __syncthreads();
  return r;
}

// Sorts cand[0 .. n) (n <= kCap) into decreasing order by a bitonic network
// over the next power of two (padding sorts last).
__device__ __noinline__ void sort_cand(unsigned long long* cand, int n) {
  const int tid = threadIdx.x;
  int npow = 1;
  while (npow < n) npow <<= 1;
  for (int j = n + tid; j < npow; j += kThreads) cand[j] = 0ull;
  __syncthreads();
  for (int size = 2; size <= npow; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int j = tid; j < npow; j += kThreads) {
        const int o = j ^ stride;
        if (o > j) {
          const unsigned long long a = cand[j], c = cand[o];
          const bool desc = (j & size) == 0;
          if (desc ? a < c : a > c) {
            cand[j] = c;
            cand[o] = a;
          }
        }
      }
      __syncthreads();
    }
  }
}

// Masses of the first n sorted candidates.
__device__ void cand_masses(const unsigned long long* cand, int n, const Mass& ms, double* cmass) {
  for (int j = threadIdx.x; j < n; j += kThreads)
    cmass[j] = ms(key_value(static_cast<unsigned int>(cand[j] >> 32)));
  __syncthreads();
}

// The tokens of bins lo..hi, sorted (decreasing logit, increasing index);
// their number, or -1 past kCap.
__device__ __noinline__ int gather_bins(const float* row, int V, float mref, int lo, int hi,
                           unsigned long long* cand, int* ish) {
  const int tid = threadIdx.x;
  if (tid == 0) ish[kThreads] = 0;
  __syncthreads();
  scan_row(row, V, [&](float x, int v) {
    const int bn = bin_of(x, mref);
    if (bn >= lo && bn <= hi) {
      const int slot = atomicAdd(&ish[kThreads], 1);
      if (slot < kCap) cand[slot] = cand_key(x, v);
    }
  });
  __syncthreads();
  const int n = ish[kThreads];
  __syncthreads();
  if (n > kCap) return -1;
  sort_cand(cand, n);
  return n;
}

// Exact selection by radix passes over the whole row, for a boundary bin that
// holds more tokens than the LDS candidate list: top-k by 8-bit digits of the
// key with integer histograms, top-p by 8-bit digits on binary64 masses.
// Updates (tau, tie).
__device__ void radix_select(const float* row, int V, const Mass& ms, int top_k, float top_p,
                             unsigned int& tau, int& tie, double* dsh, double& above_sh,
                             int* ish) {
  const int tid = threadIdx.x;
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
      if (kept_by(order_key(x), v, tau, tie)) s1 += ms(x);
    }
    s1 = block_sum(s1, dsh);
    const double need = static_cast<double>(top_p) * s1;
    unsigned int prefix = 0u, pmask = 0u;
    double above = 0.0;
    // digit masses in fixed point (dsh as 256 high then 256 low chunk sums)
    u64* const dhi = reinterpret_cast<u64*>(dsh);
    u64* const dlo = dhi + 256;
    static_assert(kThreads == 512, "dsh holds the 2 x 256 digit chunk sums");
    for (int shift = 24; shift >= 0; shift -= 8) {
      dhi[tid] = 0ull;                          // (dhi and dlo: 512 words)
      __syncthreads();
      for (int v = tid; v < V; v += kThreads) {
        const float x = row[v];
        const unsigned int key = order_key(x);
        if ((key & pmask) == prefix && kept_by(key, v, tau, tie)) {
          const unsigned int d = (key >> shift) & 255u;
          fx_add(dhi + d, dlo + d, ms(x));
        }
      }
      __syncthreads();
      if (tid == 0) {
        // highest digit whose mass brings the running sum to `need`; if
        // rounding leaves it short, the lowest digit holding any mass
        int pick = -1, last = -1;
        double run = above;
        for (int d = 255; d >= 0; --d) {
          const double md = fx_value(dhi[d], dlo[d]);
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
          for (int d = 255; d > pick; --d) run += fx_value(dhi[d], dlo[d]);
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
    const double e_tau = ms(key_value(prefix));
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

}

// Rows split into W slices (few rows per call): the pass over a row --
// maximum, argmax, validity, then the bins (or the whole mass when nothing
// truncates) against the row's provisional reference -- is taken per slice
// by W workgroups per row, and so is the gather of the boundary bins' tokens.
// Maxima and whole masses merge in slice order; each slice adds its nonzero
// bins into the row's histogram, and its gathered tokens into the row's
// candidate list, with device atomics on integers (counts, the fixed-point
// mass chunks, list slots): the histogram is exact in any order and the list
// is sorted before use.
struct SlicePart {
  float m;                          // slice maximum (-inf when empty)
  int am;                           // smallest index of it (V when empty)
  int flags;                        // 1: NaN or +inf seen, 2: a logit above the
                                    // reference, 4: no usable reference
  int pad;
};
static_assert(sizeof(SlicePart) == 16, "slice record layout");
constexpr int kMaxSlices = 16;
static_assert(kMaxSlices <= 64, "one slice record per lane");
// per row: counts (int), then the high and the low mass chunk sums (u64)
constexpr size_t kRowHistBytes = kBins * (sizeof(int) + 2 * sizeof(u64));
struct RowPlan {                    // per row, for the slices' gather and the rows launch
  float ref;                        // the row's provisional reference
  int lo, hi;                       // bins the slices gather (none when lo > hi)
  int ncand;                        // tokens gathered (past kCap: overflow)
  int ticket;                       // slices done with the pass
  float mx;                         // the merged slice records: maximum,
  int am;                           //   its smallest index,
  int flags;                        //   flags (SlicePart)
  double need;                      // top-p alone: top_p times the row's mass,
  double above;                     //   and the mass of the bins before bin lo
};
static_assert(sizeof(RowPlan) == 48, "row plan layout");

__host__ __device__ inline int slice_len(int V, int W) { return ((V + W - 1) / W + 3) & ~3; }

__device__ __forceinline__ const float* row_ptr(const float* tgt, const float* dft, int b, int rho,
                                                int k, int V) {
  return rho <= k ? tgt + (static_cast<size_t>(b) * (k + 1) + rho) * V
                  : dft + (static_cast<size_t>(b) * k + (rho - k - 1)) * V;
}

// The row's maximum, argmax and flags from its W slice records, merged in
// slice order (the same in every thread and launch).  Called by whole waves;
// the records are read at device scope (written by other workgroups of the
// same launch, when the last slice merges them).
__device__ __forceinline__ void merge_slices(const SlicePart* part, int W, float& mx, int& am,
                                             int& flags) {
  // lane w loads slice w's record (all W loads in flight at once); every
  // lane then merges the W records in order
  const int lane = threadIdx.x & 63;
  float pm = -INFINITY;
  int pa = 0x7FFFFFFF, pf = 0;
  if (lane < W) {
    const int* q = reinterpret_cast<const int*>(part + lane);
    pm = __int_as_float(__hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    pa = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    pf = __hip_atomic_load(q + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  mx = -INFINITY;
  am = 0x7FFFFFFF;
  flags = 0;
  for (int w = 0; w < W; ++w) {
    const float m = __shfl(pm, w, 64);
    const int a = __shfl(pa, w, 64);
    if (m > mx || (m == mx && a < am)) {
      mx = m;
      am = a;
    }
    flags |= __shfl(pf, w, 64);
  }
  flags |= mx == -INFINITY;
}

// The rows kernel's pass over a row (one workgroup per row) accumulates, per
// setting: the whole mass (no truncation); bin counts (top-k, with or
// without top-p: every mass that it needs comes from the gathered top
// tokens); bin masses (top-p alone); or nothing (the maximum,
// argmax and validity alone, before a second pass).  kList (top-k, once a
// bin bhat is predicted) only lists the tokens of bins <= bhat.
enum RowMode { kSum, kCount, kCountMass, kTrack, kList };

struct RowScan {                    // one thread's share of the pass
  float mx;                         // maximum seen, first at index am
  int am;
  int bad;                          // NaN or +inf seen
  int over;                         // a logit above the reference
  double sl;                        // mass (kSum)
};

struct RowLds {                     // the pass's LDS arrays
  int* hcnt;                        // bin counts
  u64* hhi;                         // bin masses, high and low fixed-point chunks
  u64* hlo;
  unsigned long long* cand;         // kCount: tokens of bins <= bhat
  int* ncand;                       //   and their number (also past kCap)
};

template <int Mode, bool Track>
__device__ __forceinline__ void row_step(float x, int v, float ref, const Mass& ms, int bhat,
                                         const RowLds& lds, RowScan& st) {
  if (Track) {
    st.bad |= !(x < INFINITY);
    st.over |= x > ref;
    if (x > st.mx) {                // each thread visits ascending indices
      st.mx = x;
      st.am = v;
    }
  }
  if (Mode == kSum) st.sl += ms(x);
  if (Mode == kCount || Mode == kCountMass) {
    const int bn = bin_of(x, ref);
    // (top-p alone needs no counts: its boundary bin's gather reports an
    // overflow of the candidate list by itself)
    if (Mode == kCount) atomicAdd(&lds.hcnt[bn], 1);
    if (Mode == kCountMass) fx_add(lds.hhi + bn, lds.hlo + bn, ms(x));
    if (Mode == kCount && bn <= bhat) {
      const int slot = atomicAdd(lds.ncand, 1);
      if (slot < kCap) lds.cand[slot] = cand_key(x, v);
    }
  }
  if (Mode == kList && bin_of(x, ref) <= bhat) {
    const int slot = atomicAdd(lds.ncand, 1);
    if (slot < kCap) lds.cand[slot] = cand_key(x, v);
  }
}

__device__ __forceinline__ void clear_bins(int Mode, const RowLds& lds) {
  for (int j = threadIdx.x; j < kBins; j += kThreads) {
    lds.hcnt[j] = 0;
    if (Mode == kCountMass) {
      lds.hhi[j] = 0ull;
      lds.hlo[j] = 0ull;
    }
  }
  if (threadIdx.x == 0) *lds.ncand = 0;
  __syncthreads();
}

// The row's first n0 = min(V, kPeek) entries, kFirst per thread in ascending
// index order (index -1 for an empty slot).
constexpr int kFirst = kPeek / kThreads;
static_assert(kFirst % 4 == 0, "whole 16-byte loads");
__device__ __forceinline__ void load_first(const float* row, int n0, bool vec, float* xs, int* vs) {
  const int tid = threadIdx.x;
  if (vec) {
    const float4* r4 = reinterpret_cast<const float4*>(row);
#pragma unroll
    for (int u = 0; u < kFirst / 4; ++u) {
      const int j = tid + u * kThreads;
      const bool in = 4 * j < n0;
      const float4 a = r4[in ? j : 0];
      xs[4 * u] = a.x;
      xs[4 * u + 1] = a.y;
      xs[4 * u + 2] = a.z;
      xs[4 * u + 3] = a.w;
#pragma unroll
      for (int c = 0; c < 4; ++c) vs[4 * u + c] = in ? 4 * j + c : -1;
    }
  } else {
#pragma unroll
    for (int u = 0; u < kFirst; ++u) {
      const int j = tid + u * kThreads;
      const bool in = j < n0;
      xs[u] = row[in ? j : 0];
      vs[u] = in ? j : -1;
    }
  }
}

// Maximum over the workgroup (binary32 maxima: exact in any order).
__device__ float block_max(float x, float* fsh) {
  const int tid = threadIdx.x;
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  if ((tid & 63) == 0) fsh[tid >> 6] = x;
  __syncthreads();
  float r = fsh[0];
  for (int w = 1; w < kThreads / 64; ++w) r = fmaxf(r, fsh[w]);
  __syncthreads();
  return r;
}

// The workgroup's maximum with its smallest index, and the OR of the flags.
__device__ void block_argmax(RowScan& st, float* fsh, int* ish) {
  const int tid = threadIdx.x;
  int flags = st.bad | (st.over << 1);
  float mx = st.mx;
  int am = st.am;
  for (int o = 32; o > 0; o >>= 1) {
    const float om = __shfl_xor(mx, o, 64);
    const int oa = __shfl_xor(am, o, 64);
    if (om > mx || (om == mx && oa < am)) {
      mx = om;
      am = oa;
    }
    flags |= __shfl_xor(flags, o, 64);
  }
  if ((tid & 63) == 0) {
    fsh[tid >> 6] = mx;
    ish[tid >> 6] = am;
    ish[kThreads / 64 + (tid >> 6)] = flags;
  }
  __syncthreads();
  mx = fsh[0];
  am = ish[0];
  flags = ish[kThreads / 64];
  for (int w = 1; w < kThreads / 64; ++w) {
    const float om = fsh[w];
    const int oa = ish[w];
    if (om > mx || (om == mx && oa < am)) {
      mx = om;
      am = oa;
    }
    flags |= ish[kThreads / 64 + w];
  }
  __syncthreads();
  st.mx = mx;
  st.am = am;
  st.bad = flags & 1;
  st.over = flags >> 1;
}

// The pass against the provisional reference ref, starting from the first
// entries held in registers.  With spec > 0 (top-k), once those entries are
// counted, bhat becomes the first bin where their count reaches spec, and
// the rest of the pass only lists every token of bins <= bhat (the counts
// then hold the first entries alone); returns bhat (-1 when nothing is
// listed, and the counts are whole).
template <int Mode>
__device__ __forceinline__ int row_pass(const float* row, int V, int n0, bool vec, const float* xs, const int* vs,
                        float ref, const Mass& ms, int spec, const RowLds& lds, RowScan& st,
                        int* ish) {
  if (Mode != kSum && Mode != kTrack) clear_bins(Mode, lds);
#pragma unroll
  for (int u = 0; u < kFirst; ++u)
    if (vs[u] >= 0) row_step<Mode, true>(xs[u], vs[u], ref, ms, -1, lds, st);
  int bhat = -1;
  if (Mode == kCount && spec > 0) {
    __syncthreads();
    int above;
    const int bh = bins_cross_count(lds.hcnt, spec, above, ish);
    if (bh < kBins) {
      bhat = bh;
#pragma unroll
      for (int u = 0; u < kFirst; ++u) {
        if (vs[u] >= 0 && bin_of(xs[u], ref) <= bhat) {
          const int slot = atomicAdd(lds.ncand, 1);
          if (slot < kCap) lds.cand[slot] = cand_key(xs[u], vs[u]);
        }
      }
    }
  }
  if (Mode == kCount && bhat >= 0)
    scan_span(row + n0, V - n0, vec, [&](float x, int v) {
      row_step<kList, true>(x, v + n0, ref, ms, bhat, lds, st);
    });
  else
    scan_span(row + n0, V - n0, vec, [&](float x, int v) {
      row_step<Mode, true>(x, v + n0, ref, ms, bhat, lds, st);
    });
  return bhat;
}

// A further pass over the whole row against the reference mx (a rare path:
// out of line, its arguments by value so that the callers' copies stay in
// registers); returns the pass's mass (kSum).
template <int Mode>
__device__ __noinline__ double row_repass(const float* row, int V, float mx, Mass ms,
                                          RowLds lds) {
  if (Mode != kSum) clear_bins(Mode, lds);
  RowScan st = {-INFINITY, V, 0, 0, 0.0};
  scan_row(row, V, [&](float x, int v) { row_step<Mode, false>(x, v, mx, ms, -1, lds, st); });
  return st.sl;
}

// grid (rows): clears what the slices add into -- the row's counts (and for
// top-p alone its mass chunks), its candidate count and its ticket.
__global__ __launch_bounds__(kThreads) void sampled_clear_kernel(char* __restrict__ hist,
                                                                 RowPlan* __restrict__ plans,
                                                                 int chunks) {
  const size_t rid = blockIdx.x;
  uint4* h = reinterpret_cast<uint4*>(hist + rid * kRowHistBytes);
  const int n16 = static_cast<int>((chunks ? kRowHistBytes : kBins * sizeof(int)) / 16);
  for (int j = threadIdx.x; j < n16; j += kThreads) h[j] = make_uint4(0u, 0u, 0u, 0u);
  if (threadIdx.x == 0) {
    plans[rid].ncand = 0;
    plans[rid].ticket = 0;
  }
}

// A slice's first kChunk entries are loaded (16-byte rows) together with the
// row's first entries, before the reference is known; the rest of a longer
// slice is scanned after them.
constexpr int kChunk4 = 8 * kThreads;           // float4 loads per chunk (16384 entries)
template <int Mode>
__device__ __forceinline__ void slice_scan(const float* row, int v0, int n, bool vec,
                                           const float4* pre, int c4, float ref, const Mass& ms,
                                           const RowLds& lds, RowScan& st) {
  if (Mode == kCount || Mode == kCountMass) clear_bins(Mode, lds);
  int done = 0;
  if (vec) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = threadIdx.x + u * kThreads;
      if (j < c4) {
        const int v = v0 + 4 * j;
        row_step<Mode, true>(pre[u].x, v, ref, ms, -1, lds, st);
        row_step<Mode, true>(pre[u].y, v + 1, ref, ms, -1, lds, st);
        row_step<Mode, true>(pre[u].z, v + 2, ref, ms, -1, lds, st);
        row_step<Mode, true>(pre[u].w, v + 3, ref, ms, -1, lds, st);
      }
    }
    done = 4 * c4;
  }
  scan_span(row + v0 + done, n - done, vec, [&](float x, int v) {
    row_step<Mode, true>(x, v0 + done + v, ref, ms, -1, lds, st);
  });
}

// grid (W, 2k+1, B): one slice's pass against the row's provisional
// reference (every slice derives the same one from the row's first
// entries); the last slice of a row to finish merges the slice records and
// plans the gather of the boundary bins.
__global__ __launch_bounds__(kThreads) void sampled_slice_pass_kernel(
    const float* __restrict__ tgt, const float* __restrict__ dft, int k, int V, int W, float T,
    int top_k, float top_p, SlicePart* __restrict__ parts, double* __restrict__ slice_s,
    char* __restrict__ hist, RowPlan* __restrict__ plans) {
  __shared__ int hcnt[kBins];
  __shared__ u64 hhi[kBins], hlo[kBins];
  __shared__ double dsh[kThreads];
  __shared__ double etab[kExpTab];
  __shared__ float fsh[kThreads / 64];
  __shared__ int ish[kThreads + 1];
  __shared__ int nc;
  const int tid = threadIdx.x;
  const int w = blockIdx.x, rho = blockIdx.y, b = blockIdx.z;
  const size_t rid = static_cast<size_t>(b) * gridDim.y + rho;
  const float* row = row_ptr(tgt, dft, b, rho, k, V);
  exp_table_init(etab);
  const bool vec = (V & 3) == 0;
  const int L = slice_len(V, W);
  const int v0 = w * L;
  const int n = v0 < V ? min(L, V - v0) : 0;
  float4 pre[8];
  const int c4 = vec ? min(n >> 2, kChunk4) : 0;
  if (c4 > 0) {
    const float4* r4 = reinterpret_cast<const float4*>(row + v0);
#pragma unroll
    for (int u = 0; u < 8; ++u) pre[u] = r4[min(static_cast<int>(threadIdx.x) + u * kThreads, c4 - 1)];
  }
  const int n0 = min(V, kPeek);
  float xs[kFirst];
  int vs[kFirst];
  load_first(row, n0, vec, xs, vs);
  float m0 = -INFINITY;
#pragma unroll
  for (int u = 0; u < kFirst; ++u)
    if (vs[u] >= 0) m0 = fmaxf(m0, xs[u]);
  m0 = block_max(m0, fsh);                      // (its barrier also orders the table)
  const bool fused = m0 > -INFINITY && m0 < INFINITY;
  const float ref = fused ? m0 + fminf(4.f, 8.f * T) : INFINITY;
  const bool trunc_k = top_k > 0 && top_k < V;
  const bool trunc = trunc_k || top_p < 1.f;
  const int mode = !fused ? kTrack : !trunc ? kSum : trunc_k ? kCount : kCountMass;
  const Mass ms(etab, ref, T);
  const RowLds lds = {hcnt, hhi, hlo, nullptr, &nc};
  RowScan st = {-INFINITY, V, 0, 0, 0.0};
  if (mode == kTrack)
    slice_scan<kTrack>(row, v0, n, vec, pre, c4, ref, ms, lds, st);
  else if (mode == kSum)
    slice_scan<kSum>(row, v0, n, vec, pre, c4, ref, ms, lds, st);
  else if (mode == kCount)
    slice_scan<kCount>(row, v0, n, vec, pre, c4, ref, ms, lds, st);
  else
    slice_scan<kCountMass>(row, v0, n, vec, pre, c4, ref, ms, lds, st);
  const double sl = st.sl;
  block_argmax(st, fsh, ish);                   // (its barriers also close the bins)
  if (mode == kSum) {
    const double s = block_sum(sl, dsh);
    if (tid == 0) slice_s[rid * W + w] = s;
  }
  char* h = hist + rid * kRowHistBytes;
  int* gc = reinterpret_cast<int*>(h);
  u64* ghi = reinterpret_cast<u64*>(h + kBins * sizeof(int));
  u64* glo = ghi + kBins;
  if (mode == kCount || mode == kCountMass) {
    for (int j = tid; j < kBins; j += kThreads) {
      if (mode == kCount) {
        const int c = hcnt[j];
        if (c != 0) atomicAdd(&gc[j], c);
      } else {
        const u64 hj = hhi[j], lj = hlo[j];
        if (hj != 0ull) atomicAdd(&ghi[j], hj);
        if (lj != 0ull) atomicAdd(&glo[j], lj);
      }
    }
  }
  if (tid == 0) {
    int* q = reinterpret_cast<int*>(parts + rid * W + w);
    __hip_atomic_store(q, __float_as_int(st.mx), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q + 1, st.am, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q + 2, st.bad | (st.over << 1) | (fused ? 0 : 4), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  // The last slice of the row to finish (device-scope ticket).  Everything
  // the other slices read -- the records and the bins -- goes through
  // device-scope stores, atomics and loads, which bypass the compute units'
  // non-coherent caches; every wave waits for its own to complete, then the
  // barrier, then the ticket is counted.  (No cache-wide fence: written back
  // and invalidated by every workgroup, it costs more than the pass.)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) ish[0] = atomicAdd(&plans[rid].ticket, 1);
  __syncthreads();
  if (ish[0] != W - 1) return;
  float mx;
  int am, rf;
  merge_slices(parts + rid * W, W, mx, am, rf);
  int lo = 1, hi = 0;
  double need = 0.0, above = 0.0;
  if (rf == 0 && (mode == kCount || mode == kCountMass)) {
    double* hmass = reinterpret_cast<double*>(hhi);
    for (int j = tid; j < kBins; j += kThreads) {
      hcnt[j] = __hip_atomic_load(gc + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (mode == kCountMass)
        hmass[j] = fx_value(__hip_atomic_load(ghi + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                            __hip_atomic_load(glo + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    }
    __syncthreads();
    if (mode == kCount) {
      int above = 0;
      const int bk = bins_cross_count(hcnt, top_k, above, ish);
      if (bk < kBins && above + hcnt[bk] <= kCap) {
        lo = 0;
        hi = bk;
      }
    } else {
      need = static_cast<double>(top_p) * sum_before(hmass, kBins, dsh);
      const int bp = cross_mass(hmass, kBins, need, above, dsh, ish);
      if (bp < kBins) {                         // (an overflowing gather shows in ncand)
        lo = bp;
        hi = bp;
      }
    }
  }
  if (tid == 0) {
    RowPlan* pl = plans + rid;
    pl->ref = ref;
    pl->lo = lo;
    pl->hi = hi;
    pl->mx = mx;
    pl->am = am;
    pl->flags = rf;
    pl->need = need;
    pl->above = above;
  }
}

// grid (W, 2k+1, B): the tokens of the planned bins in one slice, added to
// the row's candidate list (one reservation of list slots per slice).
__global__ __launch_bounds__(kThreads) void sampled_slice_gather_kernel(
    const float* __restrict__ tgt, const float* __restrict__ dft, int k, int V, int W,
    RowPlan* __restrict__ plans, unsigned long long* __restrict__ gcand) {
  __shared__ unsigned long long lc[kCap];
  __shared__ int ln, base;
  const int tid = threadIdx.x;
  const int w = blockIdx.x, rho = blockIdx.y, b = blockIdx.z;
  const size_t rid = static_cast<size_t>(b) * gridDim.y + rho;
  const int lo = plans[rid].lo, hi = plans[rid].hi;
  if (lo > hi) return;
  const float ref = plans[rid].ref;
  const float* row = row_ptr(tgt, dft, b, rho, k, V);
  const int L = slice_len(V, W);
  const int v0 = w * L;
  const int n = v0 < V ? min(L, V - v0) : 0;
  if (tid == 0) ln = 0;
  __syncthreads();
  scan_span(row + v0, n, (V & 3) == 0, [&](float x, int v) {
    const int bn = bin_of(x, ref);
    if (bn >= lo && bn <= hi) {
      const int slot = atomicAdd(&ln, 1);
      if (slot < kCap) lc[slot] = cand_key(x, v0 + v);
    }
  });
  __syncthreads();
  const int m = ln;
  if (tid == 0) base = m > 0 ? atomicAdd(&plans[rid].ncand, m) : 0;
  __syncthreads();
  const int b0 = base;
  if (m <= kCap)
    for (int j = tid; j < m && b0 + j < kCap; j += kThreads) gcand[rid * kCap + b0 + j] = lc[j];
}

// One instantiation per pass mode (the setting decides it): kSum without
// truncation, kCount for top-k (with or without top-p), kCountMass for top-p
// alone; each holds only its own code, registers and LDS.
template <int Mode>
__global__ __launch_bounds__(kThreads, Mode == kCountMass ? 4 : 6) void sampled_rows_kernel(
    const float* __restrict__ tgt, const float* __restrict__ dft, const int32_t* __restrict__ toks,
    int k, int V, float temperature, int top_k, float top_p, int W,
    const double* __restrict__ slice_s, const RowPlan* __restrict__ plans,
    const unsigned long long* __restrict__ gcand, SampledRow* __restrict__ rows) {
  static_assert(Mode == kSum || Mode == kCount || Mode == kCountMass, "pass mode");
  constexpr int kB = Mode == kSum ? 1 : kBins;
  constexpr int kC = Mode == kSum ? 1 : kCap;
  __shared__ double dsh[kThreads];
  __shared__ double above_sh;
  __shared__ int ish[kThreads + 1];
  __shared__ int hcnt[kB];
  __shared__ unsigned long long cand[kC];
  __shared__ double cmass[kC];
  __shared__ double etab[kExpTab];
  __shared__ float fsh[kThreads / 64];
  __shared__ int ncand;
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
  exp_table_init(etab);

  const size_t rid = static_cast<size_t>(b) * R + rho;
  const float T = temperature;
  constexpr int mode = Mode;
  constexpr bool trunc_k = Mode == kCount;      // top_k in (0, V)
  constexpr bool trunc = Mode != kSum;
  const bool trunc_p = top_p < 1.f;
  // (during the pass the fixed-point bins live in the candidate arrays)
  const RowLds lds = {hcnt, reinterpret_cast<u64*>(cand), reinterpret_cast<u64*>(cmass), cand,
                      &ncand};
  float mx = -INFINITY;
  int am = V;
  int bad = 0;
  // Masses exp((l - mref) / T) are taken against a reference mref >= every
  // logit of the row; the kept probabilities, ratios of such masses, do not
  // depend on which.  With one workgroup per row, mref is the maximum of the
  // row's first kPeek entries raised by min(4, 8 T), and the maximum, the
  // validity, and the counts (or masses) come out of one pass; should a
  // logit exceed mref after all, mref becomes the row maximum and the
  // accumulation takes a second pass.  (The fixed-point bin masses resolve
  // 2^-63 of mref's scale, at most e^8 of the maximum's.)  For top-k, the
  // counts of those first entries also predict a bin bhat that holds about
  // 3 top_k tokens of the row, and the pass lists the tokens down to it, so
  // that the boundary needs no second read when the prediction holds.
  float mref = -INFINITY;
  double sl = 0.0;
  int bhat = -1;
  bool local = true;                            // the bins (or mass) are this workgroup's
  bool redo = false;                            // a pass against the row maximum
  if (W > 1) {
    const int rf = plans[rid].flags;
    mx = plans[rid].mx;
    am = plans[rid].am;
    bad = rf & 1;
    // a logit above the slices' reference (or none usable): this
    // workgroup's own pass
    redo = !bad && (rf & 6);
    if (!redo) {
      mref = plans[rid].ref;
      local = false;
    }
    __syncthreads();                            // (the table)
  } else {
    const bool vec = (V & 3) == 0;
    const int n0 = min(V, kPeek);
    float xs[kFirst];
    int vs[kFirst];
    load_first(row, n0, vec, xs, vs);
    float m0 = -INFINITY;
#pragma unroll
    for (int u = 0; u < kFirst; ++u)
      if (vs[u] >= 0) m0 = fmaxf(m0, xs[u]);
    m0 = block_max(m0, fsh);                    // (its barrier also orders the table)
    const bool fused = m0 > -INFINITY && m0 < INFINITY;
    const float ref = fused ? m0 + fminf(4.f, 8.f * T) : INFINITY;
    const Mass ms(etab, ref, T);
    // top-k: the first entries' count that predicts about 3 top_k tokens
    int spec = 0;
    if (trunc_k && V > n0 && 6 * top_k <= kCap)
      spec = static_cast<int>((3ll * top_k * n0 + V - 1) / V) + 1;
    RowScan st = {-INFINITY, V, 0, 0, 0.0};
    if (!fused)
      row_pass<kTrack>(row, V, n0, vec, xs, vs, ref, ms, 0, lds, st, ish);
    else if (mode == kSum)
      row_pass<kSum>(row, V, n0, vec, xs, vs, ref, ms, 0, lds, st, ish);
    else if (mode == kCount)
      bhat = row_pass<kCount>(row, V, n0, vec, xs, vs, ref, ms, spec, lds, st, ish);
    else
      row_pass<kCountMass>(row, V, n0, vec, xs, vs, ref, ms, 0, lds, st, ish);
    const double sl1 = st.sl;
    block_argmax(st, fsh, ish);
    mx = st.mx;
    am = st.am;
    bad = st.bad | (mx == -INFINITY);
    redo = !bad && (!fused || st.over);
    if (!redo) {
      mref = ref;
      sl = sl1;
    }
  }
  if (redo) {
    mref = mx;
    bhat = -1;
    const Mass ms2(etab, mx, T);
    if (mode == kSum)
      sl = row_repass<kSum>(row, V, mx, ms2, lds);
    else if (mode == kCount)
      row_repass<kCount>(row, V, mx, ms2, lds);
    else
      row_repass<kCountMass>(row, V, mx, ms2, lds);
  }
  __syncthreads();
  out.m = mref;
  out.argmax = am;
  out.status = bad ? 2 : 0;
  out.tau = 0u;                                 // every non-NaN key exceeds 0
  out.tie = -1;
  out.temp = temperature;
  if (bad) {
    if (tid == 0) rows[static_cast<size_t>(b) * R + rho] = out;
    return;
  }
  const Mass ms(etab, mref, T);
  unsigned int tau = 0u;
  int tie = -1;

  double s = 0.0;                               // kept mass
  if (!trunc) {
    if (!local) {
      for (int w = 0; w < W; ++w) s += slice_s[rid * W + w];
    } else {
      s = block_sum(sl, dsh);
    }
  } else {
    // the top tokens, sorted (decreasing logit, increasing index): for top-k
    // every token of the bins down to the one where the count reaches top_k
    // (bin bk); for top-p alone the tokens of the bin where the mass reaches
    // need = top_p S (bin bp), after `above` in the bins before it
    int n = -1, bk = kBins, bp = kBins;
    double need = 0.0, above = 0.0;
    if (!local) {
      // W > 1: the slices' plan and gathered list
      const RowPlan& pl = plans[rid];
      if (pl.lo <= pl.hi && pl.ncand <= kCap) {
        n = pl.ncand;
        for (int j = tid; j < n; j += kThreads) cand[j] = gcand[rid * kCap + j];
        sort_cand(cand, n);
        bk = pl.hi;
        bp = pl.lo;
        need = pl.need;
        above = pl.above;
      }
    } else if (trunc_k) {
      // from the list the pass made when it holds top_k tokens or more (all
      // of those in bins <= bhat, so the top_k largest of the row), else
      // counted by a second read and gathered by a third (bins down to bk)
      if (bhat >= 0 && ncand >= top_k && ncand <= kCap) {
        n = ncand;
        sort_cand(cand, n);
      } else {
        if (bhat >= 0) {
          row_repass<kCount>(row, V, mref, ms, lds);
          __syncthreads();
        }
        int cnt_above = 0;
        bk = bins_cross_count(hcnt, top_k, cnt_above, ish);
        if (bk < kBins && cnt_above + hcnt[bk] <= kCap)
          n = gather_bins(row, V, mref, 0, bk, cand, ish);
      }
    } else {
      // binary64 bin masses in place of the high chunks (each thread its own
      // bins; the candidates overwrite them once the boundary bin is known)
      double* const hmass = reinterpret_cast<double*>(lds.hhi);
      for (int j = tid; j < kBins; j += kThreads) hmass[j] = fx_value(lds.hhi[j], lds.hlo[j]);
      __syncthreads();
      need = static_cast<double>(top_p) * sum_before(hmass, kBins, dsh);
      bp = cross_mass(hmass, kBins, need, above, dsh, ish);
      if (bp < kBins) n = gather_bins(row, V, mref, bp, bp, cand, ish);
    }
    bool exact = false;
    if (trunc_k) {
      exact = n >= top_k;
      if (exact) {
        cand_masses(cand, top_k, ms, cmass);
        int r = top_k;                          // tokens kept
        if (trunc_p) {
          // top-p on the renormalised top-k row
          const double need_k = static_cast<double>(top_p) * sum_before(cmass, top_k, dsh);
          double before = 0.0;
          const int j = cross_mass(cmass, top_k, need_k, before, dsh, ish);
          r = j < top_k ? j + 1 : top_k;
        }
        tau = static_cast<unsigned int>(cand[r - 1] >> 32);
        tie = static_cast<int>(~static_cast<unsigned int>(cand[r - 1]));
        s = sum_before(cmass, r, dsh);
      }
    } else {
      exact = n > 0;
      if (exact) {
        cand_masses(cand, n, ms, cmass);
        double before = 0.0;
        const int j = cross_mass(cmass, n, need - above, before, dsh, ish);
        const int r = j < n ? j + 1 : n;        // tokens kept from the boundary bin
        tau = static_cast<unsigned int>(cand[r - 1] >> 32);
        tie = static_cast<int>(~static_cast<unsigned int>(cand[r - 1]));
        s = above + sum_before(cmass, r, dsh);
      }
    }
    if (!exact) {
      tau = 0u;
      tie = -1;
      radix_select(row, V, ms, top_k, top_p, tau, tie, dsh, above_sh, ish);
      s = 0.0;
      scan_row(row, V, [&](float x, int v) {
        if (kept_by(order_key(x), v, tau, tie)) s += ms(x);
      });
      s = block_sum(s, dsh);
    }
  }

  // the kept probability of the row's draft token
  if (tid == 0) {
    out.tau = tau;
    out.tie = tie;
    out.s = s;
    double pd = 0.0;
    if (tok >= 0 && tok < V) {
      const float x = row[tok];
      pd = kept_by(order_key(x), tok, tau, tie) ? ms(x) / s : 0.0;
    }
    out.pd = pd;
    rows[static_cast<size_t>(b) * R + rho] = out;
  }
}

struct SampledDecision {             // per trial, written by launch 2
  int status;
  int n_acc;
  int plain;                        // draw from p_r alone (bonus position)
  int pad;
  double u2;                        // the uniform of the replacement / bonus draw
};

constexpr int kResPer = 4;                      // residual weights per thread per block
constexpr int kResBlk = kThreads * kResPer;     // 2048 vocabulary entries per block
__host__ __device__ inline int res_blocks(int V) { return (V + kResBlk - 1) / kResBlk; }

__global__ __launch_bounds__(kThreads) void sampled_decide_kernel(
    const int32_t* __restrict__ toks, int k, int V, const SampledRow* __restrict__ rows, unsigned int key0, unsigned int key1,
    unsigned int offset, SampledDecision* __restrict__ decs, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ out_n_acc, int32_t* __restrict__ out_status, float* __restrict__ p_at,
    float* __restrict__ q_at, int* __restrict__ done) {
  __shared__ int ish[2];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  if (tid == 0) done[b] = 0;                    // launch 3's completion counter
  const int R = 2 * k + 1;
  const SampledRow* rr = rows + static_cast<size_t>(b) * R;
  const int32_t* tk = toks + static_cast<size_t>(b) * k;

  // status, kept probabilities of the drafts and the accept scan: wave 0,
  // lane i for draft i (its Philox uniforms, p'_i(d_i), q'_i(d_i)); the first
  // rejection is the first set bit of one ballot
  if (tid < 64) {
    const int i = tid;
    const bool tbad = i < k && (tk[i] < 0 || tk[i] >= V);
    const bool rbad = (i < R && rr[i].status != 0) || (i + 64 < R && rr[i + 64].status != 0);
    const int status = __any(tbad) ? 1 : (__any(rbad) ? 2 : 0);
    float u = 0.f, u2 = 0.f;
    if (i <= k) {
      unsigned int ctr[4] = {static_cast<unsigned int>(i), static_cast<unsigned int>(b), offset,
                             0u};
      sv_philox_rounds(ctr, key0, key1);
      u = sv_u24(ctr[0]);
      u2 = sv_u24(ctr[1]);
    }
    double p = NAN, q = NAN;
    bool acc = true;
    if (i < k && status == 0) {
      p = rr[i].pd;
      q = rr[k + 1 + i].pd;
      // u carries 24 bits: exact in binary32 and binary64
      acc = static_cast<double>(u) * q < p;
    }
    const unsigned long long rej = __ballot(!acc);
    const int n_acc = rej ? (__ffsll(static_cast<long long>(rej)) - 1) : k;
    const float u2r = __shfl(u2, n_acc);
    if (i < k) {
      if (p_at) p_at[static_cast<size_t>(b) * k + i] = static_cast<float>(p);
      if (q_at) q_at[static_cast<size_t>(b) * k + i] = static_cast<float>(q);
    }
    if (i == 0) {
      SampledDecision dec;
      dec.status = status;
      dec.n_acc = status == 0 ? n_acc : -1;
      dec.plain = n_acc == k;
      dec.pad = 0;
      dec.u2 = static_cast<double>(u2r);
      decs[b] = dec;
      ish[0] = status;
      ish[1] = n_acc;
    }
  }
  __syncthreads();
  const int status = ish[0];
  const int n_acc = ish[1];
  int32_t* ot = out_tokens + static_cast<size_t>(b) * (k + 1);
  for (int i = tid; i <= k; i += kThreads) ot[i] = status == 0 && i < n_acc ? tk[i] : -1;
  if (tid == 0) {
    out_n_acc[b] = status == 0 ? n_acc : -1;
    out_status[b] = status;
  }
}

// The residual weights of trial b (plain: p_r alone) over one thread's 16
// entries of vocabulary block blk, summed in ascending order.
struct ResidualRows {
  const float* trow;
  const float* drow;
  Mass tmass, dmass;                // exp((l - m) / T) against each row's reference
  unsigned int ttau, dtau;
  int ttie, dtie;
  double ts, ds;
};
// The weight of entry v from its target logit x and draft logit y.
__device__ __forceinline__ double res_weight(const ResidualRows& q, float x, float y, int v,
                                             bool plain) {
  const double pv = kept_by(order_key(x), v, q.ttau, q.ttie) ? q.tmass(x) / q.ts : 0.0;
  if (plain) return pv;
  const double qv = kept_by(order_key(y), v, q.dtau, q.dtie) ? q.dmass(y) / q.ds : 0.0;
  return fmax(0.0, pv - qv);
}

// A thread's kResPer target and draft logits of block blk, all loads issued
// before any is used (entries past V read as 0 and are never weighed).
__device__ __forceinline__ void res_load(const ResidualRows& q, int V, int blk, bool plain,
                                         float* xs, float* ys) {
  const int v0 = blk * kResBlk + threadIdx.x * kResPer;
#pragma unroll
  for (int j = 0; j < kResPer; ++j) {
    const bool in = v0 + j < V;
    xs[j] = in ? q.trow[v0 + j] : 0.f;
    ys[j] = in && !plain ? q.drow[v0 + j] : 0.f;
  }
}
__device__ __forceinline__ ResidualRows residual_rows(const float* tgt, const float* dft,
                                                      const SampledRow* rows, int b, int k,
                                                      int V, int r, const double* etab) {
  const SampledRow* rr = rows + static_cast<size_t>(b) * (2 * k + 1);
  const SampledRow* rt = rr + r;
  const SampledRow* rd = r < k ? rr + k + 1 + r : rt;
  ResidualRows q = {tgt + (static_cast<size_t>(b) * (k + 1) + r) * V,
                    r < k ? dft + (static_cast<size_t>(b) * k + r) * V
                          : tgt + (static_cast<size_t>(b) * (k + 1) + r) * V,
                    Mass(etab, rt->m, rt->temp),
                    Mass(etab, rd->m, rt->temp),
                    rt->tau, rd->tau, rt->tie, rd->tie, rt->s, rd->s};
  return q;
}
__device__ __forceinline__ double thread_res_sum(const ResidualRows& q, int V, int blk, bool plain) {
  const int v0 = blk * kResBlk + threadIdx.x * kResPer;
  float xs[kResPer], ys[kResPer];
  res_load(q, V, blk, plain, xs, ys);
  double s = 0.0;
#pragma unroll
  for (int j = 0; j < kResPer; ++j)
    if (v0 + j < V) s += res_weight(q, xs[j], ys[j], v0 + j, plain);
  return s;
}

// Inclusive running sums of a[0 .. kThreads) in place (binary64, every thread
// of the workgroup takes part): the same fixed association on every call, so
// the block total that launch 3 forms (a[kThreads - 1]) is bit-identical to
// the one launch 4 reaches when it forms the same sums again.
__device__ void scan_inclusive(double* a) {
  const int tid = threadIdx.x;
  for (int off = 1; off < kThreads; off <<= 1) {
    const double v = tid >= off ? a[tid - off] : 0.0;
    __syncthreads();
    a[tid] += v;
    __syncthreads();
  }
}

// The selection of trial b, run by the last workgroup of launch 3 to finish
// it: S = sum of the block totals; the block whose running sum first exceeds
// u' S; inside it, the thread whose running sum does; that thread replays
// its entries with the same association.  The running sums of the block
// totals are formed by wave 0, lane l adding a contiguous range after the
// exclusive sum of the ranges before it (one fixed association); the totals
// are read with device-scope loads (written by other workgroups).
__device__ void select_token(const float* __restrict__ tgt, const float* __restrict__ dft, int k,
                             int V, const SampledRow* __restrict__ rows,
                             const SampledDecision& dec, double* __restrict__ totals,
                             int G, int b, const double* etab, double* wsh, double* lsh,
                             int32_t* __restrict__ out_tokens) {
  __shared__ double run_sh, thr_sh;
  __shared__ int ish[3];
  const int tid = threadIdx.x;
  double* const tot = totals + static_cast<size_t>(b) * 2 * G;
  // both rows of totals (residual, then p_r alone), 2 G doubles: into LDS
  // when they fit (lsh holds kThreads), else worked on in place after an
  // agent-scope acquire (a vocabulary past 2^19 entries)
  double* tsh = lsh;
  if (2 * G <= kThreads) {
    const unsigned long long* t64 = reinterpret_cast<const unsigned long long*>(tot);
    for (int i = tid; i < 2 * G; i += kThreads)
      tsh[i] = __longlong_as_double(static_cast<long long>(
          __hip_atomic_load(t64 + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)));
  } else {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    tsh = tot;
  }
  __syncthreads();
  if (tid < 64) {
    // running sums of row `which`, in place; S the last one
    auto run_sums = [&](int which) {
      double* t = tsh + which * G;
      const int per = (G + 63) / 64;
      const int i0 = min(G, tid * per), i1 = min(G, i0 + per);
      double c = 0.0;
      for (int i = i0; i < i1; ++i) c += t[i];
      double incl = c;
      for (int o = 1; o < 64; o <<= 1) {
        const double y = __shfl_up(incl, o, 64);
        if (tid >= o) incl += y;
      }
      double run = __shfl_up(incl, 1, 64);
      if (tid == 0) run = 0.0;
      for (int i = i0; i < i1; ++i) {
        run += t[i];
        t[i] = run;
      }
      return __shfl(incl, 63, 64);
    };
    int which = 0;
    double S = run_sums(0);
    if (!(S > 0.0)) {                           // only through rounding: w = p_r
      which = 1;
      S = run_sums(1);
    }
    const double thr = dec.u2 * S;
    // the first block whose running sum exceeds thr (wave ballots over 64
    // blocks at a time); none (rounding left thr at the end): the last block
    // with weight
    const double* t = tsh + which * G;
    int blk = -1;
    for (int c0 = 0; c0 < G; c0 += 64) {
      const int i = c0 + tid;
      const unsigned long long hit = __ballot(i < G && t[i] > thr);
      if (hit) {
        blk = c0 + __ffsll(static_cast<long long>(hit)) - 1;
        break;
      }
    }
    if (blk < 0) {
      int lastnz = -1;
      for (int c0 = 0; c0 < G; c0 += 64) {
        const int i = c0 + tid;
        const bool nz = i < G && (i == 0 ? t[0] > 0.0 : t[i] > t[i - 1]);
        const unsigned long long m = __ballot(nz);
        if (m) lastnz = c0 + 63 - __clzll(static_cast<long long>(m));
      }
      blk = lastnz < 0 ? 0 : lastnz;
    }
    if (tid == 0) {
      ish[0] = blk;
      ish[1] = which;
      run_sh = blk > 0 ? t[blk - 1] : 0.0;
      thr_sh = thr;
    }
  }
  __syncthreads();
  const int blk = ish[0];
  const bool plain = dec.plain != 0 || ish[1] == 1;
  const ResidualRows q = residual_rows(tgt, dft, rows, b, k, V, dec.n_acc, etab);
  const double mine = thread_res_sum(q, V, blk, plain);
  wsh[tid] = mine;
  __syncthreads();
  // the running sums of the thread sums as the block total was formed; the
  // owner is the first thread whose running sum crosses the threshold (they
  // never decrease); rounding that leaves none: the last thread with weight
  scan_inclusive(wsh);
  if (tid == 0) {
    ish[2] = kThreads;
    ish[0] = -1;
  }
  __syncthreads();
  {
    const double run = run_sh, thr = thr_sh;
    const double before = tid > 0 ? wsh[tid - 1] : 0.0;
    if (run + wsh[tid] > thr && !(run + before > thr)) atomicMin(&ish[2], tid);
    if (mine > 0.0) atomicMax(&ish[0], tid);
  }
  __syncthreads();
  if (tid == 0) {
    int owner = ish[2];
    if (owner == kThreads) owner = ish[0];
    ish[2] = owner;
    run_sh = run_sh + (owner > 0 ? wsh[owner - 1] : 0.0);
  }
  __syncthreads();
  if (tid == ish[2]) {
    const int v0 = blk * kResBlk + tid * kResPer;
    const double thr = thr_sh, pre = run_sh;
    float xs[kResPer], ys[kResPer];
    res_load(q, V, blk, plain, xs, ys);
    double local = 0.0;
    int pick = -1, last = -1;
    for (int j = 0; j < kResPer && v0 + j < V; ++j) {
      const double w = res_weight(q, xs[j], ys[j], v0 + j, plain);
      if (w > 0.0) last = v0 + j;
      local += w;
      if (pre + local > thr) {
        pick = v0 + j;
        break;
      }
    }
    out_tokens[static_cast<size_t>(b) * (k + 1) + dec.n_acc] = pick >= 0 ? pick : last;
  }
}

// Launch 3: block totals of the residual weights (and of p_r alone, for the
// S = 0 fallback): the last of the per-thread sums' running sums, stored at
// device scope.  In a small call (fold) the last workgroup of the trial to
// finish (a device-scope counter, zeroed by launch 2) selects the token:
// every wave waits for its own stores to complete before the barrier and the
// count.  In a large one a fourth launch selects (the waits would hold every
// workgroup's slot).
__global__ __launch_bounds__(kThreads) void sampled_resid_kernel(
    const float* __restrict__ tgt, const float* __restrict__ dft, int k, int V,
    const SampledRow* __restrict__ rows, const SampledDecision* __restrict__ decs,
    double* __restrict__ totals, int fold, int* __restrict__ done,
    int32_t* __restrict__ out_tokens) {
  __shared__ double wsh[2][kThreads];
  __shared__ double etab[kExpTab];
  __shared__ int last;
  const int tid = threadIdx.x;
  const int blk = blockIdx.x;
  const int b = blockIdx.y;
  const int G = gridDim.x;
  const SampledDecision dec = decs[b];
  if (dec.status != 0) return;
  exp_table_init(etab);
  __syncthreads();
  const ResidualRows q = residual_rows(tgt, dft, rows, b, k, V, dec.n_acc, etab);
  wsh[0][tid] = thread_res_sum(q, V, blk, dec.plain != 0);
  wsh[1][tid] = dec.plain ? 0.0 : thread_res_sum(q, V, blk, true);
  __syncthreads();
  scan_inclusive(wsh[0]);
  scan_inclusive(wsh[1]);
  if (tid < 2)
    __hip_atomic_store(reinterpret_cast<unsigned long long*>(
                           totals + (static_cast<size_t>(b) * 2 + tid) * G + blk),
                       static_cast<unsigned long long>(__double_as_longlong(wsh[tid][kThreads - 1])),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (!fold) return;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) last = atomicAdd(&done[b], 1) == G - 1;
  __syncthreads();
  if (!last) return;
  // (the totals of the trial go to wsh[1] when they fit; the thread sums of
  // the chosen block to wsh[0])
  select_token(tgt, dft, k, V, rows, dec, totals, G, b, etab, wsh[0], wsh[1], out_tokens);
}

// Launch 4 of a large call: one workgroup per trial selects the token.
__global__ __launch_bounds__(kThreads) void sampled_select_kernel(
    const float* __restrict__ tgt, const float* __restrict__ dft, int k, int V,
    const SampledRow* __restrict__ rows, const SampledDecision* __restrict__ decs,
    double* __restrict__ totals, int G, int32_t* __restrict__ out_tokens) {
  __shared__ double wsh[2][kThreads];
  __shared__ double etab[kExpTab];
  const int b = blockIdx.x;
  const SampledDecision dec = decs[b];
  if (dec.status != 0) return;
  exp_table_init(etab);
  __syncthreads();
  select_token(tgt, dft, k, V, rows, dec, totals, G, b, etab, wsh[0], wsh[1], out_tokens);
}

}  // namespace

namespace {
// Slices per row: enough workgroups to cover the chip when a call has fewer
// rows than compute units and rows are long; else one workgroup per row.
// (Two slice workgroups fit a compute unit -- their registers -- so 512 fill
// one round of the chip; measured: 768, two rounds, took 4-7 us more at
// B = 1; slices of 2048 tokens at least.)
int row_slices(int B, int k, int V) {
  const long long rows = static_cast<long long>(B) * (2 * k + 1);
  if (rows >= 256 || V < 16384) return 1;
  long long w = 512 / rows;
  if (w > kMaxSlices) w = kMaxSlices;
  if (w > V / 2048) w = V / 2048;
  return static_cast<int>(w);
}
size_t align256(size_t x) { return (x + 255) / 256 * 256; }
struct SampledWs {
  size_t rows_off, dec_off, tot_off, done_off, part_off, ss_off, hist_off, plan_off, cand_off,
      bytes;
  int W;
};
SampledWs sampled_ws(int B, int k, int V) {
  SampledWs w;
  const size_t nrow = static_cast<size_t>(B) * (2 * k + 1);
  w.W = row_slices(B, k, V);
  w.rows_off = 0;
  w.dec_off = align256(nrow * sizeof(SampledRow));
  w.tot_off = align256(w.dec_off + static_cast<size_t>(B) * sizeof(SampledDecision));
  w.done_off = align256(w.tot_off + static_cast<size_t>(B) * 2 * res_blocks(V) * sizeof(double));
  w.bytes = w.done_off + static_cast<size_t>(B) * sizeof(int);
  w.part_off = w.ss_off = w.hist_off = w.plan_off = w.cand_off = 0;
  if (w.W > 1) {
    w.part_off = align256(w.bytes);
    w.ss_off = align256(w.part_off + nrow * w.W * sizeof(SlicePart));
    w.hist_off = align256(w.ss_off + nrow * w.W * sizeof(double));
    w.plan_off = align256(w.hist_off + nrow * kRowHistBytes);
    w.cand_off = align256(w.plan_off + nrow * sizeof(RowPlan));
    w.bytes = w.cand_off + nrow * kCap * sizeof(unsigned long long);
  }
  // temperature 0 runs as a chain tree, whose span partials share the space
  const size_t chain = sv_greedy_chain_workspace_bytes(B, k, V);
  if (chain > w.bytes) w.bytes = chain;
  return w;
}
}  // namespace

extern "C" size_t sv_verify_sampled_workspace_bytes(int B, int k, int V) {
  if (B < 1 || k < 1 || k > SV_MAX_ROWS || V < 1) return 0;
  return sampled_ws(B, k, V).bytes;
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
  const SampledWs L = sampled_ws(B, k, V);
  char* ws = static_cast<char*>(workspace);
  SampledRow* rows = reinterpret_cast<SampledRow*>(ws + L.rows_off);
  SampledDecision* decs = reinterpret_cast<SampledDecision*>(ws + L.dec_off);
  double* totals = reinterpret_cast<double*>(ws + L.tot_off);
  int* done = reinterpret_cast<int*>(ws + L.done_off);
  const int G = res_blocks(V);
  // Greedy verification (T = 0) is the chain tree d_0 <- d_1 <- .. of the
  // draft-tree kernels: row maxima over many workgroups per row, then one
  // wave per trial.
  if (T == 0.f)
    return sv_greedy_chain(target_logits, draft_tokens, B, k, V, out_tokens, out_n_acc,
                           out_status, p_at, q_at, workspace, stream);
  SlicePart* parts = reinterpret_cast<SlicePart*>(ws + L.part_off);
  double* slice_s = reinterpret_cast<double*>(ws + L.ss_off);
  char* hist = ws + L.hist_off;
  RowPlan* plans = reinterpret_cast<RowPlan*>(ws + L.plan_off);
  unsigned long long* gcand = reinterpret_cast<unsigned long long*>(ws + L.cand_off);
  if (L.W > 1) {
    // mass chunks only for top-p alone
    const int chunks = !(sampling->top_k > 0 && sampling->top_k < V) && sampling->top_p < 1.f;
    hipLaunchKernelGGL(sampled_clear_kernel, dim3(B * (2 * k + 1)), dim3(kThreads), 0, stream,
                       hist, plans, chunks);
    SV_LAUNCH_CHECK();
    hipLaunchKernelGGL(sampled_slice_pass_kernel, dim3(L.W, 2 * k + 1, B), dim3(kThreads), 0,
                       stream, target_logits, draft_logits, k, V, L.W, T, sampling->top_k,
                       sampling->top_p, parts, slice_s, hist, plans);
    SV_LAUNCH_CHECK();
    if (chunks || (sampling->top_k > 0 && sampling->top_k < V)) {
      hipLaunchKernelGGL(sampled_slice_gather_kernel, dim3(L.W, 2 * k + 1, B), dim3(kThreads),
                         0, stream, target_logits, draft_logits, k, V, L.W, plans, gcand);
      SV_LAUNCH_CHECK();
    }
  }
  {
    const bool tk = sampling->top_k > 0 && sampling->top_k < V;
    const bool tp = sampling->top_p < 1.f;
    auto rows_kernel = tk ? sampled_rows_kernel<kCount>
                          : tp ? sampled_rows_kernel<kCountMass> : sampled_rows_kernel<kSum>;
    hipLaunchKernelGGL(rows_kernel, dim3(2 * k + 1, B), dim3(kThreads), 0, stream,
                       target_logits, draft_logits, draft_tokens, k, V, T, sampling->top_k,
                       sampling->top_p, L.W, slice_s, plans, gcand, rows);
  }
  SV_LAUNCH_CHECK();
  hipLaunchKernelGGL(sampled_decide_kernel, dim3(B), dim3(kThreads), 0, stream, draft_tokens, k,
                     V, rows, static_cast<unsigned int>(seed & 0xFFFFFFFFu),
                     static_cast<unsigned int>(seed >> 32), offset, decs, out_tokens, out_n_acc,
                     out_status, p_at, q_at, done);
  SV_LAUNCH_CHECK();
  // (small calls select in launch 3's last workgroup per trial; measured:
  // B = 1 3 us faster, B = 64 0.25 us per trial slower than a fourth launch)
  const int fold = static_cast<long long>(B) * G <= 2048;
  hipLaunchKernelGGL(sampled_resid_kernel, dim3(G, B), dim3(kThreads), 0, stream, target_logits,
                     draft_logits, k, V, rows, decs, totals, fold, done, out_tokens);
  SV_LAUNCH_CHECK();
  if (!fold) {
    hipLaunchKernelGGL(sampled_select_kernel, dim3(B), dim3(kThreads), 0, stream, target_logits,
                       draft_logits, k, V, rows, decs, totals, G, out_tokens);
    SV_LAUNCH_CHECK();
  }
  return SV_OK;
}
