/*
 * libspecverify -- the data-parallel hot path of speculative-decoding
 * verification on AMD Instinct MI355X (gfx950).
 *
 * The target model scores a block of k draft tokens in one pass, streaming
 * its quantized weights from HBM once for all k rows; a left-to-right
 * accept/correct step then keeps a prefix of the drafts and samples one more
 * token.  Sources (cited by page title and section):
 *   - "Speculative Decoding Clearly Explained": "Check the guesses together",
 *     "Accept from left to right", "Correct and continue".
 *   - "Karpathy's Trick for Faster Local LLMs Finally Has Proper Tooling":
 *     "Why batch-one decoding is memory-bound", "How Uzu optimizes bytes and
 *     tokens per pass", "Producing several tokens from one model pass".
 *   - "Local LLM 4x Faster -- Not Through Hardware, but Through Speculative
 *     Decoding" (int8 matrix path, random Hadamard transform).
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller; the
 *     library never allocates or frees memory.  Tensors are contiguous and
 *     row-major; every pointer must be 16-byte aligned.
 *   - Arguments are validated synchronously, before any launch; a bad
 *     argument returns SV_ERR_* and nothing is enqueued.
 *   - Work is enqueued asynchronously on `stream` (NULL = the default
 *     stream).  A failed launch returns SV_ERR_HIP.
 *   - Calls are thread-safe.  The only process-wide state is the registry of
 *     plan ids (sv_pass_run), guarded by a mutex.  Calls that share an
 *     output or workspace buffer on one device must be ordered by the caller.
 *   - bf16 = bfloat16 (upper half of an IEEE binary32), f16 = IEEE binary16,
 *     passed as `const void*`.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SV_OK = 0,
  SV_ERR_NULL = 1,          /* a required pointer is NULL                      */
  SV_ERR_INVALID_ARG = 2,   /* a size or parameter is out of range             */
  SV_ERR_ALIGN = 3,         /* a pointer is not 16-byte aligned                */
  SV_ERR_UNSUPPORTED = 4,   /* valid in principle, not implemented (e.g. group)*/
  SV_ERR_WORKSPACE = 5,     /* workspace missing or too small                  */
  SV_ERR_HIP = 6            /* the HIP runtime reported an error at launch     */
} sv_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* sv_status_str(sv_status status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int sv_version(void);

/* Maximum number of draft rows / draft tokens per call (the pages' 16-32
 * token budgets: @trymirai timeline; Karpathy's Trick ..., "Producing several
 * tokens from one model pass"). */
#define SV_MAX_ROWS 32

/*
 * sv_qgemm_w4 -- verify GEMM over 4-bit asymmetric group-quantized weights.
 *
 * Defines (Karpathy's Trick ..., "How Uzu optimizes bytes and tokens per
 * pass": the Medium checkpoint uses 4-bit asymmetric integer quantization
 * where every value of a group shares one scale; Speculative Decoding Clearly
 * Explained, "Check the guesses together": all draft positions are scored in
 * one pass):
 *
 *   Y[r, n] = sum_k X[r, k] * (C[n, k] - Z[n, k/group]) * S[n, k/group],
 *   r < m, n < N, k < K.
 *
 *   x       bf16 [m, K]        activations, one row per draft position
 *   m       1 .. SV_MAX_ROWS
 *   K       input features; K % 64 == 0
 *   codes   uint8 [N, K/2]     byte j of row n: code of k = 2j in the low
 *                              nibble, k = 2j + 1 in the high nibble
 *   scales  f16 [N, K/group]   per-group scale S
 *   zeros   f16 [N, K/group]   per-group zero point Z (any f16 value; the
 *                              dequantized weight is exact in binary32 when
 *                              Z is integer-valued)
 *   N       output features; N % 16 == 0
 *   group   must be 64 (SV_ERR_UNSUPPORTED otherwise)
 *   y       f32 [m, N]         output, fully overwritten
 *
 * Every weight byte is read from HBM once for all m rows.  Accumulation is
 * binary32; the result is deterministic (bitwise identical across runs).
 */
sv_status sv_qgemm_w4(const void* x, int m, int K,
                      const uint8_t* codes, const void* scales, const void* zeros,
                      int N, int group, float* y, hipStream_t stream);

/*
 * Packed W4 layout -- the checkpoint layout the fast verify GEMM streams.
 *
 * The pages describe a checkpoint format designed together with the kernels
 * (Karpathy's Trick ..., "How Uzu optimizes bytes and tokens per pass";
 * @trymirai timeline).  sv_w4_pack rewrites row-major W4 weights (the
 * sv_qgemm_w4 format) once into a tile-major layout whose every 1 KiB block
 * is one wave load in MFMA operand order.  With ntile = N/16, KB = K/128 and
 * block(t, j) = 32*g*KB + j*gt + (t % 32), where g = t / 32 and
 * gt = min(32, ntile - 32*g) (tiles grouped by 32; inside a group the blocks
 * of one k block are consecutive):
 *   packed_codes uint8, N*K/2 bytes: for 16-row tile t and 128-wide k block j,
 *     the block at byte block(t, j)*1024 holds, at bytes [16l, 16l+16),
 *     row 16t + (l & 15) with q = l >> 4: its codes for k = 128j + 16q + [0,16)
 *     (bytes 0-7) and k = 128j + 64 + 16q + [0,16) (bytes 8-15); inside each
 *     4-byte word covering k0..k0+7, byte b holds code k0+b in its low nibble
 *     and code k0+b+4 in its high nibble.
 *   packed_sz f16, N*(K/group)*4 bytes: for (t, j) a 128-byte record at
 *     block(t, j)*128; row n of the tile owns 8 bytes
 *     [S(2j), Z(2j), S(2j+1), Z(2j+1)].
 * Requirements: group == 64, N % 16 == 0, K % 128 == 0, N*K/2 < 2^31.  The
 * pack enqueues
 * two kernels on `stream`; the caller owns both output buffers (sizes from
 * sv_w4_packed_codes_bytes / sv_w4_packed_sz_bytes).
 */
size_t sv_w4_packed_codes_bytes(int N, int K);
size_t sv_w4_packed_sz_bytes(int N, int K, int group);
sv_status sv_w4_pack(const uint8_t* codes, const void* scales, const void* zeros,
                     int N, int K, int group, uint8_t* packed_codes, void* packed_sz,
                     hipStream_t stream);

/*
 * sv_qgemm_w4_packed -- the same product as sv_qgemm_w4,
 *   Y[r, n] = sum_k X[r, k] * (C[n, k] - Z[n, k/64]) * S[n, k/64],
 * over weights in the packed layout above: x bf16 [m, K] (m in
 * 1..SV_MAX_ROWS), y f32 [m, N] fully overwritten; N % 16 == 0,
 * K % 128 == 0, group == 64.  Every weight byte is read from HBM once for
 * all m rows; results are deterministic and, for integer zero points and a
 * one-hot activation row, exactly (C - Z) * S in binary32.
 */
sv_status sv_qgemm_w4_packed(const void* x, int m, int K, const uint8_t* packed_codes,
                             const void* packed_sz, int N, int group, float* y,
                             hipStream_t stream);

/*
 * sv_w8_pack -- rewrites row-major W8 codes (int8 [N, K]) into the streaming
 * layout of the pass executor: for 16-row tile t and 64-wide k block j, one
 * 1 KiB block at byte block(t, j) * 1024 (block() as for sv_w4_pack, with
 * KB = K/64) whose bytes [16l, 16l+16) hold row 16t + (l & 15),
 * k = 64j + 16 (l >> 4) + [0, 16) in natural order.
 * packed_codes: N*K bytes, 16-byte aligned; N % 16 == 0, K % 64 == 0.
 * The per-channel scales stay as they are (f16 [N]).
 */
sv_status sv_w8_pack(const int8_t* codes, int N, int K, uint8_t* packed_codes,
                     hipStream_t stream);

/*
 * Verify-pass executor: every GEMM of one verify pass in ONE launch.
 *
 * A pass reads every weight of the stack once for all m draft rows (Karpathy's
 * Trick ..., "Why batch-one decoding is memory-bound": the pass time is the
 * weight bytes divided by bandwidth; Speculative Decoding Clearly Explained,
 * "Check the guesses together").  Launching each GEMM separately stops the
 * HBM stream at every GEMM boundary; the executor streams all of them back to
 * back from one persistent kernel.  Formats (Karpathy's Trick ..., "How Uzu
 * optimizes bytes and tokens per pass"; Local LLM 4x Faster, int8 path):
 *
 *   SV_PASS_W4     Y = X W^T, X bf16, W 4-bit asymmetric group 64 (the
 *                  product of sv_qgemm_w4)
 *   SV_PASS_W8     Y = X W^T, X bf16, W 8-bit symmetric per channel (the
 *                  product of sv_qgemm_w8)
 *   SV_PASS_W4_I8  Y[r, n] = xscale[r] sum_g S (I - Z Xg), X int8 with
 *                  per-row scales, W 4-bit (the product of sv_qgemm_w4_i8)
 *
 * sv_pass_gemm describes one product (all pointers device, 16-byte aligned):
 *   x        bf16 [m, K] (W4, W8) or int8 [m, K] (W4_I8)
 *   xscale   f32 [m] row scales for W4_I8; NULL otherwise
 *   codes    sv_w4_pack codes (W4, W4_I8) or sv_w8_pack codes (W8) of W [N, K]
 *   scales   sv_w4_pack scales/zeros (W4, W4_I8) or f16 [N] scales (W8)
 *   y        f32 [m, N], fully overwritten
 *   K, N     N % 16 == 0; K % 128 == 0 (W4, W4_I8) or K % 64 == 0 (W8);
 *            codes, m*K activation bytes and m*N*4 below 2^31 bytes
 *   stats    NULL, or f32 pairs [m, G, 2] with G = ceil(N / 64), fully
 *            overwritten: stats[r, g] = (M, S), M = max of y[r, n] and
 *            S = sum of exp(y[r, n] - M) over n in [64g, min(64g + 64, N))
 *            (binary32, hardware exp2; S = 0 when M = -inf; S = NaN when
 *            one of those y is NaN or +inf).  The online-softmax epilogue
 *            of a vocabulary projection: sv_verify_accept_stats merges these
 *            pairs instead of reading the logits back (Speculative Decoding
 *            Clearly Explained, "Check the guesses together" and "Accept
 *            from left to right").
 * The GEMMs of one pass are independent: no y may overlap another GEMM's
 * inputs or outputs (their order inside the launch is unspecified).
 *
 * sv_pass_plan_bytes(format, gemms, count, m): bytes of the device plan
 *   buffer, 0 if an argument is invalid.
 * sv_pass_plan(format, gemms, count, m, group, plan, plan_bytes, pass, stream):
 *   validates every descriptor (SV_ERR_NULL / _INVALID_ARG / _ALIGN /
 *   _UNSUPPORTED; group must be 64 for the 4-bit formats; SV_ERR_WORKSPACE if
 *   plan_bytes is too small), splits the GEMMs into work items of 512 output
 *   channels, assigns them to one workgroup per compute unit of the current
 *   device, writes the plan into `plan` (caller-owned device memory) and fills
 *   the host struct *pass.  A setup call: it copies the plan with `stream` and
 *   synchronizes that stream before returning.  The plan stores the
 *   descriptors' pointers; it stays valid while those buffers and `plan`
 *   live, for any number of launches.
 * sv_pass_run(pass, stream): enqueues the whole pass as one kernel launch on
 *   `stream` (capturable in a HIP graph).  It returns SV_ERR_INVALID_ARG,
 *   enqueuing nothing, when the plan buffer has been planned again since
 *   *pass was filled (the library keeps, per plan buffer, the id of the last
 *   plan written into it: process-wide state behind a mutex).  A kernel that
 *   finds in the buffer a plan other than *pass describes (the caller
 *   overwrote the buffer) computes nothing; a chain kernel also sets the
 *   status word below.
 * Results are deterministic; they equal the single-GEMM entry points' up to
 * the order of the binary32 accumulation over K (the int32 group partials of
 * W4_I8 are exact).
 */
typedef enum { SV_PASS_W4 = 0, SV_PASS_W8 = 1, SV_PASS_W4_I8 = 2 } sv_pass_format;

typedef struct sv_pass_gemm {
  const void* x;
  const float* xscale;
  const uint8_t* codes;
  const void* scales;
  float* y;
  int K;
  int N;
  float* stats;     /* optional (NULL: none): softmax statistics of y       */
} sv_pass_gemm;

typedef struct sv_pass {
  void* plan;       /* device plan buffer given to sv_pass_plan   */
  int format;       /* sv_pass_format                             */
  int m;            /* draft rows of every GEMM in the pass       */
  int count;        /* number of GEMMs (links of a chain)         */
  int grid;         /* workgroups of the launch                   */
  int items;        /* work items (rounds of a chain)             */
  int max_steps;    /* longest per-workgroup chunk count          */
  int stats;        /* 1 if some GEMM writes softmax statistics   */
  int chain;        /* 1: planned by sv_pass_chain_plan           */
  uint32_t id;      /* this plan's id in its buffer (see below)   */
} sv_pass;

size_t sv_pass_plan_bytes(int format, const sv_pass_gemm* gemms, int count, int m);
sv_status sv_pass_plan(int format, const sv_pass_gemm* gemms, int count, int m, int group,
                       void* plan, size_t plan_bytes, sv_pass* pass, hipStream_t stream);
sv_status sv_pass_run(const sv_pass* pass, hipStream_t stream);

/*
 * Plan status word.  The chain kernel of sv_pass_run writes it, in the plan
 * buffer, when it cannot run the plan:
 *   SV_PASS_STATUS_STALE    the buffer holds a chain plan other than the one
 *                           *pass describes (format, m or grid differ);
 *                           nothing was computed
 *   SV_PASS_STATUS_TIMEOUT  a phase barrier of a chain waited longer than
 *                           its bound (workgroups not resident together);
 *                           the launch ended early, outputs are undefined,
 *                           and the plan must be made again
 * A buffer that holds no plan at all (its first word is not a plan's
 * magic number) is not written.  sv_pass_status reads the word (its place in
 * the plan buffer is internal; synchronizes `stream`); sv_pass_plan and
 * sv_pass_chain_plan clear it.  The unordered executor never sets it (its
 * stale plans are refused by sv_pass_run).
 */
#define SV_PASS_STATUS_STALE 1u
#define SV_PASS_STATUS_TIMEOUT 2u
#define SV_PASS_STATUS_OFFSET 36   /* status word of an sv_pass_plan plan */
sv_status sv_pass_status(const sv_pass* pass, uint32_t* status, hipStream_t stream);

/*
 * Verify pass in model order: sv_pass_chain_plan / sv_pass_run.
 *
 * One forward pass hands each layer's output to the next layer (Karpathy's
 * Trick ..., "How Uzu optimizes bytes and tokens per pass": the activations
 * are the intermediate values passed between layers; "Why batch-one decoding
 * is memory-bound": the pass reads every layer's weight blocks once).  A
 * chain is an ordered array of links, each one W4 or W8 GEMM
 *   y = x W^T                         (y f32 [m, N], fully overwritten)
 * that may also write the bf16 input of a later link
 *   xo = bf16_rne(alpha * y[:, :xo_cols])     (xo bf16 [m, xo_cols]).
 * A link whose x IS an earlier link's xo (same pointer, K == xo_cols) starts
 * only after every earlier link is complete on the whole device; other links
 * follow without waiting.  The launch is one persistent kernel of one
 * workgroup per compute unit; every link is spread over all of them, and
 * the weights of later links stream while a link waits.  Every workgroup
 * must be resident at once: run a chain alone on its device (a barrier that
 * waits past its bound sets SV_PASS_STATUS_TIMEOUT).
 *
 * sv_pass_link (all pointers device):
 *   x        bf16 [m, K], 16-byte aligned
 *   codes    sv_w4_pack codes of W [N, K];  scales: sv_w4_pack scales/zeros
 *   y        f32 [m, N]
 *   xo       NULL (xo_cols == 0) or bf16 [m, xo_cols], 128-byte aligned
 *   alpha    scale applied before the bf16 rounding of xo
 *   K, N     K % 128 == 0, N % 16 == 0; xo_cols % 64 == 0, xo_cols <= N
 * Buffer rules (SV_ERR_INVALID_ARG otherwise): an x that overlaps an earlier
 * link's xo is exactly that xo; no xo overlaps the x of its own or an
 * earlier link, or another xo; no y overlaps any x, xo or other y.  Later
 * links may read only xo, never y, of earlier links.
 * Formats: SV_PASS_W4 (codes and scale/zero records from sv_w4_pack; group
 * 64) and SV_PASS_W8 (codes from sv_w8_pack, `scales` the f16 [N] channel
 * scales); SV_PASS_W4_I8 returns SV_ERR_UNSUPPORTED.
 * sv_pass_chain_bytes: plan buffer bytes (0 if an argument is invalid); the
 * plan buffer must be 256-byte aligned.  sv_pass_chain_plan validates,
 * writes the plan (its barrier counters included) with `stream`,
 * synchronizes, and fills *pass; the plan stays valid for any number of
 * sv_pass_run launches on that stream order.  Results are deterministic:
 * each y equals the single-GEMM product up to the order of the binary32
 * accumulation over K, and xo is the binary32 product alpha * y rounded to
 * nearest even in bf16.
 */
typedef struct sv_pass_link {
  const void* x;
  const uint8_t* codes;
  const void* scales;
  float* y;
  void* xo;
  float alpha;
  int K;
  int N;
  int xo_cols;
} sv_pass_link;

size_t sv_pass_chain_bytes(int format, const sv_pass_link* links, int count, int m);
/* The plan image sv_pass_chain_plan would upload, built on the host for a
 * device of `cus` compute units into caller-owned HOST memory `image`
 * (image_bytes >= the size sv_pass_chain_bytes reports for such a device);
 * *grid receives the workgroup count.  Touches no device: for inspecting
 * and testing the plan (its layout is internal to this library).  Same
 * validation and status codes as sv_pass_chain_plan. */
sv_status sv_pass_chain_image(int format, const sv_pass_link* links, int count, int m, int group,
                              int cus, void* image, size_t image_bytes, int* grid);
sv_status sv_pass_chain_plan(int format, const sv_pass_link* links, int count, int m, int group,
                             void* plan, size_t plan_bytes, sv_pass* pass, hipStream_t stream);

/*
 * sv_qgemm_w8 -- verify GEMM over 8-bit symmetric per-output-channel weights.
 *
 * Defines (Karpathy's Trick ..., "How Uzu optimizes bytes and tokens per
 * pass": the Large checkpoint uses 8-bit symmetric quantization):
 *
 *   Y[r, n] = S[n] * sum_k X[r, k] * C[n, k]
 *
 *   x       bf16 [m, K], m in 1 .. SV_MAX_ROWS, K % 64 == 0
 *   codes   int8 [N, K], values in [-127, 127] (-128 is rejected by nothing
 *           but is outside the format; it dequantizes as -128 * S)
 *   scales  f16 [N]
 *   N % 16 == 0;  y f32 [m, N], fully overwritten.
 *
 * Every weight byte is read from HBM once for all m rows; binary32
 * accumulation; deterministic.  SV_ERR_INVALID_ARG for m or K out of range
 * or N % 16 != 0; SV_ERR_ALIGN for pointers not 16-byte aligned;
 * SV_ERR_UNSUPPORTED for N * K >= 2^31 (a matrix of 2 GiB or more).
 */
sv_status sv_qgemm_w8(const void* x, int m, int K, const int8_t* codes,
                      const void* scales, int N, float* y, hipStream_t stream);

/*
 * sv_hadamard_i8 -- randomized block-diagonal Hadamard rotation of the
 * activations followed by per-token symmetric int8 quantization.
 *
 * Defines (Karpathy's Trick ..., "How Uzu optimizes bytes and tokens per
 * pass": random sign flips, then mixing by a +-1 Hadamard matrix with one
 * overall scale, each block mixed on its own, exactly reversible; activations
 * quantized to 8 bits on the fly so both GEMM operands are integers):
 *
 *   xt[r, b*B + i] = B^-1/2 * sum_j H_B[i, j] * signs[b*B + j] * x[r, b*B + j]
 *   xscale[r] = max_k |xt[r, k]| / 127   (1 if the row is all zero)
 *   xq[r, k]  = clamp(round_half_even(xt[r, k] / xscale[r]), -127, 127)
 *
 * with H_B the Sylvester Hadamard matrix, H[i, j] = (-1)^popcount(i & j).
 * The rotation is summed in binary64 and rounded once to binary32; the scale
 * and the rounding decision are binary32.
 *
 *   x       bf16 [m, K], m in 1 .. 2^20 (rows are independent tokens; a
 *           verify pass may batch all its activation rows in one call)
 *   signs   int8 [K], each +1 or -1 (other values are used as given)
 *   block   power of two, 2 <= block <= 4096, block divides K
 *   K       K % 64 == 0, K <= 16384
 *   xq      int8 [m, K]  output
 *   xscale  f32 [m]      output
 */
sv_status sv_hadamard_i8(const void* x, int m, int K, const int8_t* signs, int block,
                         int8_t* xq, float* xscale, hipStream_t stream);

/*
 * sv_qgemm_w4_i8 -- the int8 matrix path: int8 activations times 4-bit
 * weights with exact int32 per-group partials.
 *
 * Defines (Local LLM 4x Faster: the 4-bit checkpoint runs on the GPU's int8
 * matrix path; Karpathy's Trick ..., "How Uzu optimizes bytes and tokens per
 * pass"):
 *
 *   I[r, n, g]  = sum_{k in g} C[n, k] * xq[r, k]          (exact int32)
 *   Xg[r, g]    = sum_{k in g} xq[r, k]                    (exact int32)
 *   Y[r, n]     = xscale[r] * sum_g S[n, g] * (I[r, n, g] - Z[n, g] * Xg[r, g])
 *
 *   xq      int8 [m, K], xscale f32 [m] (typically from sv_hadamard_i8)
 *   codes, scales, zeros, N, group: as sv_qgemm_w4
 *   y       f32 [m, N], fully overwritten.
 */
sv_status sv_qgemm_w4_i8(const int8_t* xq, const float* xscale, int m, int K,
                         const uint8_t* codes, const void* scales, const void* zeros,
                         int N, int group, float* y, hipStream_t stream);

/*
 * sv_verify_accept -- fused vocabulary softmax for target and draft, the
 * left-to-right accept scan, and the residual / bonus resample.
 *
 * Defines (Speculative Decoding Clearly Explained, "Accept from left to
 * right" and "Correct and continue"; Karpathy's Trick ..., "Producing several
 * tokens from one model pass"), per independent trial b:
 *
 *   p_i = softmax(target[b, i, :]),  q_i = softmax(draft[b, i, :])
 *   (temperature 1; a logit of -inf is probability 0)
 *   For i = 0, 1, ..: accept draft d_i iff u_i * q_i(d_i) < p_i(d_i); stop at
 *   the first rejection.  n_acc = number accepted (0..k).
 *   r = n_acc.  If r < k: w_v = max(0, p_r(v) - q_r(v)); else w_v = p_k(v)
 *   (the bonus token after all drafts).  S = sum_v w_v (if S == 0, w = p_r).
 *   The new token is the smallest v whose running sum, in ascending vocab
 *   order, exceeds u'_r * S.
 *   out_tokens[b, 0..n_acc-1] = d_0..d_{n_acc-1}; out_tokens[b, n_acc] = new
 *   token; entries after it are -1.  Tokens emitted = n_acc + 1.
 *
 * Random numbers: Philox4x32-10 (Salmon et al., SC'11) with key =
 * (seed & 0xffffffff, seed >> 32) and counter = (i, b, offset, 0); output
 * word 0 gives u_i, word 1 gives u'_i, each as (word >> 8) * 2^-24.
 *
 *   target_logits  f32 [B, k+1, V]  (row k scores the bonus position)
 *   draft_logits   f32 [B, k, V]
 *   draft_tokens   int32 [B, k]
 *   B >= 1, 1 <= k <= SV_MAX_ROWS, V >= 1, (k+1)*V < 2^31
 *   out_tokens     int32 [B, k+1]
 *   out_n_acc      int32 [B]    (-1 when out_status[b] != 0)
 *   out_status     int32 [B]    0 ok; 1 a draft token outside [0, V);
 *                               2 a row holds NaN or +inf or no finite logit
 *   p_at, q_at     f32 [B, k]   optional (NULL to skip): p_i(d_i), q_i(d_i)
 *   lse            f32 [B, 2k+1] optional: log-sum-exp of target rows 0..k,
 *                               then draft rows 0..k-1
 *   workspace      device scratch of at least
 *                  sv_verify_accept_workspace_bytes(B, k, V) bytes; contents
 *                  need no initialization and are clobbered.
 *
 * Device-data problems are reported through out_status, never raised.
 */
size_t sv_verify_accept_workspace_bytes(int B, int k, int V);
sv_status sv_verify_accept(const float* target_logits, const float* draft_logits,
                           const int32_t* draft_tokens, int B, int k, int V,
                           uint64_t seed, uint32_t offset,
                           int32_t* out_tokens, int32_t* out_n_acc, int32_t* out_status,
                           float* p_at, float* q_at, float* lse,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * sv_verify_accept_noalloc -- sv_verify_accept for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): no workspace argument and no allocation
 * of any kind.  Its workspace is a fixed array of SV_ACCEPT_SCRATCH_BYTES
 * (2 MiB) per device, held by the library until the process ends; the
 * device's address of it is looked up once per device, on the first call
 * made with that device current.
 *
 * Arguments, outputs, results and errors as sv_verify_accept, except:
 *   SV_ERR_WORKSPACE  sv_verify_accept_workspace_bytes(B, k, V) exceeds
 *                     SV_ACCEPT_SCRATCH_BYTES (e.g. B = 64, k = 32 and
 *                     V = 262144 fit; B = 256, k = 32, V = 152000 does not);
 *                     nothing is enqueued
 *   SV_ERR_HIP        the array's device address could not be looked up
 * Every call on one device shares that device's array: calls that overlap on
 * one device (other streams, other host threads) race and must be ordered by
 * the caller.  The array keeps the last call's contents; nothing in it needs
 * to start at zero.
 */
#define SV_ACCEPT_SCRATCH_BYTES (2u << 20)
size_t sv_verify_accept_noalloc_max_bytes(void);
sv_status sv_verify_accept_noalloc(const float* target_logits, const float* draft_logits,
                                   const int32_t* draft_tokens, int B, int k, int V,
                                   uint64_t seed, uint32_t offset,
                                   int32_t* out_tokens, int32_t* out_n_acc, int32_t* out_status,
                                   float* p_at, float* q_at, float* lse, hipStream_t stream);

/*
 * sv_verify_accept_stats -- sv_verify_accept whose target softmax statistics
 * come from the vocabulary projection's epilogue (the sv_pass_gemm `stats`
 * output) instead of a read of the target logits: the fused LM-head verify.
 *
 * Defines exactly what sv_verify_accept defines (Speculative Decoding Clearly
 * Explained, "Check the guesses together", "Accept from left to right",
 * "Correct and continue"); only the log-sum-exp of each target row is formed
 * by merging its (max, sum of exp) pairs of 64 logits.
 *
 *   target_logits  f32 [B, k+1, V]: still read at the draft tokens and along
 *                  the one residual / bonus row
 *   target_stats   f32 pairs [B, k+1, ceil(V/64), 2] (not NULL): the stats of
 *                  a pass GEMM with N = V over m = B (k+1) rows, trial-major
 *   every other argument, the outputs, the workspace
 *   (sv_verify_accept_workspace_bytes) and the errors as sv_verify_accept.
 * A pair with a NaN sum marks its row invalid (status 2), as a NaN or +inf
 * logit does.  Decisions equal sv_verify_accept's on the same logits up to
 * the binary32 rounding of the row normalizers.
 */
sv_status sv_verify_accept_stats(const float* target_logits, const float* target_stats,
                                 const float* draft_logits, const int32_t* draft_tokens, int B,
                                 int k, int V, uint64_t seed, uint32_t offset,
                                 int32_t* out_tokens, int32_t* out_n_acc, int32_t* out_status,
                                 float* p_at, float* q_at, float* lse,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * sv_verify_sampled -- verification under a request's sampling settings:
 * temperature, top-k and top-p, or greedy verification at temperature 0.
 *
 * Settings (Karpathy's Trick for Faster Local LLMs, "Call Uzu through a local
 * application endpoint": the server honours temperature, top_p and top_k;
 * "Use one client for Uzu, MLX, and llama.cpp": temperature 0):
 *   temperature T  0: greedy; > 0 (finite): logits are divided by T
 *   top_k          0 (or >= V): no truncation; else keep the top_k largest
 *                  logits, smaller indices first among equal logits
 *   top_p          in (0, 1]; 1: no truncation; else, on the renormalised
 *                  top-k row, keep the shortest prefix of tokens in
 *                  decreasing probability (ties by ascending index) whose
 *                  sum reaches top_p (the crossing token is kept)
 * Defines, per independent trial b (Speculative Decoding Clearly Explained,
 * "Accept from left to right" and "Correct and continue"):
 *   T > 0: p'_i, q'_i = the target and draft rows after temperature, top-k
 *   and top-p, renormalised; then exactly the rule of sv_verify_accept on
 *   p', q' with the same Philox uniforms (a draft token outside q's kept set
 *   has q' = 0 and is accepted iff p' > 0).
 *   T = 0: g_i = argmax of target row i (smallest index among equal
 *   maxima); accept d_i iff d_i == g_i, stop at the first mismatch r and
 *   emit g_r; after k matches emit g_k.  No random numbers; draft rows are
 *   not read.
 *   Outputs as sv_verify_accept; p_at / q_at hold p'_i(d_i), q'_i(d_i)
 *   (greedy: 1 if d_i == g_i else 0, and 1).
 *
 *   target_logits, draft_logits, draft_tokens, B, k, V, seed, offset,
 *   out_tokens, out_n_acc, out_status, p_at, q_at: as sv_verify_accept
 *   (B <= 65535)
 *   sampling   host pointer to the settings; invalid settings return
 *              SV_ERR_INVALID_ARG before any launch
 *   workspace  device scratch of at least
 *              sv_verify_sampled_workspace_bytes(B, k, V) bytes; contents need
 *              no initialization and are clobbered.
 */
typedef struct sv_sampling {
  float temperature;
  int top_k;
  float top_p;
} sv_sampling;
size_t sv_verify_sampled_workspace_bytes(int B, int k, int V);
sv_status sv_verify_sampled(const float* target_logits, const float* draft_logits,
                            const int32_t* draft_tokens, int B, int k, int V,
                            const sv_sampling* sampling, uint64_t seed, uint32_t offset,
                            int32_t* out_tokens, int32_t* out_n_acc, int32_t* out_status,
                            float* p_at, float* q_at, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/*
 * sv_verify_coupled -- Gumbel-max coupled verification: the drafter and the
 * target draw with the same noise, so matching distributions give matching
 * tokens (@trymirai timeline, the post on speculators rejected although they
 * predict the distribution correctly; Speculative Decoding Clearly
 * Explained, "Accept from left to right" and "Correct and continue").
 *
 * Defines, per independent trial b and position i = 0..k:
 *   u_i[v] = Philox4x32-10 word (v mod 4) with key = (seed & 0xffffffff,
 *            seed >> 32) and counter (v / 4, i, b, 3 + 256 * offset), as
 *            (word >> 8) * 2^-24: one counter serves four consecutive entries
 *   g_i[v] = -log(-log u_i[v])  (binary64; u = 0 gives -inf)
 *   c_i    = argmax_v (target[b, i, v] + g_i[v]), the smallest index among
 *            equal scores (a draw from softmax(target[b, i, :]))
 *   Accept d_i iff d_i == c_i; stop at the first disagreement r and emit c_r;
 *   after k agreements emit c_k.  The drafter is expected to have drawn d_i
 *   as the argmax of its own logits plus the same g_i.
 *
 *   target_logits  f32 [B, k+1, V]
 *   draft_tokens   int32 [B, k]
 *   B 1..65535, 1 <= k <= SV_MAX_ROWS, V >= 1, (k+1)*V < 2^31,
 *   offset < 2^24
 *   out_tokens     int32 [B, k+1]: d_0..d_{n_acc-1}, then c_{n_acc}, then -1
 *   out_n_acc      int32 [B]  (-1 when out_status[b] != 0)
 *   out_status     int32 [B]  0 ok; 1 a draft token outside [0, V);
 *                             2 a target row holds NaN or +inf or no finite
 *                             logit
 *   choices        int32 [B, k+1] optional (NULL to skip): c_0..c_k
 *   workspace      device scratch of at least
 *                  sv_verify_coupled_workspace_bytes(B, k, V) bytes; contents
 *                  need no initialization and are clobbered.
 */
size_t sv_verify_coupled_workspace_bytes(int B, int k, int V);
sv_status sv_verify_coupled(const float* target_logits, const int32_t* draft_tokens, int B,
                            int k, int V, uint64_t seed, uint32_t offset, int32_t* out_tokens,
                            int32_t* out_n_acc, int32_t* out_status, int32_t* choices,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * sv_verify_tree -- greedy verification of a draft tree.
 *
 * Source: Karpathy's Trick for Faster Local LLMs, "Issue with parallel draft
 * generation" (the main model verifies the drafted tree and accepts its
 * longest valid path) and "Verifying a draft tree without restoring model
 * state" (one target pass scores every branch); Local LLM 4x Faster (the
 * whole tree verified at once, every output token confirmed by the target).
 *
 * Defines, per independent trial b, for a tree of n draft nodes (node j: token
 * tok[j], parent par[j], -1 for a child of the last accepted token; parents
 * come before children):
 *   row 0 of the target is its distribution at the root's children, row j+1
 *   its distribution after node j;
 *   c_r    = argmax_v target[b, r, v], the smallest index among equal maxima
 *   node j is valid iff par[j] is -1 or a valid node, and tok[j] == c_{par[j]+1}
 *   The accepted path is the longest chain of valid nodes from the root; among
 *   equally long chains the one ending at the smallest node index.  Emitted:
 *   the path's tokens, then c at the row after its last node (c_0 if empty).
 *
 *   target_logits  f32 [B, n+1, V]
 *   tokens         int32 [B, n]
 *   parents        int32 [B, n]
 *   B 1..65535, 1 <= n <= SV_MAX_ROWS, V >= 1, (n+1)*V < 2^31
 *   out_tokens     int32 [B, n+1]: the path's tokens, the bonus, then -1
 *   out_n_acc      int32 [B]  path length (-1 when out_status[b] != 0)
 *   out_status     int32 [B]  0 ok; 1 a token outside [0, V); 2 a target row
 *                             holds NaN or +inf or no finite logit; 3 a parent
 *                             outside [-1, j) (checked in this order)
 *   out_path       int32 [B, n] optional (NULL to skip): the accepted node
 *                  indices from the root, then -1
 *   workspace      device scratch of at least
 *                  sv_verify_tree_workspace_bytes(B, n, V) bytes; contents need
 *                  no initialization and are clobbered.
 * All pointers are device memory, 16-byte aligned; the call is asynchronous
 * on `stream`.  Errors are returned before any launch.
 */
size_t sv_verify_tree_workspace_bytes(int B, int n, int V);
sv_status sv_verify_tree(const float* target_logits, const int32_t* tokens,
                         const int32_t* parents, int B, int n, int V, int32_t* out_tokens,
                         int32_t* out_n_acc, int32_t* out_status, int32_t* out_path,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * sv_philox4x32_10 -- the device Philox4x32-10 bijection used by
 * sv_verify_accept, exposed so callers can check it against the published
 * known-answer vectors.  ctr uint32 [n, 4], key uint32 [n, 2], out uint32
 * [n, 4]; n >= 1.
 */
sv_status sv_philox4x32_10(const uint32_t* ctr, const uint32_t* key, uint32_t* out,
                           int n, hipStream_t stream);

/*
 * sv_read_bandwidth_probe -- streams `bytes` bytes from `src` with 16-byte
 * loads and writes one 32-bit checksum per workgroup to `sink`
 * (sink must hold sv_read_probe_sink_words() words).  A plain read kernel
 * used to state the measured HBM read peak next to roofline fractions.
 * bytes % 16 == 0.
 */
int sv_read_probe_sink_words(void);
sv_status sv_read_bandwidth_probe(const void* src, size_t bytes, uint32_t* sink,
                                  hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
