"""Fused LM-head verification, in binary64 (test infrastructure).

Source: Speculative Decoding Clearly Explained, "Check the guesses together"
(the target scores every draft position in one forward pass, whose last step
is the projection onto the vocabulary) and "Accept from left to right" (p is
the target's probability of a guess, so every scored row is normalized over
the vocabulary); Karpathy's Trick for Faster Local LLMs, "Why batch-one
decoding is memory-bound" (a pass streams every weight once, the vocabulary
projection's included) and "How Uzu optimizes bytes and tokens per pass"
(4-bit asymmetric group weights).

Readings taken where the pages are silent:

1. The vocabulary projection is a 4-bit asymmetric group-64 product like the
   other matrices of the pass (oracle.qgemm.qgemm_w4): logits = H W^T over
   the B (k + 1) hidden rows, trial-major (rows b (k+1) .. b (k+1) + k are
   trial b's k + 1 scored positions).
2. Softmax statistics per row and per 64 consecutive vocabulary entries g
   (the last group may be shorter): M_g = max, S_g = sum exp(l - M_g);
   S_g = 0 when M_g = -inf; a group holding a NaN or +inf logit is invalid.
3. A row's log-sum-exp is the merge of its groups: M = max_g M_g,
   lse = M + log sum_g S_g exp(M_g - M); a row with an invalid group, or with
   M = -inf, is invalid (status 2, as in oracle.accept).
4. The accept step is oracle.accept's on the projected logits.
5. Near ties: the logits come out of a binary32 GEMM (error around 1e-6 of
   the row norm, so each weight p(v) moves by a few 1e-6 of itself and a
   running sum of the residual weights by at most that fraction of S).  An
   accept decision is flagged when |u q - p| < 1e-4 p (p itself is often
   near 1e-4 here, so the band is relative), a residual draw when its
   threshold lies within 1e-5 S of the chosen bin's edges.  Over a vocabulary
   of V entries a bin averages S / V, so at V in the hundred thousands most
   draws are near a tie in this sense: any token whose bin comes within
   1e-5 S of the threshold is then a correct draw (the result carries the
   running sums and the threshold to check that).

Parity: pinned -- constant rows give M = c and S = group size; merged group
statistics equal the log-sum-exp of the whole row and its closed form on
rows of log(1..V); NaN, +inf and all -inf groups; one-hot hidden rows
through a designed projection give known integer logits, so the fused
verification equals oracle.accept on them.
"""

import numpy as np

from .accept import verify_accept
from .qgemm import qgemm_w4

GROUP_STATS = 64
NEAR_TIE_LMHEAD = (0.0, 1e-5, 1e-4)         # (accept, residual, accept / p), reading 5


def group_softmax_stats(logits, group=GROUP_STATS):
    """Reading 2: (M, S, bad) per row and group, each [..., ceil(V / group)]."""
    a = np.asarray(logits, dtype=np.float64)
    V = a.shape[-1]
    G = (V + group - 1) // group
    pad = G * group - V
    a = np.concatenate([a, np.full(a.shape[:-1] + (pad,), -np.inf)], axis=-1)
    a = a.reshape(a.shape[:-1] + (G, group))
    bad = np.isnan(a).any(axis=-1) | np.isposinf(a).any(axis=-1)
    M = np.max(np.where(np.isnan(a), -np.inf, a), axis=-1)
    safe = np.where(np.isfinite(M), M, 0.0)
    with np.errstate(invalid="ignore", over="ignore"):
        S = np.sum(np.exp(a - safe[..., None]), axis=-1)
    S = np.where(M == -np.inf, 0.0, S)
    return M, S, bad


def merge_group_stats(M, S, bad):
    """Reading 3: (lse, ok) per row from its group statistics."""
    M = np.asarray(M, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    top = np.max(M, axis=-1)
    ok = ~np.asarray(bad).any(axis=-1) & np.isfinite(top)
    safe = np.where(ok, top, 0.0)
    with np.errstate(invalid="ignore", over="ignore"):
        total = np.sum(np.where(M == -np.inf, 0.0, S * np.exp(M - safe[..., None])), axis=-1)
        lse = safe + np.log(total)
    return np.where(ok, lse, np.nan), ok


def lm_head_logits(hidden, codes, scales, zeros, B, k, group=64, chunk=8192):
    """Reading 1: logits [B, k + 1, V] of the W4 vocabulary projection (the
    product is formed in vocabulary chunks only to bound memory)."""
    V = np.asarray(codes).shape[0]
    out = np.empty((np.asarray(hidden).shape[0], V))
    for n0 in range(0, V, chunk):
        n1 = min(V, n0 + chunk)
        out[:, n0:n1] = qgemm_w4(hidden, codes[n0:n1], scales[n0:n1], zeros[n0:n1], group)
    return out.reshape(B, k + 1, V)


def lm_head_verify(hidden, codes, scales, zeros, draft_logits, draft_tokens, seed, offset=0,
                   group=64):
    """The fused verify: projection (reading 1), then oracle.accept with the
    near-tie widths of reading 5.  Returns (logits, results)."""
    toks = np.asarray(draft_tokens)
    B, k = toks.shape
    logits = lm_head_logits(hidden, codes, scales, zeros, B, k, group)
    res = verify_accept(logits, draft_logits, toks, seed, offset, ties=NEAR_TIE_LMHEAD)
    return logits, res
