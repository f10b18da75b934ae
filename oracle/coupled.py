"""Gumbel-max coupled verification, in binary64 (test infrastructure).

Source: @trymirai timeline, the post on speculators that predict the
distribution correctly and are still rejected ("The random number from 1 to
10 inclusive is"): sample both the speculator and the LLM with the same seed
through the Gumbel-max trick; shared randomness gives a shared outcome when
the distributions match (100% acceptance in that case).  Speculative Decoding
Clearly Explained, "Accept from left to right" and "Correct and continue":
keep the drafts up to the first disagreement and emit the target's own token
there; after k agreements the target supplies one more.

Readings taken where the pages are silent:

1. Noise: position i of trial b draws one uniform per vocabulary entry v from
   Philox4x32-10 (the generator of philox.py) with key = seed: entry v takes
   word v mod 4 of counter (floor(v / 4), i, b, 3 + 256 * offset), as
   u = (w >> 8) 2^-24, so one counter serves four consecutive entries.  The
   Gumbel noise is g = -log(-log(u)) in binary64; u = 0 gives g = -inf
   (never chosen).
2. The target's choice at position i is argmax_v (l_i[v] + g_i[v]) with the
   logit in binary64, the smallest index among equal scores.  The Gumbel-max
   trick makes it a draw from softmax(l_i).  The drafter draws its token with
   the same noise on its own logits; the draft tokens are inputs here.
3. Accept d_i iff it equals the target's choice at i; stop at the first
   disagreement r and emit the target's choice at r; after k agreements emit
   the target's choice at position k (its own noise).  Temperature 1, no
   truncation; the draft logits are not needed.
4. A row of the target with a NaN, a +inf or no finite logit makes the trial
   invalid (status 2); a draft token outside [0, V) status 1.
5. Near tie: a target row whose two best scores differ by less than 1e-9 is
   flagged; a binary64 implementation with another logarithm may order them
   the other way.

Parity: pinned -- equal draft and target rows accept every draft for any
seed (the page's claim); the target's choice follows softmax(l) (chi-square
over trials, and the two-token case against its closed form); the noise is
the documented Philox counter (known-answer vectors pin the generator).
"""

import numpy as np

from .accept import AcceptResult, row_lse
from .philox import philox4x32_10, uniforms24

TAG_COUPLED = 3
NEAR_TIE_COUPLED = 1e-9


def gumbel_noise(seed, trial, position, V, offset=0):
    """Binary64 Gumbel noise of one position (reading 1), length V."""
    seed = int(seed)
    g = np.arange((V + 3) // 4, dtype=np.uint64)          # counter of entries 4g .. 4g+3
    ctr = np.stack([g,
                    np.full_like(g, int(position) & 0xFFFFFFFF),
                    np.full_like(g, int(trial) & 0xFFFFFFFF),
                    np.full_like(g, (TAG_COUPLED + 256 * int(offset)) & 0xFFFFFFFF)], axis=-1)
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], dtype=np.uint64)
    words = philox4x32_10(ctr, key)                       # [counters, 4]: word v mod 4
    u = uniforms24(words.reshape(-1)[:V])
    with np.errstate(divide="ignore"):
        return -np.log(-np.log(u))


def coupled_choice(logits, noise):
    """argmax of logits + noise (smallest index among equal scores) and the
    near-tie flag of reading 5."""
    score = np.asarray(logits, dtype=np.float64) + noise
    order = np.lexsort((np.arange(score.shape[-1]), -score))
    top = int(order[0])
    flag = len(order) > 1 and (score[order[0]] - score[order[1]]) < NEAR_TIE_COUPLED
    return top, bool(flag)


def coupled_trial(target_logits, draft_tokens, seed, trial, offset=0):
    """One trial of coupled verification.  target_logits [k + 1, V], draft
    tokens [k].  extra["choices"] holds the target's choices, extra["flags"]
    the near-tie flags of rows 0..k."""
    t = np.asarray(target_logits, dtype=np.float64)
    toks = np.asarray(draft_tokens, dtype=np.int64)
    k = toks.shape[0]
    V = t.shape[-1]
    if t.shape != (k + 1, V):
        raise ValueError("expected target [k+1, V]")
    if np.any((toks < 0) | (toks >= V)):
        return AcceptResult(status=1, n_acc=-1, tokens=[])
    _, ok = row_lse(t)
    if not ok.all():
        return AcceptResult(status=2, n_acc=-1, tokens=[])
    choices, flags = [], []
    for i in range(k + 1):
        c, f = coupled_choice(t[i], gumbel_noise(seed, trial, i, V, offset))
        choices.append(c)
        flags.append(f)
    n_acc = k
    for i in range(k):
        if toks[i] != choices[i]:
            n_acc = i
            break
    return AcceptResult(status=0, n_acc=n_acc,
                        tokens=[int(x) for x in toks[:n_acc]] + [choices[n_acc]],
                        residual_row=n_acc,
                        extra={"choices": choices, "flags": flags})


def verify_coupled(target_logits, draft_tokens, seed, offset=0, trial_base=0):
    """Batch of independent trials; trial b uses counter word 2 = trial_base + b."""
    t = np.asarray(target_logits)
    toks = np.asarray(draft_tokens)
    return [coupled_trial(t[b], toks[b], seed, trial_base + b, offset)
            for b in range(toks.shape[0])]


def coupled_drafts(draft_logits, seed, offset=0, trial_base=0):
    """The drafter's side (test inputs): argmax of its logits plus the same
    noise, position by position."""
    d = np.asarray(draft_logits, dtype=np.float64)
    B, k, V = d.shape
    out = np.zeros((B, k), dtype=np.int32)
    for b in range(B):
        for i in range(k):
            out[b, i] = coupled_choice(d[b, i], gumbel_noise(seed, trial_base + b, i, V,
                                                             offset))[0]
    return out
