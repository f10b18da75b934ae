"""Verification under a request's sampling settings, in binary64 (test
infrastructure).

Source: Karpathy's Trick for Faster Local LLMs, "Call Uzu through a local
application endpoint" (the local server honours temperature, top_p and
top_k) and "Use one client for Uzu, MLX, and llama.cpp" (the benchmark client
asks for temperature 0, the same answer on every run); the SDK listings of the
same page select a greedy sampling method.  Speculative Decoding Clearly
Explained, "Accept from left to right" and "Correct and continue": the accept
rule and the residual draw, here applied to the distributions the settings
define.

Readings taken where the pages are silent:

1. Temperature T > 0 divides the logits by T.  T = 0 is greedy verification:
   the target's choice at position i is the argmax of its row i (the smallest
   index among equal maxima); a draft is accepted iff it equals that choice,
   the first mismatch is replaced by the choice, and after k matches the bonus
   is the argmax of row k.  No uniforms are used and the draft rows are not
   consulted (an invalid draft row does not invalidate the trial).
2. Order: temperature, then top-k, then top-p on the renormalised top-k
   distribution.  top-k and top-p act on ranks, which a positive temperature
   does not change.
3. top-k keeps the k largest logits; among equal logits at the boundary the
   smaller vocabulary indices are kept.  top_k = 0 or top_k >= V keeps all.
4. top-p orders the probabilities decreasingly (ties by ascending index) and
   keeps the shortest prefix whose sum reaches top_p; the token that crosses
   top_p is kept.  top_p = 1 keeps all.
5. Target and draft rows are truncated and renormalised alike; the accept rule
   and the residual/bonus draw of accept.py then run on those distributions.
   A draft token outside the draft's kept set has q = 0 and is accepted iff
   p > 0 (u * 0 < p).
6. Masses are compared in binary64.  Near-tie flag: a top-p boundary whose
   running sum lies within 1e-9 of top_p (either side of the crossing token)
   may be drawn the other way by a binary64 implementation that sums in
   another order.  The settings are the binary32 values an implementation
   receives; callers pass them rounded.

Parity: pinned -- the default settings reproduce accept.py exactly; top_k = 1
and greedy verification agree for any uniforms; hand-worked truncations
(boundary inclusion, ties by index, temperature) in tests/golden; the exact
output law equals the truncated target distribution by quadrature over the
uniforms.
"""

import numpy as np

from .accept import AcceptResult, accept_on_probs, row_lse
from .philox import accept_uniforms

NEAR_TIE_TOP_P = 1e-9


def check_settings(temperature, top_k, top_p):
    """Raise ValueError for settings outside the domain stated above."""
    if not (np.isfinite(temperature) and temperature >= 0.0):
        raise ValueError("temperature must be finite and >= 0")
    if int(top_k) != top_k or top_k < 0:
        raise ValueError("top_k must be an integer >= 0")
    if not (0.0 < top_p <= 1.0):
        raise ValueError("top_p must lie in (0, 1]")


def rank_order(logits):
    """Vocabulary indices by decreasing logit, ties by ascending index."""
    a = np.asarray(logits, dtype=np.float64)
    return np.lexsort((np.arange(a.shape[-1]), -a))


def truncated_probs(logits, temperature=1.0, top_k=0, top_p=1.0):
    """Distribution of one row after temperature, top-k and top-p.

    Returns (probs [V] binary64, kept mask [V], top-p near-tie flag).  The row
    must hold a finite maximum (check with row_lse first).
    """
    check_settings(temperature, top_k, top_p)
    if temperature == 0.0:
        raise ValueError("temperature 0 is greedy verification: no distribution")
    a = np.asarray(logits, dtype=np.float64)
    V = a.shape[-1]
    order = rank_order(a)
    kept = np.zeros(V, dtype=bool)
    kept[order[:top_k] if 0 < top_k < V else order] = True
    m = a[order[0]]
    with np.errstate(invalid="ignore"):
        e = np.where(kept, np.exp((a - m) / temperature), 0.0)
    flag = False
    if top_p < 1.0:
        ranked = order[kept[order]]
        p1 = e[ranked] / e[ranked].sum()
        c = np.cumsum(p1)
        j = int(np.searchsorted(c, top_p, side="left"))   # first with c >= top_p
        j = min(j, len(ranked) - 1)
        flag = abs(c[j] - top_p) < NEAR_TIE_TOP_P or \
            (j > 0 and abs(c[j - 1] - top_p) < NEAR_TIE_TOP_P)
        kept = np.zeros(V, dtype=bool)
        kept[ranked[:j + 1]] = True
        e = np.where(kept, e, 0.0)
    return e / e.sum(), kept, bool(flag)


def greedy_choice(logits):
    """Argmax of a row, the smallest index among equal maxima."""
    return int(rank_order(logits)[0])


def accept_trial_sampled(target_logits, draft_logits, draft_tokens, u, u2,
                         temperature=1.0, top_k=0, top_p=1.0):
    """One trial of verification under the given settings (readings 1-6).

    Shapes as accept.accept_trial.  The result's extra["top_p_flags"] lists
    the rows (target rows 0..k, then draft rows 0..k-1) whose top-p boundary
    is a near tie.
    """
    check_settings(temperature, top_k, top_p)
    t = np.asarray(target_logits, dtype=np.float64)
    d = np.asarray(draft_logits, dtype=np.float64)
    toks = np.asarray(draft_tokens, dtype=np.int64)
    k = toks.shape[0]
    V = t.shape[-1]
    if t.shape != (k + 1, V) or d.shape != (k, V):
        raise ValueError("expected target [k+1, V] and draft [k, V]")
    if np.any((toks < 0) | (toks >= V)):
        return AcceptResult(status=1, n_acc=-1, tokens=[])
    _, ok_t = row_lse(t)
    _, ok_d = row_lse(d)
    # greedy verification does not depend on the draft rows
    if not (ok_t.all() and (ok_d.all() or temperature == 0.0)):
        return AcceptResult(status=2, n_acc=-1, tokens=[])
    if temperature == 0.0:
        g = [greedy_choice(t[i]) for i in range(k + 1)]
        n_acc = k
        for i in range(k):
            if toks[i] != g[i]:
                n_acc = i
                break
        return AcceptResult(
            status=0, n_acc=n_acc,
            tokens=[int(x) for x in toks[:n_acc]] + [g[n_acc]],
            p_at=np.array([1.0 if toks[i] == g[i] else 0.0 for i in range(k)]),
            q_at=np.ones(k), accept_flags=np.zeros(min(n_acc + 1, k), dtype=bool),
            residual_row=n_acc, extra={"greedy": g, "top_p_flags": []})
    rows_t = [truncated_probs(t[i], temperature, top_k, top_p) for i in range(k + 1)]
    rows_d = [truncated_probs(d[i], temperature, top_k, top_p) for i in range(k)]
    P = np.stack([r[0] for r in rows_t])
    Q = np.stack([r[0] for r in rows_d])
    res = accept_on_probs(P, Q, toks, u, u2)
    res.extra["top_p_flags"] = [i for i, r in enumerate(rows_t + rows_d) if r[2]]
    return res


def verify_accept_sampled(target_logits, draft_logits, draft_tokens, seed, offset=0,
                          temperature=1.0, top_k=0, top_p=1.0, trial_base=0):
    """Batch of independent trials with the uniforms of accept.verify_accept."""
    t = np.asarray(target_logits)
    d = np.asarray(draft_logits)
    toks = np.asarray(draft_tokens)
    B, k = toks.shape
    out = []
    for b in range(B):
        u, u2 = accept_uniforms(seed, trial_base + b, k, offset=offset)
        out.append(accept_trial_sampled(t[b], d[b], toks[b], u, u2,
                                        temperature, top_k, top_p))
    return out


def sample_drafts(draft_logits, seed, temperature=1.0, top_k=0, top_p=1.0,
                  trial_base=0):
    """Draft tokens drawn from the truncated draft rows (test inputs).

    Inverse CDF in ascending vocab order on the Philox uniforms with tag 1
    (counter (i, b, 0, 1), word 0); greedy settings take the argmax.
    """
    d = np.asarray(draft_logits, dtype=np.float64)
    B, k, V = d.shape
    out = np.zeros((B, k), dtype=np.int32)
    for b in range(B):
        u, _ = accept_uniforms(seed, trial_base + b, k, tag=1)
        for i in range(k):
            if temperature == 0.0:
                out[b, i] = greedy_choice(d[b, i])
                continue
            q, _, _ = truncated_probs(d[b, i], temperature, top_k, top_p)
            c = np.cumsum(q)
            out[b, i] = min(int(np.searchsorted(c, u[i] * c[-1], side="right")), V - 1)
    return out
