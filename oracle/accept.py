"""Accept/correct step of speculative sampling in binary64 (test infrastructure).

Source: Speculative Decoding Clearly Explained --
* "Accept from left to right": with p the target's probability for a guess
  and q the draft's, accept with probability min(1, p/q), stopping at the
  first rejection;
* "Correct and continue": discard the rejected token and every later guess,
  sample the replacement from the positive part of (target - draft),
  normalized into probabilities; "on", "the" accepted, "red" rejected,
  replaced by "big": three tokens from one pass; if every guess is accepted
  the target supplies one additional token.
Karpathy's Trick for Faster Local LLMs, "Producing several tokens from one
model pass": five drafts with the first four accepted advance the sequence by
five tokens (four drafts plus the target's own token).

Readings taken where the pages are silent:

1. Probabilities are the plain softmax of the logits (temperature 1, no
   truncation).  A logit of -inf is probability 0; a row with a NaN, a +inf
   or no finite logit is invalid (status 2).
2. "Accept with probability min(1, p/q)" is decided as u * q(d) < p(d) with u
   uniform on [0, 1): the acceptance probability is then exactly min(1, p/q);
   p = 0 always rejects.
3. The target supplies k + 1 rows: row i scores draft position i, row k is
   the distribution after all k drafts (the bonus token).
4. Replacement at the first rejected position r: weights
   w_v = max(0, p_r(v) - q_r(v)); bonus: w_v = p_k(v).  S = sum w; the token
   is the smallest v whose running sum C_v (ascending vocab order) exceeds
   u' * S.  If S is 0 (possible only through rounding), w = p_r.
5. A draft token outside [0, V) makes the trial invalid (status 1).
6. Near-tie flags: an accept decision with |u q - p| < 1e-6, or a residual
   draw whose threshold lies within 1e-6 * S of the chosen bin's edges, is
   marked; a binary32 implementation may legitimately decide it the other
   way.  A decision with p = 0 (always rejected) or q = 0 < p (always
   accepted) is exact in any precision and is not marked.

Parity: pinned -- worked examples (tests/golden), exact output law by
quadrature over the uniforms on tiny vocabularies, chi-square on Philox-driven
trials, acceptance-length expectation, and the special cases p = q (all
accepted, bonus) and p(d) = 0 (always rejected, residual = p).
"""

from dataclasses import dataclass, field

import numpy as np

from .philox import accept_uniforms

NEAR_TIE_ACCEPT = 1e-6
NEAR_TIE_RESIDUAL = 1e-6


def row_lse(logits):
    """Log-sum-exp of each row in binary64 and a validity flag per row."""
    a = np.asarray(logits, dtype=np.float64)
    bad = np.isnan(a).any(axis=-1) | np.isposinf(a).any(axis=-1)
    mx = np.max(np.where(np.isnan(a), -np.inf, a), axis=-1)
    bad |= ~np.isfinite(mx)
    safe_mx = np.where(np.isfinite(mx), mx, 0.0)
    with np.errstate(invalid="ignore", over="ignore"):
        ssum = np.sum(np.exp(a - safe_mx[..., None]), axis=-1)
        lse = safe_mx + np.log(ssum)
    return np.where(bad, np.nan, lse), ~bad


def probs(logits, lse):
    """Softmax row from its logits and log-sum-exp (exp(-inf) = 0)."""
    return np.exp(np.asarray(logits, dtype=np.float64) - lse)


@dataclass
class AcceptResult:
    status: int                     # 0 ok, 1 draft token out of range, 2 invalid row
    n_acc: int                      # accepted drafts (-1 when status != 0)
    tokens: list                    # accepted drafts then the replacement/bonus
    p_at: np.ndarray = None         # p_i(d_i), i < k
    q_at: np.ndarray = None         # q_i(d_i), i < k
    lse_target: np.ndarray = None   # [k + 1]
    lse_draft: np.ndarray = None    # [k]
    accept_flags: np.ndarray = None  # near-tie flag per examined position
    residual_flag: bool = False
    residual_row: int = -1
    weights_sum: float = float("nan")
    extra: dict = field(default_factory=dict)

    @property
    def n_out(self):
        return self.n_acc + 1 if self.status == 0 else 0


def accept_trial(target_logits, draft_logits, draft_tokens, u, u2, ties=None, force=None):
    """One trial of the accept/correct step with explicit uniforms.

    target_logits [k + 1, V], draft_logits [k, V], draft_tokens [k];
    u, u2: uniforms on [0, 1) for positions 0..k (u2[r] is used for the
    replacement or bonus draw at position r).
    """
    t = np.asarray(target_logits, dtype=np.float64)
    d = np.asarray(draft_logits, dtype=np.float64)
    toks = np.asarray(draft_tokens, dtype=np.int64)
    k = toks.shape[0]
    V = t.shape[-1]
    if t.shape != (k + 1, V) or d.shape != (k, V):
        raise ValueError("expected target [k+1, V] and draft [k, V]")
    if np.any((toks < 0) | (toks >= V)):
        return AcceptResult(status=1, n_acc=-1, tokens=[])
    lse_t, ok_t = row_lse(t)
    lse_d, ok_d = row_lse(d)
    if not (ok_t.all() and ok_d.all()):
        return AcceptResult(status=2, n_acc=-1, tokens=[],
                            lse_target=lse_t, lse_draft=lse_d)

    P = probs(t, lse_t[:, None])
    Q = probs(d, lse_d[:, None])
    res = accept_on_probs(P, Q, toks, u, u2, ties, force)
    res.lse_target = lse_t
    res.lse_draft = lse_d
    return res


def accept_on_probs(P, Q, draft_tokens, u, u2, ties=None, force=None):
    """The accept scan and the replacement/bonus draw on explicit rows.

    P [k + 1, V]: the target's distributions (row k for the bonus), Q [k, V]:
    the draft's, both binary64 and normalised; draft tokens in [0, V).  The
    rule is the one of accept_trial (readings 2, 4 and 6).  ties = (accept,
    residual[, accept relative to p]) replaces the near-tie widths of
    reading 6: an accept decision is flagged when |u q - p| is below
    max(accept, relative * p) (flags only; the decisions do not depend on it).

    force = {position: accepted} takes the given decision at a position whose
    decision is flagged (a near tie of reading 6, which a binary32 evaluation
    may take either way) and continues the trial from it; forcing a position
    that is not flagged raises ValueError.  It lets a comparison follow the
    device's choice at an undecidable position and check everything after it.
    """
    tie_a, tie_r, tie_p = ((NEAR_TIE_ACCEPT, NEAR_TIE_RESIDUAL, 0.0) if ties is None
                           else (tuple(ties) + (0.0,))[:3])
    P = np.asarray(P, dtype=np.float64)
    Q = np.asarray(Q, dtype=np.float64)
    toks = np.asarray(draft_tokens, dtype=np.int64)
    k = toks.shape[0]
    V = P.shape[-1]
    idx = np.arange(k)
    p_at = P[idx, toks]
    q_at = Q[idx, toks]

    # Left to right, stop at the first rejection.
    n_acc = k
    flags = np.zeros(k, dtype=bool)
    for i in range(k):
        lhs = u[i] * q_at[i]
        flags[i] = (abs(lhs - p_at[i]) < max(tie_a, tie_p * p_at[i]) and p_at[i] > 0.0
                    and q_at[i] > 0.0)
        accepted = lhs < p_at[i]
        if force is not None and i in force:
            if not flags[i]:
                raise ValueError(f"position {i} is not a near tie; its decision is fixed")
            accepted = bool(force[i])
        if not accepted:
            n_acc = i
            break

    r = n_acc
    p_r = P[r]
    if r < k:
        w = np.maximum(0.0, p_r - Q[r])
    else:
        w = p_r
    csum = np.cumsum(w)
    if not csum[-1] > 0.0:
        w = p_r
        csum = np.cumsum(w)
    S = csum[-1]
    thr = u2[r] * S
    v = int(np.searchsorted(csum, thr, side="right"))
    v = min(v, V - 1)
    lo = csum[v - 1] if v > 0 else 0.0
    rflag = (abs(thr - lo) < tie_r * S) or (abs(csum[v] - thr) < tie_r * S)
    return AcceptResult(status=0, n_acc=n_acc,
                        tokens=[int(x) for x in toks[:n_acc]] + [v],
                        p_at=p_at, q_at=q_at,
                        accept_flags=flags[:min(n_acc + 1, k)],
                        residual_flag=bool(rflag), residual_row=r,
                        weights_sum=float(S),
                        extra={"residual_csum": csum, "residual_thr": float(thr)})


def verify_accept(target_logits, draft_logits, draft_tokens, seed, offset=0,
                  trial_base=0, ties=None):
    """Batch of independent trials; trial b draws Philox counter (i, b, offset, 0).

    target_logits [B, k + 1, V], draft_logits [B, k, V], draft_tokens [B, k].
    Returns a list of AcceptResult.
    """
    t = np.asarray(target_logits)
    d = np.asarray(draft_logits)
    toks = np.asarray(draft_tokens)
    B, k = toks.shape
    out = []
    for b in range(B):
        u, u2 = accept_uniforms(seed, trial_base + b, k, offset=offset)
        out.append(accept_trial(t[b], d[b], toks[b], u, u2, ties))
    return out
