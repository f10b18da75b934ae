"""Greedy verification of a draft tree, in binary64 (test infrastructure).

Source: Karpathy's Trick for Faster Local LLMs, "Issue with parallel draft
generation" (Weaver keeps several coherent paths; the main model verifies the
tree and accepts the longest valid path) and "Verifying a draft tree without
restoring model state" (the target computes what every candidate branch needs
in one pass; state is committed only along the accepted path); Local LLM 4x
Faster (the 9B model verifies the entire tree at once and accepts the longest
path; every output token is confirmed by it).  Greedy acceptance as in
oracle.sampling (temperature 0).

Readings taken where the pages are silent:

1. A tree of n draft nodes: node j holds a draft token tok[j] and a parent
   par[j], -1 for a child of the root (the last accepted token); parents come
   before children (-1 <= par[j] < j).
2. The target scores n + 1 rows: row 0 is its distribution at the root's
   children, row j + 1 its distribution after node j (at node j's children).
3. The target's choice at a row is its argmax, the smallest index among equal
   maxima.  A node is valid iff its parent is the root or a valid node and its
   token equals the choice at its parent's row (row par[j] + 1, row 0 for the
   root's children).
4. The accepted path is the longest chain of valid nodes from the root; among
   equally long chains the one ending at the smallest node index.  Emitted:
   the path's tokens, then the target's choice at the row after the path's
   last node (row 0 for an empty path).  n_acc = path length.
5. A draft token outside [0, V) is status 1, a target row with a NaN, a +inf
   or no finite logit status 2, a parent outside [-1, j) status 3.

Parity: pinned -- a chain (par[j] = j - 1) is greedy verification of the same
drafts (oracle.sampling at temperature 0); hand-built trees fix the longest
path, its tie rule, the emitted bonus and the status codes.
"""

import numpy as np

from .accept import AcceptResult, row_lse
from .sampling import greedy_choice


def tree_trial(target_logits, tokens, parents):
    """One trial: target_logits [n + 1, V], tokens [n], parents [n].  The
    result's extra["path"] lists the accepted node indices, extra["choices"]
    the target's choice per row."""
    t = np.asarray(target_logits, dtype=np.float64)
    tok = np.asarray(tokens, dtype=np.int64)
    par = np.asarray(parents, dtype=np.int64)
    n = tok.shape[0]
    V = t.shape[-1]
    if t.shape != (n + 1, V) or par.shape != (n,):
        raise ValueError("expected target [n+1, V], tokens [n], parents [n]")
    if np.any((tok < 0) | (tok >= V)):
        return AcceptResult(status=1, n_acc=-1, tokens=[])
    _, ok = row_lse(t)
    if not ok.all():
        return AcceptResult(status=2, n_acc=-1, tokens=[])
    if any(not (-1 <= par[j] < j) for j in range(n)):
        return AcceptResult(status=3, n_acc=-1, tokens=[])
    choice = [greedy_choice(t[r]) for r in range(n + 1)]
    depth = [0] * n                      # path length ending at node j, 0 if invalid
    for j in range(n):
        p = par[j]
        parent_ok = p < 0 or depth[p] > 0
        if parent_ok and tok[j] == choice[p + 1]:
            depth[j] = 1 + (depth[p] if p >= 0 else 0)
    best = -1
    for j in range(n):
        if depth[j] > 0 and (best < 0 or depth[j] > depth[best]):
            best = j
    path = []
    j = best
    while j >= 0:
        path.append(int(j))
        j = int(par[j])
    path.reverse()
    bonus_row = best + 1                 # 0 for an empty path
    return AcceptResult(status=0, n_acc=len(path),
                        tokens=[int(tok[j]) for j in path] + [choice[bonus_row]],
                        residual_row=bonus_row,
                        extra={"path": path, "choices": choice})


def verify_tree(target_logits, tokens, parents):
    """Batch: target_logits [B, n + 1, V], tokens [B, n], parents [B, n]."""
    t = np.asarray(target_logits)
    tok = np.asarray(tokens)
    par = np.asarray(parents)
    return [tree_trial(t[b], tok[b], par[b]) for b in range(tok.shape[0])]
