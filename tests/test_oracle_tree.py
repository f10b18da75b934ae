"""Pins of the oracle's greedy draft-tree verification.

* a chain tree is greedy verification of the same drafts (oracle.sampling at
  temperature 0);
* hand-built trees fix the longest valid path (Karpathy's Trick for Faster
  Local LLMs, "Issue with parallel draft generation": the main model accepts
  the longest valid path), the tie rule, the bonus token and the statuses.
"""
import numpy as np

from oracle import accept_trial_sampled, greedy_choice
from oracle.tree import tree_trial, verify_tree


def _rows(choices, V):
    """Target rows whose argmax is the given token (margin 5)."""
    t = np.zeros((len(choices), V))
    for r, c in enumerate(choices):
        t[r, c] = 5.0
    return t


def test_chain_tree_is_greedy_verification():
    rng = np.random.default_rng(4)
    k, V = 6, 25
    for trial in range(200):
        t = rng.normal(0, 1, (k + 1, V))
        toks = rng.integers(0, V, k)
        agree = rng.integers(0, k + 1)
        for i in range(agree):
            toks[i] = greedy_choice(t[i])
        chain = tree_trial(t, toks, np.arange(k) - 1)
        g = accept_trial_sampled(t, np.zeros((k, V)), toks, None, None, 0.0)
        assert chain.n_acc == g.n_acc and chain.tokens == g.tokens
        assert chain.extra["path"] == list(range(chain.n_acc))


def test_longest_valid_branch():
    # rows: 0 root, j+1 after node j.  Choices: root -> 2, after node 0 -> 4,
    # after node 2 -> 1, after node 4 -> 3.
    V = 6
    choices = [2, 4, 0, 1, 0, 3, 0, 0]
    t = _rows(choices, V)
    toks = [2, 3, 4, 5, 1, 4, 0]
    par = [-1, -1, 0, 0, 2, 1, 4]
    r = tree_trial(t, toks, par)
    # node 0 (2 = root choice) valid, node 1 not; node 2 (4 = choice after
    # node 0) valid, node 3 not; node 4 (1 = choice after node 2) valid;
    # node 5 has an invalid parent; node 6 (0 != 3) is not valid
    assert r.extra["path"] == [0, 2, 4]
    assert r.n_acc == 3 and r.tokens == [2, 4, 1, 3]


def test_equal_lengths_end_at_the_smaller_index():
    # two root children with the root's choice (duplicate sibling tokens),
    # each with one valid child
    V = 5
    choices = [1, 2, 3, 0, 4]        # rows 0..4
    t = _rows(choices, V)
    toks = [1, 1, 3, 2]               # nodes 0, 1 at the root; 2 under 1, 3 under 0
    par = [-1, -1, 1, 0]
    r = tree_trial(t, toks, par)
    # node 3 (2 = choice after node 0) and node 2 (3 = choice after node 1)
    # both end paths of length 2: the smaller end index, node 2, wins
    assert r.extra["path"] == [1, 2]
    assert r.tokens == [1, 3, choices[3]]


def test_nothing_valid_emits_the_root_choice():
    V = 4
    t = _rows([3, 0, 0], V)
    r = tree_trial(t, [0, 1], [-1, 0])
    assert r.n_acc == 0 and r.tokens == [3] and r.extra["path"] == []


def test_statuses():
    t = np.zeros((3, 4))
    assert tree_trial(t, [0, 4], [-1, 0]).status == 1
    assert tree_trial(t, [0, 1], [-1, 1]).status == 3
    assert tree_trial(t, [0, 1], [-2, 0]).status == 3
    bad = t.copy()
    bad[2, 1] = np.inf
    assert tree_trial(bad, [0, 1], [-1, 0]).status == 2
    res = verify_tree(np.stack([t, t]), [[0, 1], [0, 1]], [[-1, 0], [-1, -1]])
    assert [r.status for r in res] == [0, 0]
