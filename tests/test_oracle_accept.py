"""Pins of the oracle's accept/correct step.

* worked examples printed by the pages (tests/golden), for any uniforms;
* exact output law by quadrature over the uniforms on tiny vocabularies with
  rational distributions (the law of every emitted token equals the target's
  distribution, the distribution-preservation claim of Speculative Decoding
  Clearly Explained, "Correct and continue");
* chi-square and acceptance-length checks on Philox-driven trials;
* special cases p = q, p(d) = 0, invalid inputs.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import accept_trial, verify_accept, accept_uniforms, row_lse
from conftest import load_worked_example


def _logits(rows):
    with np.errstate(divide="ignore"):
        return np.log(np.array(rows, dtype=np.float64))


@pytest.mark.parametrize("name", ["worked_example_page1.txt",
                                  "worked_example_page4.txt",
                                  "worked_example_bonus.txt"])
def test_worked_examples_for_any_uniforms(name):
    ex = load_worked_example(name)
    k = len(ex["tokens"])
    rng = np.random.default_rng(0)
    cases = [(np.zeros(k + 1), np.zeros(k + 1)),
             (np.full(k + 1, 1 - 2.0 ** -24), np.full(k + 1, 1 - 2.0 ** -24))]
    cases += [(rng.random(k + 1), rng.random(k + 1)) for _ in range(200)]
    cases += [accept_uniforms(seed, 0, k) for seed in range(50)]
    for u, u2 in cases:
        res = accept_trial(ex["target"], ex["draft"], ex["tokens"], u, u2)
        assert res.status == 0
        assert res.n_acc == ex["expect_n_acc"]
        assert res.tokens == ex["expect_tokens"]
        assert res.n_out == len(ex["expect_tokens"])


def test_page1_example_gives_three_tokens():
    ex = load_worked_example("worked_example_page1.txt")
    res = verify_accept(ex["target"][None], ex["draft"][None], ex["tokens"][None], seed=0)[0]
    assert res.n_out == 3
    assert [ex["vocab"][t] for t in res.tokens] == ["on", "the", "big"]


def _grid(M):
    return [(i + 0.5) / M for i in range(M)]


def test_exact_law_k1_by_quadrature():
    # p, q with ratios and residual breakpoints on a 1/24 lattice: the midpoint
    # grid integrates the uniforms exactly.
    p0 = [Fraction(3, 8), Fraction(1, 8), Fraction(2, 8), Fraction(2, 8)]
    q0 = [Fraction(1, 8), Fraction(3, 8), Fraction(1, 8), Fraction(3, 8)]
    p1 = [Fraction(1, 8), Fraction(1, 2), Fraction(1, 4), Fraction(1, 8)]
    V, M = 4, 24
    t = _logits([[float(v) for v in p0], [float(v) for v in p1]])
    d = _logits([[float(v) for v in q0]])
    first = [Fraction(0)] * V
    second = [Fraction(0)] * V
    reach = Fraction(0)
    g = _grid(M)
    for dt in range(V):
        for u0 in g:
            for a in g:
                for b in g:
                    res = accept_trial(t, d, [dt], [u0, 0.0], [a, b])
                    w = q0[dt] / (M ** 3)
                    first[res.tokens[0]] += w
                    if res.n_out == 2:
                        reach += w
                        second[res.tokens[1]] += w
    assert first == p0
    # given the draft was accepted, the bonus token follows the target's row 1
    assert [s / reach for s in second] == p1
    # acceptance probability = sum_v min(p, q)
    assert reach == sum(min(a, b) for a, b in zip(p0, q0))


def test_exact_law_k2_second_position():
    p0 = [Fraction(1, 2), Fraction(1, 4), Fraction(1, 4)]
    q0 = [Fraction(1, 4), Fraction(1, 2), Fraction(1, 4)]
    p1 = [Fraction(1, 2), Fraction(1, 3), Fraction(1, 6)]
    q1 = [Fraction(1, 6), Fraction(1, 6), Fraction(2, 3)]
    p2 = [Fraction(1, 3)] * 3
    V, M = 3, 12
    t = _logits([[float(v) for v in r] for r in (p0, p1, p2)])
    d = _logits([[float(v) for v in r] for r in (q0, q1)])
    g = _grid(M)
    # position 1, conditional on reaching it; u'_0 and u'_2 held fixed
    pos1 = [Fraction(0)] * V
    reach = Fraction(0)
    for d0 in range(V):
        for d1 in range(V):
            for u0 in g:
                for u1 in g:
                    for b in g:
                        res = accept_trial(t, d, [d0, d1], [u0, u1, 0.0], [0.37, b, 0.61])
                        w = q0[d0] * q1[d1] / (M ** 3)
                        if res.n_out >= 2:
                            reach += w
                            pos1[res.tokens[1]] += w
    assert [x / reach for x in pos1] == p1
    # position 0 law with u'_0 on the grid
    pos0 = [Fraction(0)] * V
    for d0 in range(V):
        for d1 in range(V):
            for u0 in g:
                for a in g:
                    res = accept_trial(t, d, [d0, d1], [u0, 0.5, 0.0], [a, 0.29, 0.83])
                    pos0[res.tokens[0]] += q0[d0] * q1[d1] / (M ** 2)
    assert pos0 == p0


def _chi2(counts, probs):
    n = counts.sum()
    e = n * probs
    keep = e > 0
    assert np.all(counts[~keep] == 0)
    return (((counts - e) ** 2)[keep] / e[keep]).sum(), keep.sum() - 1


def test_chi_square_and_acceptance_length_philox_trials():
    rng = np.random.default_rng(11)
    k, V, B = 3, 8, 20000
    t = rng.normal(0, 2, size=(k + 1, V))
    d = t[:k] + rng.normal(0, 1, size=(k, V))
    p = np.exp(t - row_lse(t)[0][:, None])
    q = np.exp(d - row_lse(d)[0][:, None])
    drafts = np.stack([rng.choice(V, size=B, p=q[i]) for i in range(k)], axis=1)
    T = np.broadcast_to(t, (B, k + 1, V))
    D = np.broadcast_to(d, (B, k, V))
    res = verify_accept(T, D, drafts, seed=7)
    n_acc = np.array([r.n_acc for r in res])
    # every emitted position j, conditional on reaching it, follows p_j
    for j in range(k + 1):
        toks = np.array([r.tokens[j] for r in res if r.n_out > j])
        chi2, dof = _chi2(np.bincount(toks, minlength=V).astype(float), p[j])
        assert chi2 < dof + 6 * np.sqrt(2 * dof) + 10, (j, chi2, dof)
    beta = np.minimum(p[:k], q).sum(axis=1)
    P = np.cumprod(beta)                       # P(n_acc >= j), j = 1..k
    mean = P.sum()
    var = sum((2 * j + 1) * P[j] for j in range(k)) - mean ** 2
    z = (n_acc.mean() - mean) / np.sqrt(var / B)
    assert abs(z) < 4, z


def test_identical_distributions_accept_everything():
    rng = np.random.default_rng(12)
    k, V = 5, 50
    t = rng.normal(0, 2, size=(k + 1, V))
    d = t[:k].copy()
    for seed in range(20):
        toks = rng.integers(0, V, size=k)
        u, u2 = accept_uniforms(seed, 0, k)
        res = accept_trial(t, d, toks, u, u2)
        assert res.n_acc == k and res.n_out == k + 1
        assert res.tokens[:k] == toks.tolist()


def test_zero_target_probability_always_rejects_and_resamples_from_p():
    V = 6
    p = np.array([0.0, 0.1, 0.2, 0.3, 0.4, 0.0])
    q = np.array([0.0, 0.0, 0.0, 0.0, 0.0, 1.0])     # draft is certain of token 5
    t = _logits([p, np.full(V, 1 / V)])
    d = _logits([q])
    counts = np.zeros(V)
    for seed in range(4000):
        u, u2 = accept_uniforms(seed, 0, 1)
        res = accept_trial(t, d, [5], u, u2)
        assert res.n_acc == 0 and res.residual_row == 0
        counts[res.tokens[0]] += 1
    chi2, dof = _chi2(counts, p)        # residual max(0, p - q) = p here
    assert chi2 < dof + 6 * np.sqrt(2 * dof) + 10


def test_minus_inf_logits_are_never_emitted():
    rng = np.random.default_rng(13)
    k, V = 4, 30
    t = rng.normal(0, 2, size=(k + 1, V)); d = rng.normal(0, 2, size=(k, V))
    t[:, ::3] = -np.inf
    for seed in range(300):
        toks = rng.integers(0, V, size=k)
        u, u2 = accept_uniforms(seed, 0, k)
        res = accept_trial(t, d, toks, u, u2)
        for i, tok in enumerate(res.tokens):
            if i < res.n_acc:
                assert tok == toks[i]
            else:
                assert tok % 3 != 0


def test_invalid_inputs_status():
    V, k = 5, 2
    t = np.zeros((k + 1, V)); d = np.zeros((k, V))
    u = np.zeros(k + 1)
    assert accept_trial(t, d, [0, 5], u, u).status == 1
    assert accept_trial(t, d, [-1, 0], u, u).status == 1
    t2 = t.copy(); t2[1, 2] = np.nan
    assert accept_trial(t2, d, [0, 1], u, u).status == 2
    d2 = d.copy(); d2[0, :] = -np.inf
    assert accept_trial(t, d2, [0, 1], u, u).status == 2
    t3 = t.copy(); t3[2, 0] = np.inf
    assert accept_trial(t3, d, [0, 1], u, u).status == 2


def test_k1_reduces_to_single_position():
    # with one draft the output has one or two tokens and n_acc in {0, 1}
    rng = np.random.default_rng(14)
    V = 10
    t = rng.normal(size=(2, V)); d = rng.normal(size=(1, V))
    seen = set()
    for seed in range(500):
        tok = int(rng.integers(0, V))
        u, u2 = accept_uniforms(seed, 0, 1)
        res = accept_trial(t, d, [tok], u, u2)
        assert res.n_acc in (0, 1) and res.n_out == res.n_acc + 1
        seen.add(res.n_acc)
    assert seen == {0, 1}


def test_forced_decision_at_a_near_tie_continues_the_trial():
    # position 0 is an exact tie: u q(d) = 1/2 * 1/2 = 1/4 = p(d), so the
    # strict test rejects; forcing "accept" there must continue exactly as a
    # trial whose u lies just below the tie (accepting naturally), and
    # forcing "reject" must reproduce the unforced trial
    from oracle import accept_on_probs
    P = np.array([[0.25, 0.25, 0.25, 0.25], [0.375, 0.25, 0.25, 0.125],
                  [0.125, 0.25, 0.25, 0.375], [0.25, 0.25, 0.25, 0.25]])
    Q = np.array([[0.5, 0.125, 0.125, 0.25], [0.125, 0.25, 0.25, 0.375],
                  [0.375, 0.25, 0.25, 0.125]])
    toks = [0, 0, 3]
    u = np.array([0.5, 0.3, 0.9, 0.0])
    u2 = np.array([0.6, 0.2, 0.7, 0.4])
    plain = accept_on_probs(P, Q, toks, u, u2)
    assert plain.n_acc == 0 and plain.accept_flags[0]
    forced_rej = accept_on_probs(P, Q, toks, u, u2, force={0: False})
    assert (forced_rej.n_acc, forced_rej.tokens) == (plain.n_acc, plain.tokens)
    forced_acc = accept_on_probs(P, Q, toks, u, u2, force={0: True})
    below = accept_on_probs(P, Q, toks, np.array([0.5 - 1e-9, 0.3, 0.9, 0.0]), u2)
    assert forced_acc.n_acc >= 1
    assert (forced_acc.n_acc, forced_acc.tokens) == (below.n_acc, below.tokens)
    assert forced_acc.tokens != plain.tokens
    # a position whose decision is not a near tie cannot be forced
    with pytest.raises(ValueError):
        accept_on_probs(P, Q, toks, np.array([0.2, 0.3, 0.9, 0.0]), u2, force={0: False})
