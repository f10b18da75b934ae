"""Pins of the oracle's Gumbel-max coupled verification.

* equal draft and target distributions accept every draft, for any seed --
  the claim of the @trymirai timeline post ("The random number from 1 to 10
  inclusive is": 100% acceptance when the distributions match);
* the target's choice follows softmax(l) (Gumbel-max trick): chi-square
  over trials, and the two-token case against sigmoid(a - b);
* the noise is standard Gumbel (Kolmogorov-Smirnov against exp(-exp(-g))),
  and differs across positions, trials and offsets;
* dominant logits make the accept/emit rule deterministic: agreement up to
  the first disagreement, then the target's choice.
"""
import math

import numpy as np
import pytest

from oracle.coupled import (coupled_drafts, coupled_trial, gumbel_noise, verify_coupled,
                            coupled_choice)


def test_equal_distributions_accept_everything():
    rng = np.random.default_rng(2)
    k, V = 6, 40
    for seed in range(5):
        t = rng.normal(0, 2, (8, k + 1, V))
        toks = coupled_drafts(t[:, :k], seed, offset=seed)
        for r in verify_coupled(t, toks, seed, offset=seed):
            assert r.status == 0 and r.n_acc == k and r.n_out == k + 1


def test_random_number_from_one_to_ten():
    # uniform target and uniform speculator over ten numbers: every guess is
    # taken, and the emitted numbers are uniform
    k, V, B = 4, 10, 3000
    t = np.zeros((B, k + 1, V))
    toks = coupled_drafts(t[:, :k], seed=10)
    res = verify_coupled(t, toks, seed=10)
    assert all(r.n_acc == k for r in res)
    counts = np.bincount([r.tokens[0] for r in res], minlength=V)
    chi2 = ((counts - B / V) ** 2 / (B / V)).sum()
    assert chi2 < 27.9                   # chi-square, 9 dof, p = 0.001


def test_choice_follows_softmax():
    p = np.array([0.4, 0.3, 0.15, 0.1, 0.05])
    logits = np.log(p)
    n = 20000
    counts = np.zeros(len(p))
    for trial in range(n):
        c, _ = coupled_choice(logits, gumbel_noise(7, trial, 0, len(p)))
        counts[c] += 1
    chi2 = ((counts - n * p) ** 2 / (n * p)).sum()
    assert chi2 < 18.5                   # 4 dof, p = 0.001


def test_two_token_choice_is_logistic():
    a, b = 0.7, -0.4
    n = 20000
    hits = sum(coupled_choice([a, b], gumbel_noise(3, trial, 1, 2))[0] == 0
               for trial in range(n))
    p0 = 1.0 / (1.0 + math.exp(-(a - b)))
    z = (hits - n * p0) / math.sqrt(n * p0 * (1 - p0))
    assert abs(z) < 4


def test_noise_is_standard_gumbel_and_varies_with_the_counter():
    g = gumbel_noise(11, 0, 0, 50000)
    x = np.sort(g[np.isfinite(g)])
    cdf = np.exp(-np.exp(-x))
    ks = np.max(np.abs(cdf - (np.arange(1, len(x) + 1) / len(x))))
    assert ks < 1.95 / math.sqrt(len(x))  # KS, p = 0.001
    base = gumbel_noise(11, 0, 0, 64)
    for other in (gumbel_noise(11, 1, 0, 64), gumbel_noise(11, 0, 1, 64),
                  gumbel_noise(11, 0, 0, 64, offset=1), gumbel_noise(12, 0, 0, 64)):
        assert not np.array_equal(base, other)


def test_noise_takes_four_words_per_counter():
    # entry v: word v mod 4 of counter (v // 4, position, trial, tag), so the
    # four entries of one counter differ and entry 4 starts the next counter
    from oracle.philox import philox4x32_10, uniforms24
    seed, trial, pos = 11, 2, 5
    g = gumbel_noise(seed, trial, pos, 10)
    key = np.array([seed, 0], dtype=np.uint64)
    for v in (0, 3, 4, 9):
        w = philox4x32_10(np.array([[v // 4, pos, trial, 3]], dtype=np.uint64), key)[0, v % 4]
        u = float(uniforms24(np.array([w]))[0])
        assert abs(g[v] + math.log(-math.log(u))) <= 1e-14 * max(1.0, abs(g[v]))
    assert len(set(g[:4].tolist())) == 4


def test_dominant_logits_give_the_emit_rule():
    k, V = 4, 12
    t = np.zeros((k + 1, V))
    best = [3, 7, 1, 9, 5]
    for i, v in enumerate(best):
        t[i, v] = 100.0                  # far above any noise on 12 entries
    # agreement at 0 and 1, disagreement at 2: emit the target's choice there
    r = coupled_trial(t, [3, 7, 2, 9], seed=1, trial=0)
    assert r.n_acc == 2 and r.tokens == [3, 7, 1]
    # all agree: the bonus is the target's choice at position k
    r = coupled_trial(t, [3, 7, 1, 9], seed=1, trial=0)
    assert r.n_acc == 4 and r.tokens == [3, 7, 1, 9, 5]
    # disagreement at once
    r = coupled_trial(t, [0, 7, 1, 9], seed=1, trial=0)
    assert r.n_acc == 0 and r.tokens == [3]


def test_invalid_inputs():
    t = np.zeros((3, 5))
    assert coupled_trial(t, [0, 5], 0, 0).status == 1
    assert coupled_trial(t, [-1, 0], 0, 0).status == 1
    t[1, 2] = np.nan
    assert coupled_trial(t, [0, 1], 0, 0).status == 2
    t = np.full((3, 5), -np.inf)
    assert coupled_trial(t, [0, 1], 0, 0).status == 2
