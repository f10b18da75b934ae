"""Pins of the oracle's verification under sampling settings.

* hand-worked truncations (tests/golden/sampling_truncation.txt): boundary
  inclusion of top-p, ties of top-k by index, temperature, and their order;
* the default settings reproduce the plain accept step exactly;
* top_k = 1 (and a vanishing top_p) equal greedy verification for any
  uniforms, and the page's worked example holds under greedy verification;
* exact output law by quadrature over the uniforms: the first emitted token
  follows the truncated target distribution (distribution preservation,
  Speculative Decoding Clearly Explained, "Correct and continue", applied to
  the truncated rows).
"""
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import (accept_trial, verify_accept, accept_uniforms, truncated_probs,
                    accept_trial_sampled, verify_accept_sampled, greedy_choice,
                    sample_drafts)
from oracle.sampling import check_settings
from conftest import GOLDEN, load_worked_example


def _log(rows):
    with np.errstate(divide="ignore"):
        return np.log(np.array(rows, dtype=np.float64))


def _golden_cases():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "sampling_truncation.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *rest = line.split()
            if key == "case":
                cur = {"name": rest[0]}
                cases.append(cur)
            elif key == "probs":
                cur["probs"] = [float(v) for v in rest]
            elif key == "settings":
                cur["settings"] = (float(rest[0]), int(rest[1]), float(rest[2]))
            elif key == "expect":
                cur["expect"] = [float(v) for v in rest]
    return cases


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_truncation_worked_by_hand(case):
    p, kept, flag = truncated_probs(_log(case["probs"]), *case["settings"])
    np.testing.assert_allclose(p, case["expect"], rtol=0, atol=1e-12)
    assert list(kept) == [e > 0 for e in case["expect"]]
    assert not flag


def test_default_settings_are_the_plain_accept_step():
    rng = np.random.default_rng(5)
    B, k, V = 40, 4, 50
    t = rng.normal(0, 2, (B, k + 1, V))
    d = rng.normal(0, 2, (B, k, V))
    toks = sample_drafts(d, seed=3)
    a = verify_accept(t, d, toks, seed=9, offset=2)
    b = verify_accept_sampled(t, d, toks, seed=9, offset=2)
    for x, y in zip(a, b):
        assert (x.status, x.n_acc, x.tokens) == (y.status, y.n_acc, y.tokens)
        np.testing.assert_allclose(x.p_at, y.p_at, rtol=1e-13)
        np.testing.assert_allclose(x.q_at, y.q_at, rtol=1e-13)


@pytest.mark.parametrize("settings", [(1.0, 1, 1.0), (0.7, 0, 1e-9), (2.0, 1, 0.3)])
def test_single_token_truncation_is_greedy_verification(settings):
    rng = np.random.default_rng(6)
    k, V = 5, 30
    for trial in range(60):
        t = rng.normal(0, 1, (k + 1, V))
        d = rng.normal(0, 1, (k, V))
        # drafts that agree with the target's argmax for a random prefix
        toks = rng.integers(0, V, k)
        agree = rng.integers(0, k + 1)
        for i in range(agree):
            toks[i] = greedy_choice(t[i])
        u, u2 = rng.random(k + 1), rng.random(k + 1)
        g = accept_trial_sampled(t, d, toks, u, u2, 0.0)
        s = accept_trial_sampled(t, d, toks, u, u2, *settings)
        assert g.n_acc == s.n_acc and g.tokens == s.tokens
        assert g.n_acc >= agree


def test_greedy_on_the_page_example():
    # The page's example also holds under greedy verification: "on" and
    # "the" are the target's argmax, "red" is not and "big" is.
    ex = load_worked_example("worked_example_page1.txt")
    res = accept_trial_sampled(ex["target"], ex["draft"], ex["tokens"], None, None, 0.0)
    assert res.n_acc == ex["expect_n_acc"] and res.tokens == ex["expect_tokens"]


def _grid(M):
    return [(i + 0.5) / M for i in range(M)]


@pytest.mark.parametrize("settings,p_expect", [
    # top-k 3: target keeps {0, 2, 3} (2 before 3 by index) -> 3:2:2 of 7;
    # draft keeps {1, 3, 0} -> q' = 1:3:0:3 of 7
    ((1.0, 3, 1.0), [Fraction(3, 7), Fraction(0), Fraction(2, 7), Fraction(2, 7)]),
    # top-p 0.6: target 3/8 + 2/8 (index 2 before 3) >= 0.6 -> {0, 2}, 3:2 of 5;
    # draft 3/8 + 3/8 -> {1, 3}, 1:1
    ((1.0, 0, 0.6), [Fraction(3, 5), Fraction(0), Fraction(2, 5), Fraction(0)]),
])
def test_exact_law_of_the_first_token_is_the_truncated_target(settings, p_expect):
    p0 = [Fraction(3, 8), Fraction(1, 8), Fraction(2, 8), Fraction(2, 8)]
    q0 = [Fraction(1, 8), Fraction(3, 8), Fraction(1, 8), Fraction(3, 8)]
    V, M = 4, 30                       # breakpoints on a 1/30 lattice
    t = _log([[float(v) for v in p0], [0.25] * 4])
    d = _log([[float(v) for v in q0]])
    q_t, kept, _ = truncated_probs(d[0], *settings)
    # the draft's truncated law as exact fractions
    qk = [q0[v] if kept[v] else Fraction(0) for v in range(V)]
    qk = [x / sum(qk) for x in qk]
    np.testing.assert_allclose(q_t, [float(x) for x in qk], rtol=1e-15)
    first = [Fraction(0)] * V
    g = _grid(M)
    for dt in range(V):
        if qk[dt] == 0:
            continue
        for u0 in g:
            for a in g:
                res = accept_trial_sampled(t, d, [dt], [u0, 0.5], [a, 0.5], *settings)
                first[res.tokens[0]] += qk[dt] / (M * M)
    assert first == p_expect


def test_truncated_rows_never_emit_outside_the_target_kept_set():
    rng = np.random.default_rng(8)
    k, V = 3, 40
    for trial in range(100):
        t = rng.normal(0, 2, (k + 1, V))
        d = rng.normal(0, 2, (k, V))
        toks = rng.integers(0, V, k)
        u, u2 = accept_uniforms(trial, 0, k)
        res = accept_trial_sampled(t, d, toks, u, u2, 0.8, 7, 0.9)
        r = res.residual_row
        _, kept, _ = truncated_probs(t[r], 0.8, 7, 0.9)
        assert kept[res.tokens[-1]]


def test_settings_domain():
    for bad in [(-1.0, 0, 1.0), (np.inf, 0, 1.0), (1.0, -1, 1.0), (1.0, 0, 0.0),
                (1.0, 0, 1.5), (1.0, 2.5, 1.0)]:
        with pytest.raises(ValueError):
            check_settings(*bad)
    check_settings(0.0, 0, 1.0)
