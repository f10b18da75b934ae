"""Pins of the oracle's fused LM-head verification (oracle.lmhead).

* group statistics of constant rows: M = c, S = the group's size (the last
  group shorter);
* merged group statistics equal the log-sum-exp of the whole row, and on rows
  l_v = log(v + 1) the closed form log(V (V + 1) / 2);
* NaN, +inf and all -inf groups;
* one-hot hidden rows through a designed 4-bit projection (scale 1, zero 0)
  give the codes themselves as logits, so the fused verification equals
  oracle.accept on those integer logits (Speculative Decoding Clearly
  Explained, "Check the guesses together").
"""
import math

import numpy as np

from oracle import (group_softmax_stats, merge_group_stats, lm_head_logits, lm_head_verify,
                    row_lse, verify_accept)


def test_constant_rows():
    for V in (64, 100, 1000):
        M, S, bad = group_softmax_stats(np.full((2, V), 1.5))
        G = (V + 63) // 64
        assert M.shape == (2, G) and np.all(M == 1.5) and not bad.any()
        sizes = [64] * (V // 64) + ([V % 64] if V % 64 else [])
        assert np.allclose(S, np.array(sizes, dtype=float)[None, :], rtol=0, atol=1e-12)


def test_merge_is_the_row_log_sum_exp():
    rng = np.random.default_rng(3)
    for V in (1, 63, 64, 65, 4000, 152000):
        x = rng.normal(0, 3, (3, V))
        x[0, rng.integers(0, V, max(1, V // 10))] = -np.inf
        M, S, bad = group_softmax_stats(x)
        lse, ok = merge_group_stats(M, S, bad)
        ref, ref_ok = row_lse(x)
        assert np.array_equal(ok, ref_ok)
        assert np.allclose(lse[ok], ref[ok], rtol=1e-13, atol=1e-12)


def test_closed_form():
    for V in (10, 1000, 152000):
        x = np.log(np.arange(1, V + 1, dtype=np.float64))[None, :]
        lse, ok = merge_group_stats(*group_softmax_stats(x))
        assert ok[0] and abs(lse[0] - math.log(V * (V + 1) / 2)) < 1e-12 * math.log(V * V)


def test_invalid_groups():
    x = np.zeros((4, 200))
    x[0, 70] = np.nan
    x[1, 199] = np.inf
    x[2, :64] = -np.inf                 # one all -inf group: valid, S = 0
    x[3, :] = -np.inf                   # no finite logit: invalid row
    M, S, bad = group_softmax_stats(x)
    assert bad[0].tolist() == [False, True, False, False]
    assert bad[1].tolist() == [False, False, False, True]
    assert M[2, 0] == -np.inf and S[2, 0] == 0.0 and not bad[2].any()
    lse, ok = merge_group_stats(M, S, bad)
    assert ok.tolist() == [False, False, True, False]
    assert abs(lse[2] - math.log(136)) < 1e-12


def _designed_head(V, K, rng):
    codes = rng.integers(0, 256, (V, K // 2), dtype=np.uint8)
    one = np.float16(1.0).view(np.uint16)
    scales = np.full((V, K // 64), one, dtype=np.uint16).view(np.float16)
    zeros = np.zeros((V, K // 64), dtype=np.float16)
    return codes, scales, zeros


def test_projection_of_one_hot_rows():
    rng = np.random.default_rng(8)
    B, k, V, K = 2, 3, 300, 128
    codes, scales, zeros = _designed_head(V, K, rng)
    cols = rng.integers(0, K, B * (k + 1))
    h = np.zeros((B * (k + 1), K))
    h[np.arange(B * (k + 1)), cols] = 1.0
    logits = lm_head_logits(h, codes, scales, zeros, B, k, chunk=128)
    # brute force from the bytes: code k sits in byte k // 2, low nibble for even k
    want = np.empty((B * (k + 1), V))
    for r, c in enumerate(cols):
        byte = codes[:, c // 2].astype(int)
        want[r] = (byte & 15) if c % 2 == 0 else (byte >> 4)
    assert np.array_equal(logits.reshape(-1, V), want)


def test_fused_verify_equals_accept_on_the_projected_logits():
    rng = np.random.default_rng(9)
    B, k, V, K = 3, 4, 250, 128
    codes, scales, zeros = _designed_head(V, K, rng)
    h = np.zeros((B * (k + 1), K))
    h[np.arange(B * (k + 1)), rng.integers(0, K, B * (k + 1))] = 0.5
    draft = rng.normal(0, 2, (B, k, V))
    toks = rng.integers(0, V, (B, k))
    logits, res = lm_head_verify(h, codes, scales, zeros, draft, toks, seed=5, offset=1)
    direct = verify_accept(logits, draft, toks, seed=5, offset=1)
    for a, b in zip(res, direct):
        assert a.status == b.status == 0
        assert a.n_acc == b.n_acc and a.tokens == b.tokens
    assert np.array_equal(logits, lm_head_logits(h, codes, scales, zeros, B, k))


def test_residual_draw_lies_in_its_bin():
    # the running sums and threshold the fused-verify comparison uses: the
    # emitted token's bin [C_{v-1}, C_v) holds the threshold u' S
    rng = np.random.default_rng(12)
    B, k, V = 6, 3, 500
    t = rng.normal(0, 2, (B, k + 1, V))
    d = rng.normal(0, 2, (B, k, V))
    toks = rng.integers(0, V, (B, k))
    for r in verify_accept(t, d, toks, seed=2):
        c, thr, v = r.extra["residual_csum"], r.extra["residual_thr"], r.tokens[-1]
        assert (c[v - 1] if v > 0 else 0.0) <= thr < c[v]
        assert abs(c[-1] - r.weights_sum) == 0.0
