"""Pins of the oracle's randomized Hadamard rotation and int8 quantizer."""
import numpy as np
import pytest

from oracle import sylvester, rht, quantize_per_token, hadamard_i8


def _popcount_matrix(b):
    i = np.arange(b)
    pc = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1, -1)


@pytest.mark.parametrize("b", [1, 2, 4, 8, 32, 128, 256])
def test_h_times_h_is_b_identity(b):
    h = sylvester(b).astype(np.int64)
    assert np.array_equal(h @ h, b * np.eye(b, dtype=np.int64))
    assert set(np.unique(h)) <= {-1, 1}


@pytest.mark.parametrize("b", [2, 16, 64])
def test_entries_follow_popcount_definition(b):
    assert np.array_equal(sylvester(b), _popcount_matrix(b))


def test_order_two_closed_form():
    x = np.array([[3.0, 1.0, -2.0, 5.0]])
    y = rht(x, np.ones(4), 2)
    r = np.sqrt(0.5)
    assert np.allclose(y, [[4 * r, 2 * r, 3 * r, -7 * r]], atol=1e-15)


def test_signs_applied_before_mixing():
    x = np.array([[1.0, 2.0]])
    s = np.array([-1.0, 1.0])
    # signs first: (-1, 2) -> (1, -3)/sqrt2 ; mixing first would give (-3, -1)/sqrt2
    assert np.allclose(rht(x, s, 2), [[1 / np.sqrt(2), -3 / np.sqrt(2)]])


def test_reversible_and_norm_preserving():
    rng = np.random.default_rng(0)
    K, b = 1024, 256
    x = rng.standard_normal((3, K))
    s = rng.choice([-1.0, 1.0], size=K)
    y = rht(x, s, b)
    back = rht(y, np.ones(K), b) * s[None, :]
    assert np.allclose(back, x, atol=1e-12)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


def test_block_diagonal_blocks_are_independent():
    rng = np.random.default_rng(1)
    K, b = 96, 32
    x = rng.standard_normal((1, K)); s = rng.choice([-1.0, 1.0], size=K)
    y = rht(x, s, b)
    x2 = x.copy(); x2[0, 40] += 10.0                # perturb block 1 only
    y2 = rht(x2, s, b)
    assert np.array_equal(y[0, :32], y2[0, :32]) and np.array_equal(y[0, 64:], y2[0, 64:])
    assert not np.allclose(y[0, 32:64], y2[0, 32:64])


def test_outlier_spreads_into_moderate_values():
    K = b = 4096
    x = np.zeros((1, K)); x[0, 123] = 50.0
    y = rht(x, np.ones(K), b)
    assert np.allclose(np.abs(y), 50.0 / 64.0)      # 50 / sqrt(4096) everywhere
    rng = np.random.default_rng(2)
    xo = rng.standard_normal((4, K))
    chans = rng.permutation(K)[:41]
    xo[:, chans] *= 50
    s = rng.choice([-1.0, 1.0], size=K)
    yo = rht(xo, s, b)
    ratio_in = np.abs(xo).max(1) / np.sqrt((xo ** 2).mean(1))
    ratio_out = np.abs(yo).max(1) / np.sqrt((yo ** 2).mean(1))
    assert np.all(ratio_out < 0.5 * ratio_in)


def test_rotated_gemm_equivalence():
    # rotating activations and weights by the same orthogonal map leaves X W^T unchanged
    rng = np.random.default_rng(3)
    K, b = 256, 64
    X = rng.standard_normal((5, K)); W = rng.standard_normal((7, K))
    s = rng.choice([-1.0, 1.0], size=K)
    assert np.allclose(rht(X, s, b) @ rht(W, s, b).T, X @ W.T, atol=1e-10)


def test_quantize_known_values_and_ties():
    xt = np.array([[127.0, 63.5, -127.0, 0.5, 1.5, -2.5]])
    for decide in ("f32", "f64"):
        q, s = quantize_per_token(xt, decide=decide)
        assert s[0] == 1.0
        assert q.tolist() == [[127, 64, -127, 0, 2, -2]]      # half to even


def test_quantize_zero_row_and_scale():
    xt = np.array([[0.0, 0.0, 0.0], [0.3, -1.27, 0.0]])
    q, s = quantize_per_token(xt, decide="f64")
    assert s[0] == 1.0 and q[0].tolist() == [0, 0, 0]
    assert abs(s[1] - 0.01) < 1e-15 and q[1].tolist() == [30, -127, 0]
    assert np.abs(q).max() <= 127


def test_hadamard_i8_reconstructs_within_half_step():
    rng = np.random.default_rng(4)
    K = 4096
    x = rng.standard_normal((2, K))
    s = rng.choice([-1, 1], size=K).astype(np.int8)
    q, scale, xt = hadamard_i8(x, s, 4096)
    err = np.abs(q * scale[:, None] - xt)
    assert np.all(err <= 0.5 * scale[:, None] * (1 + 1e-6))
    assert np.all(np.abs(q).max(axis=1) == 127)
