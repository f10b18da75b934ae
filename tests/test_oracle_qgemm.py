"""Pins of the oracle's W4 / W8 / int8 GEMMs.

Independent checks: pure-Python brute force from raw bytes, structured inputs
that isolate nibble order, group index and zero-point sign, one-hot
activations, and the agreement of the integer route with the float route.
"""
import numpy as np
import pytest

from oracle import f16_to_f64
from oracle import (unpack_w4, dequant_w4, qgemm_w4, dequant_w8, qgemm_w8,
                    qgemm_w4_i8, group_int_partials, bf16_bits_to_f64)


def _f16(a):
    return np.asarray(a, dtype=np.float16)


def _rand_w4(rng, N, K, group=64):
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = _f16(rng.uniform(0.01, 0.05, size=(N, K // group)))
    zeros = _f16(rng.integers(0, 16, size=(N, K // group)))
    return codes, scales, zeros


def test_bf16_decode_bit_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0080, 0x0001, 0x7F80, 0x0000], dtype=np.uint16)
    v = bf16_bits_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -2.0
    assert v[2] == 2.0 ** -126 and v[3] == 2.0 ** -133
    assert np.isinf(v[4]) and v[5] == 0.0


def test_f16_decode_raw_bit_patterns():
    """f16_to_f64 on raw binary16 words (uint16 and int16 views) and on
    numpy float16: 1.0, -2.0, the smallest normal 2^-14 and the smallest
    subnormal 2^-24, +inf and -0."""
    words = [0x3C00, 0xC000, 0x0400, 0x0001, 0x7C00, 0x8000]
    want = [1.0, -2.0, 2.0 ** -14, 2.0 ** -24, np.inf, -0.0]
    for arr in (np.array(words, dtype=np.uint16), np.array(words, dtype=np.uint16).view(np.int16),
                np.array(words, dtype=np.uint16).view(np.float16)):
        v = f16_to_f64(arr)
        assert v.dtype == np.float64
        assert v.tolist() == want
        assert np.signbit(v[5])


def test_w4_bruteforce_from_raw_bytes():
    rng = np.random.default_rng(1)
    m, K, N, group = 3, 128, 5, 64
    codes, scales, zeros = _rand_w4(rng, N, K, group)
    x = rng.standard_normal((m, K))
    y = qgemm_w4(x, codes, scales, zeros, group)
    for r in range(m):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                byte = int(codes[n, k // 2])
                c = (byte >> 4) if (k % 2) else (byte & 15)
                w = (c - float(zeros[n, k // group])) * float(scales[n, k // group])
                acc += x[r, k] * w
            assert abs(acc - y[r, n]) <= 1e-12 * (1 + abs(acc))
    assert y.shape == (m, N)


def test_w4_nibble_order():
    K, N = 64, 2
    codes = np.zeros((N, K // 2), dtype=np.uint8)
    codes[1, 3] = 0x21        # low nibble 1 -> k = 6, high nibble 2 -> k = 7
    w = dequant_w4(codes, _f16(np.ones((N, 1))), _f16(np.zeros((N, 1))), 64)
    expect = np.zeros((N, K))
    expect[1, 6], expect[1, 7] = 1.0, 2.0
    assert np.array_equal(w, expect)


def test_w4_group_index_with_one_hot_rows():
    K, N, group = 256, 3, 64
    codes = np.full((N, K // 2), 0x11, dtype=np.uint8)           # every code = 1
    scales = _f16(np.arange(N * (K // group)).reshape(N, K // group) + 1)
    zeros = _f16(np.zeros((N, K // group)))
    for k in (0, 63, 64, 130, 255):
        x = np.zeros((1, K)); x[0, k] = 1.0
        y = qgemm_w4(x, codes, scales, zeros, group)[0]
        assert np.array_equal(y, scales[:, k // group].astype(np.float64))


def test_w4_zero_point_sign():
    K, N = 64, 1
    codes = np.full((N, K // 2), 0x55, dtype=np.uint8)           # c = 5
    s = _f16([[0.5]])
    assert np.all(dequant_w4(codes, s, _f16([[3]]), 64) == 1.0)   # (5 - 3) * 0.5
    assert np.all(dequant_w4(codes, s, _f16([[7]]), 64) == -1.0)  # (5 - 7) * 0.5
    assert np.all(dequant_w4(codes, s, _f16([[5]]), 64) == 0.0)


def test_w4_dequant_exact_in_binary32():
    # (c - z) * s with integer z and fp16 s has at most 16 significant bits
    rng = np.random.default_rng(2)
    codes, scales, zeros = _rand_w4(rng, 16, 256)
    w = dequant_w4(codes, scales, zeros)
    assert np.array_equal(w, w.astype(np.float32).astype(np.float64))


def test_w4_rows_and_columns_not_transposed():
    rng = np.random.default_rng(3)
    m, K, N = 2, 64, 3
    codes, scales, zeros = _rand_w4(rng, N, K)
    W = dequant_w4(codes, scales, zeros)
    x = np.zeros((m, K)); x[0, 5] = 1.0; x[1, 9] = 2.0
    y = qgemm_w4(x, codes, scales, zeros)
    assert np.array_equal(y[0], W[:, 5]) and np.array_equal(y[1], 2 * W[:, 9])


def test_w8_bruteforce_and_sign():
    rng = np.random.default_rng(4)
    m, K, N = 2, 40, 3
    codes = rng.integers(-127, 128, size=(N, K), dtype=np.int8)
    scales = _f16(rng.uniform(0.01, 0.05, size=N))
    x = rng.standard_normal((m, K))
    y = qgemm_w8(x, codes, scales)
    for r in range(m):
        for n in range(N):
            acc = sum(x[r, k] * int(codes[n, k]) * float(scales[n]) for k in range(K))
            assert abs(acc - y[r, n]) <= 1e-12 * (1 + abs(acc))
    c = np.array([[-127, 127, -1, 0]], dtype=np.int8)
    assert np.array_equal(dequant_w8(c, _f16([2.0]))[0], [-254.0, 254.0, -2.0, 0.0])


def test_int8_partials_bruteforce():
    rng = np.random.default_rng(5)
    m, K, N, group = 2, 128, 3, 64
    codes, _, _ = _rand_w4(rng, N, K, group)
    xq = rng.integers(-127, 128, size=(m, K), dtype=np.int8)
    inner, xs = group_int_partials(xq, codes, group)
    for r in range(m):
        for g in range(K // group):
            assert xs[r, g] == sum(int(xq[r, k]) for k in range(g * group, (g + 1) * group))
            for n in range(N):
                ref = 0
                for k in range(g * group, (g + 1) * group):
                    byte = int(codes[n, k // 2])
                    c = (byte >> 4) if (k % 2) else (byte & 15)
                    ref += c * int(xq[r, k])
                assert inner[r, n, g] == ref


def test_int8_route_equals_float_route():
    # integer partials with the zero-point correction must equal the plain
    # dequantize-and-multiply of the dequantized activations
    rng = np.random.default_rng(6)
    m, K, N = 4, 512, 9
    codes, scales, zeros = _rand_w4(rng, N, K)
    zeros = _f16(rng.uniform(0, 15, size=zeros.shape))            # fractional too
    xq = rng.integers(-127, 128, size=(m, K), dtype=np.int8)
    xscale = rng.uniform(0.001, 0.05, size=m)
    y_int = qgemm_w4_i8(xq, xscale, codes, scales, zeros)
    y_flt = qgemm_w4(xq.astype(np.float64) * xscale[:, None], codes, scales, zeros)
    assert np.allclose(y_int, y_flt, rtol=1e-12, atol=1e-12)


def test_unpack_shape_and_range():
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 256, size=(4, 32), dtype=np.uint8)
    c = unpack_w4(codes)
    assert c.shape == (4, 64) and c.min() >= 0 and c.max() <= 15
    assert np.array_equal(c[:, 0::2] + 16 * c[:, 1::2], codes.astype(np.int64))
