"""Dequantize-then-multiply reference for the verify GEMM (test infrastructure).

The target model "scores all four positions in one forward pass" (Speculative
Decoding Clearly Explained, "Check the guesses together"): every weight is
read once and applied to all m draft rows.  The weight formats are the two
checkpoint tiers of Karpathy's Trick for Faster Local LLMs, "How Uzu optimizes
bytes and tokens per pass": Medium = 4-bit asymmetric integer quantization
with one scale per group, Large = 8-bit symmetric quantization.

Readings taken where the pages are silent:

* W4 storage: codes uint8 [N, K/2]; byte j of output row n holds the code of
  input k = 2j in its low nibble and k = 2j + 1 in its high nibble.  Groups
  are `group` consecutive k within one output row.  Scales and zero points
  are fp16 [N, K/group]; w = (c - z) * s.
* W8 storage: codes int8 [N, K] in [-127, 127], one fp16 scale per output
  channel; w = c * s.
* int8 activation path: Y[r, n] = s_r * sum_g S[n, g] * (I - Z[n, g] * X_g)
  with I = sum_{k in g} C[n, k] * Xq[r, k] and X_g = sum_{k in g} Xq[r, k],
  both exact integers (Karpathy's Trick..., "How Uzu optimizes bytes and
  tokens per pass": both operands of the matrix multiplication are integers).

All arithmetic is binary64 on exactly decoded inputs; the matrix product is a
library primitive (numpy matmul).

Parity: pinned -- by pure-Python brute force from raw bytes on tiny shapes,
by structured inputs that isolate nibble order, group index and zero-point
sign, and by one-hot activations that expose single dequantized weights.
"""

import numpy as np

from .formats import bf16_bits_to_f64, f16_to_f64


def unpack_w4(codes):
    """uint8 [N, K/2] -> int64 codes [N, K] (low nibble = even k)."""
    c = np.asarray(codes, dtype=np.uint8)
    n, half = c.shape
    out = np.empty((n, 2 * half), dtype=np.int64)
    out[:, 0::2] = c & 0x0F
    out[:, 1::2] = c >> 4
    return out


def dequant_w4(codes, scales, zeros, group=64):
    """Dequantized W4 weights in binary64: w[n, k] = (c - z) * s."""
    c = unpack_w4(codes).astype(np.float64)
    s = np.repeat(f16_to_f64(scales), group, axis=1)
    z = np.repeat(f16_to_f64(zeros), group, axis=1)
    if c.shape != s.shape:
        raise ValueError("scale/zero shape does not match codes and group")
    return (c - z) * s


def _x_f64(x):
    """Accept activations as bf16 bit patterns (uint16/int16) or floats."""
    a = np.asarray(x)
    if a.dtype in (np.uint16, np.int16):
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)


def qgemm_w4(x, codes, scales, zeros, group=64):
    """Y[r, n] = sum_k X[r, k] * w[n, k] for the m draft rows of X."""
    return _x_f64(x) @ dequant_w4(codes, scales, zeros, group).T


def dequant_w8(codes, scales):
    """W8 symmetric per-output-channel weights: w[n, k] = c[n, k] * s[n]."""
    c = np.asarray(codes, dtype=np.int8).astype(np.float64)
    return c * f16_to_f64(scales)[:, None]


def qgemm_w8(x, codes, scales):
    return _x_f64(x) @ dequant_w8(codes, scales).T


def group_int_partials(xq, codes, group=64):
    """Exact per-group integer sums of the int8 path.

    Returns (I [m, N, G], X_g [m, G]) as int64, where
    I[r, n, g] = sum_{k in g} C[n, k] * Xq[r, k] and X_g = sum_{k in g} Xq[r, k].
    """
    q = np.asarray(xq, dtype=np.int8).astype(np.int64)
    c = unpack_w4(codes)
    m, K = q.shape
    n = c.shape[0]
    g = K // group
    qg = q.reshape(m, g, group)
    cg = c.reshape(n, g, group)
    inner = np.einsum("rgk,ngk->rng", qg, cg)   # int64 exact
    return inner, qg.sum(axis=2)


def qgemm_w4_i8(xq, xscale, codes, scales, zeros, group=64):
    """int8-activation W4 GEMM in binary64 from exact integer partials."""
    inner, xs = group_int_partials(xq, codes, group)
    s = f16_to_f64(scales)            # [N, G]
    z = f16_to_f64(zeros)             # [N, G]
    corr = inner.astype(np.float64) - z[None, :, :] * xs[:, None, :].astype(np.float64)
    y = np.einsum("rng,ng->rn", corr, s)
    return y * np.asarray(xscale, dtype=np.float64)[:, None]
