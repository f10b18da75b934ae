"""Randomized Hadamard rotation and per-token int8 quantization (test infra).

Source: Karpathy's Trick for Faster Local LLMs Finally Has Proper Tooling,
"How Uzu optimizes bytes and tokens per pass": a block-diagonal Random
Hadamard Transform applied before quantization; the Hadamard matrix holds
only +1/-1 entries plus one overall scale; "random" means random sign flips
applied before the mixing; each block is mixed on its own; the transform is
exactly reversible.  The same section says activations are quantized to
8 bits on the fly so both matrix operands are integers; Local LLM 4x Faster
adds that the checkpoint runs on the int8 matrix path.

Readings taken where the pages are silent:

* H_b is the Sylvester Hadamard matrix, H[i, j] = (-1)**popcount(i & j), and
  the overall scale is b**-0.5 (the choice that makes the map orthogonal,
  hence exactly reversible by applying it again and undoing the signs).
* Per-token symmetric quantization: s_r = max_k |x~[r, k]| / 127,
  code = clamp(round-half-to-even(x~ / s_r), -127, 127); an all-zero row
  gets s_r = 1 and all codes 0.
* The decision x~/s -> code is taken in binary32 (the kernel's precision)
  from the binary64 rotation rounded to binary32; `decide="f64"` keeps it in
  binary64.  Near a rounding boundary the two can differ by one code.

Parity: pinned -- H H = b I, the b = 2 closed form, entrywise popcount
definition vs the recursive construction, reversibility, norm preservation,
outlier spreading and rotated-GEMM equivalence.
"""

import functools

import numpy as np

from .formats import bf16_bits_to_f64


@functools.lru_cache(maxsize=8)
def sylvester(b):
    """Sylvester Hadamard matrix of order b (a power of two), int8 entries."""
    if b < 1 or (b & (b - 1)) != 0:
        raise ValueError("Hadamard order must be a power of two")
    h = np.ones((1, 1), dtype=np.int8)
    while h.shape[0] < b:
        h = np.block([[h, h], [h, -h]])
    h.setflags(write=False)
    return h


def _x_f64(x):
    a = np.asarray(x)
    if a.dtype in (np.uint16, np.int16):
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)


def rht(x, signs, block):
    """x~ = blockdiag(b**-0.5 * H_b) (signs * x), row by row, in binary64."""
    xf = _x_f64(x)
    m, K = xf.shape
    if K % block:
        raise ValueError("block must divide K")
    sg = np.asarray(signs, dtype=np.float64)
    h = sylvester(block).astype(np.float64)
    flipped = (xf * sg[None, :]).reshape(m, K // block, block)
    mixed = flipped @ h.T            # H is symmetric; .T kept for clarity
    return (mixed / np.sqrt(block)).reshape(m, K)


def quantize_per_token(xt, decide="f32"):
    """Symmetric per-row int8 quantization; returns (codes int8, scale f64).

    With decide="f32" the scale and the rounding decision are computed in
    binary32 from x~ rounded to binary32; with "f64" in binary64.
    """
    if decide == "f32":
        a = np.asarray(xt, dtype=np.float64).astype(np.float32)
        amax = np.max(np.abs(a), axis=1)
        scale = (amax / np.float32(127.0)).astype(np.float32)
        scale = np.where(amax > 0, scale, np.float32(1.0)).astype(np.float32)
        ratio = (a / scale[:, None]).astype(np.float32)
    else:
        a = np.asarray(xt, dtype=np.float64)
        amax = np.max(np.abs(a), axis=1)
        scale = np.where(amax > 0, amax / 127.0, 1.0)
        ratio = a / scale[:, None]
    codes = np.clip(np.rint(ratio), -127, 127).astype(np.int8)
    return codes, scale.astype(np.float64)


def hadamard_i8(x, signs, block, decide="f32"):
    """Rotate then quantize: returns (codes int8 [m, K], scale [m], x~ f64)."""
    xt = rht(x, signs, block)
    codes, scale = quantize_per_token(xt, decide=decide)
    return codes, scale, xt
