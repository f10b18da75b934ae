"""Storage-format decoding for the oracle (test infrastructure only).

Parity: pinned.  bf16 is the upper half of an IEEE binary32 word; fp16 is
IEEE binary16.  The tests pin both against hand-written bit patterns
(1.0, -2.0, smallest normal, a subnormal).
"""

import numpy as np


def bf16_bits_to_f64(bits):
    """Decode bfloat16 values given as their raw 16-bit patterns.

    A bfloat16 is the top 16 bits of a binary32 number, so placing the
    pattern in the upper half of a 32-bit word recovers the binary32 value
    exactly; widening to binary64 is exact as well.
    """
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f16_to_f64(h):
    """Decode IEEE binary16 values (numpy float16 or raw uint16 bits)."""
    a = np.asarray(h)
    if a.dtype == np.uint16 or a.dtype == np.int16:
        a = a.view(np.float16)
    return a.astype(np.float64)
