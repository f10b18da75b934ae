"""The hand-off between the GEMMs of a verify pass in model order (test
infrastructure only).

One forward pass passes intermediate values from layer to layer (Karpathy's
Trick for Faster Local LLMs, "How Uzu optimizes bytes and tokens per pass";
"Why batch-one decoding is memory-bound": the runtime reads each layer's
weight blocks and the next layer works on what the previous one produced).
The pages do not define the arithmetic between the GEMMs (attention,
normalization and the MLP activation are outside the verify GEMMs), so the
chained pass uses the plainest hand-off that keeps activations in the
pass's input format and at unit scale:

    xo = bf16_rne(fl32(alpha * y[:, :cols]))

with y the binary32 output of a GEMM, alpha a binary32 scale and bf16_rne
the round-to-nearest-even of a binary32 value to bfloat16 (its upper 16
bits).

Parity: pinned.  `bf16_rne` is checked against torch's binary32 -> bfloat16
conversion (a library routine) and against hand-written bit patterns (ties
to even, overflow to infinity, NaN, signed zero); `glue` against those; the
GEMM itself is `qgemm.qgemm_w4` (pinned in its own module).
"""

import numpy as np


def bf16_rne(v):
    """binary32 values -> bfloat16 bit patterns (uint16), round to nearest,
    ties to even.

    A bfloat16 keeps the sign, the 8 exponent bits and the top 7 fraction bits
    of a binary32 word.  Rounding looks at the 16 dropped bits: above half of
    the last kept bit rounds away from zero, below half truncates, exactly
    half goes to the neighbour whose last kept bit is 0.  Carrying out of the
    fraction raises the exponent (and turns the largest finite values into
    infinity).  A NaN stays a NaN (quiet bit set).
    """
    u = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    kept = u >> np.uint64(16)
    dropped = u & np.uint64(0xFFFF)
    half = np.uint64(0x8000)
    odd = (kept & np.uint64(1)) == 1
    up = (dropped > half) | ((dropped == half) & odd)
    out = kept + up.astype(np.uint64)
    nan = (u & np.uint64(0x7FFFFFFF)) > np.uint64(0x7F800000)
    out = np.where(nan, kept | np.uint64(0x40), out)
    return out.astype(np.uint16)


def glue(y32, alpha, cols):
    """The hand-off of one GEMM: bf16 bits [m, cols] of fl32(alpha * y)."""
    y = np.asarray(y32, dtype=np.float32)[:, :cols]
    return bf16_rne(np.float32(alpha) * y)


def glue_candidates(y64, err, alpha, cols):
    """The hand-off for every binary32 y within `err` of the binary64 value
    y64 (elementwise): the bf16 patterns at the two ends of that interval.
    alpha > 0, so the hand-off is monotone and the two ends bound every
    result a binary32 accumulation inside the interval can give; where they
    agree the result is unique."""
    y = np.asarray(y64, dtype=np.float64)[:, :cols]
    e = np.asarray(err, dtype=np.float64)
    if e.ndim == 2:
        e = e[:, :cols]                         # per-element bounds of the whole y
    e = np.broadcast_to(e, y.shape)
    lo = bf16_rne(np.float32(alpha) * (y - e).astype(np.float32))
    hi = bf16_rne(np.float32(alpha) * (y + e).astype(np.float32))
    return lo, hi
