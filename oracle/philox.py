"""Philox4x32-10 counter-based generator (test infrastructure only).

The pages say the accept step draws random numbers ("Accept it with
probability min(1, p/q)", Speculative Decoding Clearly Explained, "Accept from
left to right") but do not name a generator.  Reading taken: the published
Philox4x32-10 of Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As
Easy as 1, 2, 3" (SC'11), with

* key   = (seed & 0xffffffff, seed >> 32),
* counter = (position i, trial b, offset, tag), tag 0 for accept/resample,
* output word 0 -> u_i (accept test), word 1 -> u'_i (residual/bonus draw),
* u = (word >> 8) * 2**-24, a multiple of 2**-24 in [0, 1), exact in both
  binary32 and binary64.

Parity: pinned by the known-answer vectors published with the Random123
library (tests/golden/philox_kat.txt).
"""

import numpy as np

_MASK = np.uint64(0xFFFFFFFF)
# Round multipliers and Weyl key increments as published by Salmon et al.
_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = np.uint64(0x9E3779B9)
_W1 = np.uint64(0xBB67AE85)


def philox4x32_10(ctr, key):
    """Ten-round Philox4x32 bijection.

    ctr: integer array [..., 4]; key: integer array [..., 2] (broadcast).
    Returns uint32 array [..., 4].
    """
    ctr = np.asarray(ctr, dtype=np.uint64) & _MASK
    key = np.asarray(key, dtype=np.uint64) & _MASK
    c0, c1, c2, c3 = (ctr[..., j] for j in range(4))
    k0, k1 = key[..., 0], key[..., 1]
    for _ in range(10):
        prod0 = _M0 * c0          # < 2**64: no wrap in uint64
        prod1 = _M1 * c2
        hi0, lo0 = prod0 >> np.uint64(32), prod0 & _MASK
        hi1, lo1 = prod1 >> np.uint64(32), prod1 & _MASK
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
        k0 = (k0 + _W0) & _MASK
        k1 = (k1 + _W1) & _MASK
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def uniforms24(words):
    """Map 32-bit words to uniforms on [0, 1) with 24 random bits."""
    w = np.asarray(words, dtype=np.uint32)
    return (w >> np.uint32(8)).astype(np.float64) * (2.0 ** -24)


def accept_uniforms(seed, trial, k, offset=0, tag=0):
    """Uniform pairs (u_i, u'_i) for positions i = 0..k of one trial.

    Returns two float64 arrays of length k + 1 (position k serves the bonus
    draw when every draft is accepted).
    """
    seed = int(seed)
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], dtype=np.uint64)
    i = np.arange(k + 1, dtype=np.uint64)
    ctr = np.stack([i,
                    np.full_like(i, int(trial) & 0xFFFFFFFF),
                    np.full_like(i, int(offset) & 0xFFFFFFFF),
                    np.full_like(i, int(tag) & 0xFFFFFFFF)], axis=-1)
    out = philox4x32_10(ctr, key)
    return uniforms24(out[:, 0]), uniforms24(out[:, 1])
