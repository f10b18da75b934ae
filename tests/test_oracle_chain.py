"""Pins of the oracle's hand-off between chained GEMMs (oracle/chain.py).

bf16_rne is checked against torch's binary32 -> bfloat16 conversion, an
independent library routine that rounds to nearest even, and against
hand-written bit patterns for the cases a plausible slip would break: ties
to even in both directions, carries into the exponent, overflow to
infinity, NaN, signed zeros.
"""
import numpy as np
import torch

from oracle import chain


def _bits(*words):
    return np.array(words, dtype=np.uint32).view(np.float32)


def test_bf16_rne_hand_patterns():
    v = _bits(0x3F800000,   # 1.0
              0x3F808000,   # 1 + 2^-8: a tie, kept word even -> stays
              0x3F818000,   # tie, kept word odd -> rounds up to even
              0x3F808001,   # just above the tie -> up
              0x3F807FFF,   # just below -> down
              0x3FFF8000,   # tie, odd, carry into the exponent -> 2.0
              0x7F7FFFFF,   # largest binary32 -> infinity
              0x7F800000,   # +inf
              0xFF800000,   # -inf
              0x80000000,   # -0
              0x80008000,   # tiny negative tie, kept word even -> -0
              0xBF818000)   # -(tie, odd) -> away from zero to even
    got = chain.bf16_rne(v)
    assert got.tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0x3F80, 0x4000, 0x7F80, 0x7F80,
                            0xFF80, 0x8000, 0x8000, 0xBF82]
    nan = chain.bf16_rne(_bits(0x7FC00000, 0x7F800001, 0xFFC12345))
    assert all((b & 0x7F80) == 0x7F80 and (b & 0x7F) != 0 for b in nan.tolist())


def test_bf16_rne_matches_torch_conversion():
    rng = np.random.default_rng(7)
    # every exponent, random fractions, and forced ties (low half 0x8000)
    words = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    ties = (words & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    v = np.concatenate([words, ties]).view(np.float32)
    v = v[np.isfinite(v)]
    ref = torch.from_numpy(v.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(chain.bf16_rne(v), ref)


def test_glue_scales_in_binary32_then_rounds():
    y = np.array([[1.0, 3.0, 1.0 + 2 ** -8, 7.0]], dtype=np.float32)
    assert chain.glue(y, 0.5, 4).tolist() == [[0x3F00, 0x3FC0, 0x3F00, 0x4060]]
    # only the first `cols` channels are handed on
    assert chain.glue(y, 2.0, 2).tolist() == [[0x4000, 0x40C0]]
    # the product is rounded to binary32 first: (1 + 2^-8 - 2^-23)(1 + 2^-23)
    # = 1 + 2^-8 + 2^-31 - 2^-46 is 1 + 2^-8 in binary32, a tie that goes to
    # the even neighbour 1.0 (the exact product would round up)
    y2 = _bits(0x3F807FFF).reshape(1, 1)
    assert chain.glue(y2, np.float32(1.0 + 2 ** -23), 1).tolist() == [[0x3F80]]


def test_glue_candidates_bracket_the_rounding_boundary():
    y = np.array([[1.0 + 2 ** -8, 1.5, -3.0]])   # a tie, then two values far from one
    lo, hi = chain.glue_candidates(y, 1e-6, 1.0, 3)
    assert lo.tolist() == [[0x3F80, 0x3FC0, 0xC040]]
    assert hi.tolist() == [[0x3F81, 0x3FC0, 0xC040]]
