"""Pins of the memory-bound model against the figures the pages print."""
from oracle import (tokens_per_s_bound, stack_weight_count, stack_weight_bytes_w4,
                    stack_weight_bytes_w8, w4_bytes_per_weight)


def test_batch_one_bound_29():
    # Karpathy's Trick ..., "Why batch-one decoding is memory-bound" and Local LLM 4x
    # Faster: 153 GB/s over a 5.2 GB 4-bit checkpoint gives about 29 tokens/s.
    b = tokens_per_s_bound(153e9, 5.2e9)
    assert round(b) == 29 and 29.0 < b < 29.5


def test_tokens_per_pass_scales_bound():
    # Local LLM 4x Faster: 7.5 tokens per pass is how 92 tok/s exceeds the 29 bound.
    assert tokens_per_s_bound(153e9, 5.2e9, 7.5) > 92


def test_stack_accounting():
    # 32 layers x (4 * 4096^2 + 3 * 4096 * 12288) weights
    assert stack_weight_count() == 32 * (4 * 4096 * 4096 + 3 * 4096 * 12288)
    assert w4_bytes_per_weight(64) == 0.5625
    assert abs(stack_weight_bytes_w4() - 3.926e9) < 1e6
    assert abs(stack_weight_bytes_w8() - 6.982e9) < 1e6
