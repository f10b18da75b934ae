"""Memory-bound decode model and weight-byte accounting (test infrastructure).

Source: Karpathy's Trick for Faster Local LLMs, "Why batch-one decoding is
memory-bound": each pass streams every weight once, so tokens per second are
bounded by bandwidth / checkpoint bytes per pass; a base M5 at 153 GB/s with
a 5.2 GB 4-bit 9B checkpoint gives 153 / 5.2 = about 29 tokens per second.
Local LLM 4x Faster states the same bound; with several accepted tokens per
pass the bound scales by tokens per pass.

Parity: pinned by the printed figure (about 29 tokens/s).
"""


def tokens_per_s_bound(bandwidth_bytes_per_s, bytes_per_pass, tokens_per_pass=1.0):
    return bandwidth_bytes_per_s / bytes_per_pass * tokens_per_pass


def w4_bytes_per_weight(group=64, scale_bytes=2, zero_bytes=2):
    """4-bit code plus one fp16 scale and one fp16 zero point per group."""
    return 0.5 + (scale_bytes + zero_bytes) / group


def decoder_stack_shapes(hidden=4096, ffn=12288):
    """(name, N, K) of the seven matrices of one decoder layer."""
    return [("q", hidden, hidden), ("k", hidden, hidden), ("v", hidden, hidden),
            ("o", hidden, hidden), ("gate", ffn, hidden), ("up", ffn, hidden),
            ("down", hidden, ffn)]


def stack_weight_count(layers=32, hidden=4096, ffn=12288):
    return layers * sum(n * k for _, n, k in decoder_stack_shapes(hidden, ffn))


def stack_weight_bytes_w4(layers=32, hidden=4096, ffn=12288, group=64):
    return stack_weight_count(layers, hidden, ffn) * w4_bytes_per_weight(group)


def stack_weight_bytes_w8(layers=32, hidden=4096, ffn=12288):
    """int8 codes plus one fp16 scale per output channel."""
    shapes = decoder_stack_shapes(hidden, ffn)
    return layers * sum(n * k + 2 * n for _, n, k in shapes)
