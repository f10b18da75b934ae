"""Seeded synthetic workloads for the verify pass.

This module only draws random inputs: it holds none of the verify-pass
arithmetic (no dequantization, rotation, softmax or accept rule) and imports
neither the HIP binding nor the test oracle, so both sides can be fed the
same tensors.  Every generator takes an explicit seed and a device; the same
(seed, device type) always gives the same tensor.

Workload shapes and distributions:

* W4 weights: codes uniform over all bytes (both nibbles uniform in 0..15),
  zero points integer-valued in 0..15 stored as fp16, scales U(0.01, 0.05)
  stored as fp16, group 64 along K.
* W8 weights: codes uniform in [-127, 127], one fp16 scale U(0.01, 0.05) per
  output channel.
* Activations: N(0, 1) rounded to bf16; the outlier variant multiplies
  round(1% of K) seeded channels by 50.
* Hadamard signs: uniform +-1 int8.
* Accept inputs: draft logits N(0, sd); target = draft + N(0, sigma) noise
  (with an extra independent target row for the bonus position); draft
  tokens sampled from the draft distribution with the Gumbel-max trick.
* LM-head verify: hidden rows N(0, 0.15^2) in bf16 (with the W4 weights
  above the logits then have a standard deviation near 2, as the accept
  inputs); draft logits N(0, 2) independent of the target; draft tokens
  uniform over the vocabulary (so p/q spreads on both sides of 1).
* Draft trees: node j hangs under node j - 1 with probability `chain`, else
  under a uniform pick of the root or an earlier node; target rows are
  N(0, sd) with one planted token per row lifted by 12 sd; a node's token is
  the planted token of its parent's row with probability `agree`, else
  uniform over the vocabulary.
"""

import torch


def _gen(seed, device):
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed))
    return g


def w4_matrix(N, K, seed, device="cpu", group=64):
    """Returns (codes uint8 [N, K/2], scales fp16 [N, K/group], zeros fp16)."""
    g = _gen(seed, device)
    codes = torch.randint(0, 256, (N, K // 2), generator=g, device=device,
                          dtype=torch.int32).to(torch.uint8)
    scales = (torch.rand((N, K // group), generator=g, device=device)
              * 0.04 + 0.01).to(torch.float16)
    zeros = torch.randint(0, 16, (N, K // group), generator=g, device=device,
                          dtype=torch.int32).to(torch.float16)
    return codes, scales, zeros


def w8_matrix(N, K, seed, device="cpu"):
    """Returns (codes int8 [N, K] in [-127, 127], scales fp16 [N])."""
    g = _gen(seed, device)
    codes = torch.randint(-127, 128, (N, K), generator=g, device=device,
                          dtype=torch.int32).to(torch.int8)
    scales = (torch.rand((N,), generator=g, device=device) * 0.04 + 0.01).to(torch.float16)
    return codes, scales


def activations(m, K, seed, device="cpu", scale=1.0):
    """bf16 [m, K] ~ N(0, scale^2)."""
    g = _gen(seed, device)
    return (torch.randn((m, K), generator=g, device=device) * scale).to(torch.bfloat16)


def outlier_activations(m, K, seed, device="cpu", frac=0.01, factor=50.0):
    """N(0, 1) activations with round(frac * K) seeded channels scaled by factor."""
    g = _gen(seed, device)
    x = torch.randn((m, K), generator=g, device=device)
    n_out = int(round(frac * K))
    chans = torch.randperm(K, generator=g, device=device)[:n_out]
    x[:, chans] *= factor
    return x.to(torch.bfloat16), chans


def hadamard_signs(K, seed, device="cpu"):
    g = _gen(seed, device)
    bits = torch.randint(0, 2, (K,), generator=g, device=device, dtype=torch.int32)
    return (bits * 2 - 1).to(torch.int8)


def int8_activations(m, K, seed, device="cpu"):
    """Direct inputs for the int8 GEMM: codes in [-127, 127], scales > 0."""
    g = _gen(seed, device)
    xq = torch.randint(-127, 128, (m, K), generator=g, device=device,
                       dtype=torch.int32).to(torch.int8)
    xs = torch.rand((m,), generator=g, device=device) * 0.05 + 0.001
    return xq, xs.to(torch.float32)


def gumbel_max_tokens(logits, seed, device=None):
    """One token per row of `logits` drawn from softmax(logits).

    Uses argmax(logits + G) with G standard Gumbel noise, which samples the
    softmax distribution exactly (up to the resolution of the uniforms).
    """
    dev = logits.device if device is None else torch.device(device)
    g = _gen(seed, dev)
    u = torch.rand(logits.shape, generator=g, device=dev, dtype=torch.float64)
    u = u.clamp_min(torch.finfo(torch.float64).tiny)
    gumbel = -torch.log(-torch.log(u))
    return torch.argmax(logits.to(torch.float64) + gumbel, dim=-1).to(torch.int32)


def accept_inputs(B, k, V, seed, sigma=1.0, sd=2.0, device="cpu"):
    """Synthetic accept/correct inputs.

    Returns (target fp32 [B, k+1, V], draft fp32 [B, k, V], tokens int32 [B, k]).
    Draft logits ~ N(0, sd); target rows 0..k-1 = draft + N(0, sigma); target
    row k (bonus position) ~ N(0, sd) + N(0, sigma) independently.  sigma=None
    draws the target independently of the draft, N(0, sd).
    """
    g = _gen(seed, device)
    base = torch.randn((B, k + 1, V), generator=g, device=device) * sd
    draft = base[:, :k, :].contiguous()
    if sigma is None:
        target = torch.randn((B, k + 1, V), generator=g, device=device) * sd
    else:
        target = base + torch.randn((B, k + 1, V), generator=g, device=device) * sigma
    tokens = gumbel_max_tokens(draft, seed + 0x5bd1e995, device=device)
    return target.contiguous(), draft, tokens


def tree_inputs(B, n, V, seed, chain=0.7, agree=0.8, sd=2.0, device="cpu"):
    """Synthetic draft trees of n nodes for greedy tree verification.

    Returns (target fp32 [B, n+1, V], tokens int32 [B, n], parents int32
    [B, n]).  Row 0 of the target belongs to the root, row j+1 to node j;
    parents precede children.
    """
    g = _gen(seed, device)
    target = torch.randn((B, n + 1, V), generator=g, device=device) * sd
    planted = torch.randint(0, V, (B, n + 1), generator=g, device=device)
    target.scatter_(2, planted.unsqueeze(-1), 12.0 * sd)
    j = torch.arange(n, device=device).expand(B, n)
    pick = (torch.rand((B, n), generator=g, device=device) * (j + 1)).floor().long() - 1
    use_chain = torch.rand((B, n), generator=g, device=device) < chain
    parents = torch.where(use_chain, j - 1, pick)
    follow = torch.gather(planted, 1, parents + 1)
    other = torch.randint(0, V, (B, n), generator=g, device=device)
    hit = torch.rand((B, n), generator=g, device=device) < agree
    tokens = torch.where(hit, follow, other)
    return target.contiguous(), tokens.to(torch.int32), parents.to(torch.int32)


def lm_head_drafts(B, k, V, seed, sd=2.0, device="cpu"):
    """Draft side of an LM-head verify: (draft logits fp32 [B, k, V] ~ N(0, sd),
    draft tokens int32 [B, k] uniform over the vocabulary)."""
    g = _gen(seed, device)
    draft = torch.randn((B, k, V), generator=g, device=device) * sd
    tokens = torch.randint(0, V, (B, k), generator=g, device=device, dtype=torch.int32)
    return draft, tokens
