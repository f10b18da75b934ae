"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
import numpy as np
import torch

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None

# Floating-point bar: norm-wise relative error per output row against the
# binary64 oracle (binary32 accumulation).
GEMM_RTOL = 2e-3


def to_dev(*ts):
    return [t.to(DEV) for t in ts]


def bf16_bits(x):
    """bf16 tensor -> numpy uint16 bit patterns (the oracle decodes them)."""
    return x.cpu().view(torch.int16).numpy().view(np.uint16)


def row_rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.linalg.norm(got - ref, axis=-1)
    den = np.maximum(np.linalg.norm(ref, axis=-1), 1e-30)
    return num / den


def assert_rows_close(got, ref, rtol=GEMM_RTOL, what=""):
    rel = row_rel_err(got, ref)
    worst = int(np.argmax(rel))
    assert rel.max() <= rtol, (
        f"{what}: row {worst} relative error {rel.max():.3e} > {rtol}; "
        f"max abs diff {np.abs(np.asarray(got) - ref).max():.3e}")
    return rel.max()
