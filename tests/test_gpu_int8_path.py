"""GPU parity of sv_hadamard_i8 and sv_qgemm_w4_i8 against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from verify_pass_sv_amd import synth
from gpu_util import DEV, to_dev, bf16_bits, assert_rows_close

pytestmark = pytest.mark.gpu


def _sv():
    import verify_pass_sv_amd as sv
    return sv


def _near_tie(xt, scale, tol=1e-6):
    """Where the oracle's binary32 ratio sits within tol of a rounding boundary."""
    a = np.asarray(xt, dtype=np.float64).astype(np.float32)
    r = (a / scale.astype(np.float32)[:, None]).astype(np.float64)
    return np.abs(np.abs(r - np.floor(r)) - 0.5) < tol


@pytest.mark.parametrize("m,K,block,outliers", [
    (4, 4096, 4096, False), (16, 4096, 4096, True), (16, 12288, 4096, True),
    (3, 1024, 32, False), (32, 4096, 256, True), (1, 64, 64, False), (5, 192, 2, False),
    (300, 4096, 4096, True),                       # many token rows in one call
    (8, 8192, 4096, False), (8, 16384, 4096, True)])   # 2 and 4 blocks (above 64 KiB of LDS)
def test_hadamard_codes_and_scales(m, K, block, outliers):
    sv = _sv()
    if outliers:
        x, _ = synth.outlier_activations(m, K, seed=m + K)
    else:
        x = synth.activations(m, K, seed=m + K)
    signs = synth.hadamard_signs(K, seed=3)
    xq, xs = sv.sv_hadamard_i8(*to_dev(x, signs), block)
    torch.cuda.synchronize()
    q_ref, s_ref, xt = oracle.hadamard_i8(bf16_bits(x), signs.numpy(), block, decide="f32")
    got_s = xs.cpu().numpy().astype(np.float64)
    assert np.array_equal(got_s.astype(np.float32), s_ref.astype(np.float32)), \
        f"scales differ: max rel {np.max(np.abs(got_s / s_ref - 1)):.3e}"
    got_q = xq.cpu().numpy().astype(np.int32)
    diff = got_q != q_ref.astype(np.int32)
    ties = _near_tie(xt, s_ref)
    assert np.all(np.abs(got_q - q_ref)[diff] <= 1)
    assert not np.any(diff & ~ties), f"{int((diff & ~ties).sum())} code mismatches off ties"


@pytest.mark.parametrize("K", [4096, 12288, 16384])
def test_hadamard_few_row_form_matches_many_row_form(K):
    """Calls of fewer than 256 rows run four waves per 4096-block, larger calls
    one wave per block: the same rows give the same codes and scales bit for
    bit (the butterflies meet the same pairs in the same order)."""
    sv = _sv()
    x, _ = synth.outlier_activations(300, K, seed=77 + K)
    xd, sd = to_dev(x, synth.hadamard_signs(K, seed=9))
    q_all, s_all = sv.sv_hadamard_i8(xd, sd, 4096)          # 300 rows: one wave per block
    for lo, hi in ((0, 1), (5, 21), (40, 295)):            # 1, 16 and 255 rows
        q, s = sv.sv_hadamard_i8(xd[lo:hi], sd, 4096)
        torch.cuda.synchronize()
        assert torch.equal(q, q_all[lo:hi]), (K, lo, hi)
        assert torch.equal(s.view(torch.int32), s_all[lo:hi].view(torch.int32)), (K, lo, hi)


def test_hadamard_zero_row():
    sv = _sv()
    K = 4096
    x = synth.activations(3, K, seed=1)
    x[1] = 0
    xq, xs = sv.sv_hadamard_i8(*to_dev(x, synth.hadamard_signs(K, seed=2)), 4096)
    torch.cuda.synchronize()
    assert xs[1].item() == 1.0 and int(xq[1].abs().max().item()) == 0
    assert int(xq[0].abs().max().item()) == 127


def test_hadamard_argument_errors():
    sv = _sv()
    x, signs = to_dev(synth.activations(2, 4096, seed=1), synth.hadamard_signs(4096, seed=2))
    with pytest.raises(sv.SvError):
        sv.sv_hadamard_i8(x, signs, 48)          # not a power of two
    with pytest.raises(sv.SvError):
        sv.sv_hadamard_i8(x, signs, 8192)        # above 4096


@pytest.mark.parametrize("m,K,N", [(4, 512, 1024), (16, 4096, 256), (1, 1024, 64),
                                   (23, 2048, 128), (8, 192, 32)])
def test_w4_i8_matches_oracle(m, K, N):
    sv = _sv()
    codes, scales, zeros = synth.w4_matrix(N, K, seed=60 + m)
    xq, xscale = synth.int8_activations(m, K, seed=61 + m)
    y = sv.sv_qgemm_w4_i8(*to_dev(xq, xscale, codes, scales, zeros))
    torch.cuda.synchronize()
    ref = oracle.qgemm_w4_i8(xq.numpy(), xscale.numpy(), codes.numpy(), scales.numpy(),
                             zeros.numpy())
    assert_rows_close(y.cpu().numpy(), ref, what=f"w4_i8 m={m} K={K} N={N}")


# sv_qgemm_w4_i8 with K % 512 == 0 runs the streaming kernel in its
# row-major int8 mode (T = ceil(N / 4096) tiles of 16 channels per
# workgroup, 1024-wide chunks, MT = 1 or 2 row tiles); other K the plain
# kernel.  Every T, both MT, waves past K, ragged chunks and a short last
# workgroup.
@pytest.mark.parametrize("m,K,N", [(16, 4608, 512),      # T 1, ragged last chunk
                                   (32, 2560, 256),      # MT 2
                                   (5, 8704, 4112),      # T 2, 9 chunks
                                   (5, 512, 4112),       # waves past K
                                   (1, 1024, 11200),     # T 3
                                   (24, 512, 16000),     # MT 2, T 4
                                   (9, 1536, 25616)])    # T 6, last workgroup 5 tiles
def test_w4_i8_streaming_kernel(m, K, N):
    sv = _sv()
    codes, scales, zeros = synth.w4_matrix(N, K, seed=80 + m)
    xq, xscale = synth.int8_activations(m, K, seed=81 + m)
    y = sv.sv_qgemm_w4_i8(*to_dev(xq, xscale, codes, scales, zeros))
    torch.cuda.synchronize()
    ref = oracle.qgemm_w4_i8(xq.numpy(), xscale.numpy(), codes.numpy(), scales.numpy(),
                             zeros.numpy())
    assert_rows_close(y.cpu().numpy(), ref, what=f"w4_i8 m={m} K={K} N={N}")


@pytest.mark.parametrize("K", [1024, 4608, 320])
def test_w4_i8_one_hot_exact(K):
    sv = _sv()
    N, m = 64, 32
    codes, scales, zeros = synth.w4_matrix(N, K, seed=70)
    cols = np.random.default_rng(7).choice(K, size=m, replace=False)
    xq = torch.zeros((m, K), dtype=torch.int8)
    xq[torch.arange(m), torch.as_tensor(cols)] = 1
    xscale = torch.ones((m,), dtype=torch.float32)
    y = sv.sv_qgemm_w4_i8(*to_dev(xq, xscale, codes, scales, zeros))
    torch.cuda.synchronize()
    W = oracle.dequant_w4(codes.numpy(), scales.numpy(), zeros.numpy())
    assert np.array_equal(y.cpu().numpy(), W[:, cols].T.astype(np.float32))


@pytest.mark.parametrize("N,K", [(4096, 4096), (12288, 4096), (24576, 4096), (4096, 12288)])
def test_w4_i8_full_size_sampled(N, K):
    # the 9B-class layer shapes at k = 16, sampled output channels
    sv = _sv()
    m = 16
    codes, scales, zeros = synth.w4_matrix(N, K, seed=71, device=DEV)
    xq, xscale = synth.int8_activations(m, K, seed=72, device=DEV)
    y = sv.sv_qgemm_w4_i8(xq, xscale, codes, scales, zeros)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(1).choice(N, size=64, replace=False))
    idx = torch.as_tensor(rows, device=DEV)
    ref = oracle.qgemm_w4_i8(xq.cpu().numpy(), xscale.cpu().numpy(), codes[idx].cpu().numpy(),
                             scales[idx].cpu().numpy(), zeros[idx].cpu().numpy())
    assert_rows_close(y[:, idx].cpu().numpy(), ref, what=f"w4_i8 full {N}x{K}")


def test_rotate_quantize_gemm_chain():
    # hadamard -> int8 GEMM against the oracle's rotate-quantize-GEMM chain
    # (the synthetic codes stand for weights already rotated offline)
    sv = _sv()
    m, K, N = 16, 4096, 512
    x, _ = synth.outlier_activations(m, K, seed=9)
    signs = synth.hadamard_signs(K, seed=3)
    codes, scales, zeros = synth.w4_matrix(N, K, seed=11)
    xd, sd, cd, scd, zd = to_dev(x, signs, codes, scales, zeros)
    xq, xs = sv.sv_hadamard_i8(xd, sd, 4096)
    y = sv.sv_qgemm_w4_i8(xq, xs, cd, scd, zd)
    torch.cuda.synchronize()
    q_ref, s_ref, _ = oracle.hadamard_i8(bf16_bits(x), signs.numpy(), 4096)
    ref = oracle.qgemm_w4_i8(q_ref, s_ref, codes.numpy(), scales.numpy(), zeros.numpy())
    assert_rows_close(y.cpu().numpy(), ref, rtol=1e-4, what="int8 chain")
