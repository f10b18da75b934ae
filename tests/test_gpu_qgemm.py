"""GPU parity of sv_qgemm_w4 / sv_qgemm_w8 against the binary64 oracle."""
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


def _w4_case(m, K, N, seed):
    codes, scales, zeros = synth.w4_matrix(N, K, seed=seed)
    x = synth.activations(m, K, seed=seed + 1)
    return x, codes, scales, zeros


def _w4_oracle(x, codes, scales, zeros, rows=None):
    c, s, z = codes.numpy(), scales.numpy(), zeros.numpy()
    if rows is not None:
        c, s, z = c[rows], s[rows], z[rows]
    return oracle.qgemm_w4(bf16_bits(x), c, s, z)


@pytest.mark.parametrize("m,K,N", [(4, 512, 1024),     # the tiny configuration
                                   (1, 1024, 256), (7, 1024, 256), (16, 2048, 128),
                                   (17, 1024, 256), (32, 4096, 64), (5, 192, 48),
                                   (3, 320, 16)])
def test_w4_matches_oracle(m, K, N):
    sv = _sv()
    x, codes, scales, zeros = _w4_case(m, K, N, seed=10 + m)
    y = sv.sv_qgemm_w4(*to_dev(x, codes, scales, zeros))
    torch.cuda.synchronize()
    assert_rows_close(y.cpu().numpy(), _w4_oracle(x, codes, scales, zeros),
                      what=f"w4 m={m} K={K} N={N}")


# sv_qgemm_w4 with K % 512 == 0 runs the streaming kernel of
# sv_qgemm_w4_packed in its row-major mode: T = ceil(N / 4096) tiles of 16
# channels per workgroup (T in 1, 2, 3, 4, 6), 1024-wide chunks of k through
# a ring of LDS slots, scales and zeros copied per pair of tiles.  These
# cases take every T, both row tiles (MT 1 and 2), waves whose block lies past
# K, one, several and ragged chunks, an odd T (a half-used scale copy) and a
# last workgroup with fewer tiles.
@pytest.mark.parametrize("m,K,N", [(16, 4608, 512),      # T 1, ragged last chunk
                                   (32, 2560, 256),      # MT 2, ragged last chunk
                                   (5, 8704, 4112),      # T 2, 9 chunks
                                   (20, 4096, 8192),     # MT 2, T 2
                                   (16, 16384, 32),      # 16 chunks, 2 tiles in total
                                   (16, 4096, 4112),     # T 2, full K
                                   (5, 512, 4112),       # waves past K
                                   (1, 1024, 11200),     # T 3
                                   (32, 2048, 8208),     # MT 2, T 3
                                   (24, 512, 16000),     # MT 2, T 4
                                   (9, 1536, 25616)])    # T 6, last workgroup 5 tiles
def test_w4_row_major_kernels(m, K, N):
    sv = _sv()
    x, codes, scales, zeros = _w4_case(m, K, N, seed=40 + m)
    y = sv.sv_qgemm_w4(*to_dev(x, codes, scales, zeros))
    torch.cuda.synchronize()
    assert_rows_close(y.cpu().numpy(), _w4_oracle(x, codes, scales, zeros),
                      what=f"w4 m={m} K={K} N={N}")


@pytest.mark.parametrize("K", [512, 4096, 4608, 320])
def test_w4_one_hot_rows_expose_exact_dequant(K):
    # an activation row e_j makes Y[r, n] the single dequantized weight
    # (c - z) * s, which is exact in binary32 for integer zero points
    sv = _sv()
    N, m = 64, 32
    codes, scales, zeros = synth.w4_matrix(N, K, seed=3)
    rng = np.random.default_rng(4)
    cols = rng.choice(K, size=m, replace=False)
    x = torch.zeros((m, K), dtype=torch.bfloat16)
    x[torch.arange(m), torch.as_tensor(cols)] = 1.0
    y = sv.sv_qgemm_w4(*to_dev(x, codes, scales, zeros))
    torch.cuda.synchronize()
    W = oracle.dequant_w4(codes.numpy(), scales.numpy(), zeros.numpy())
    expect = W[:, cols].T.astype(np.float32)
    got = y.cpu().numpy()
    bad = np.argwhere(got != expect)
    assert bad.size == 0, f"{len(bad)} mismatches, first (row, col) {bad[:5].tolist()}: " \
        f"got {got[tuple(bad[0])]} expect {expect[tuple(bad[0])]}"


def test_w4_fractional_zero_points_within_tolerance():
    sv = _sv()
    m, K, N = 8, 1024, 128
    x, codes, scales, _ = _w4_case(m, K, N, seed=21)
    zeros = (torch.rand((N, K // 64), generator=torch.Generator().manual_seed(5)) * 15).half()
    y = sv.sv_qgemm_w4(*to_dev(x, codes, scales, zeros))
    torch.cuda.synchronize()
    assert_rows_close(y.cpu().numpy(), _w4_oracle(x, codes, scales, zeros), what="w4 frac z")


@pytest.mark.parametrize("N,K", [(4096, 4096), (12288, 4096), (24576, 4096), (4096, 12288)])
def test_w4_full_size_shapes_sampled_channels(N, K):
    # the 9B-class layer shapes at k = 16 in the launch configuration the
    # bench uses; the oracle checks a sample of output channels
    sv = _sv()
    m = 16
    codes, scales, zeros = synth.w4_matrix(N, K, seed=N + K, device=DEV)
    x = synth.activations(m, K, seed=7, device=DEV)
    y = sv.sv_qgemm_w4(x, codes, scales, zeros)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(N).choice(N, size=96, replace=False))
    idx = torch.as_tensor(rows, device=DEV)
    ref = oracle.qgemm_w4(bf16_bits(x), codes[idx].cpu().numpy(), scales[idx].cpu().numpy(),
                          zeros[idx].cpu().numpy())
    assert_rows_close(y[:, idx].cpu().numpy(), ref, what=f"w4 full {N}x{K}")


def test_w4_deterministic():
    sv = _sv()
    x, codes, scales, zeros = to_dev(*_w4_case(16, 4096, 1024, seed=30))
    y1 = sv.sv_qgemm_w4(x, codes, scales, zeros)
    y2 = sv.sv_qgemm_w4(x, codes, scales, zeros)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_w4_argument_errors():
    sv = _sv()
    x, codes, scales, zeros = to_dev(*_w4_case(4, 512, 64, seed=31))
    y = torch.empty((4, 64), dtype=torch.float32, device=DEV)
    L, vp = sv.lib, __import__("ctypes").c_void_p
    P = lambda t, off=0: vp(t.data_ptr() + off)
    st = vp(torch.cuda.current_stream().cuda_stream)
    assert L.sv_qgemm_w4(P(x), 4, 512, P(codes), P(scales), P(zeros), 64, 32, P(y), st) == 4
    assert L.sv_qgemm_w4(P(x), 4, 512, P(codes), P(scales), P(zeros), 56, 64, P(y), st) == 2
    assert L.sv_qgemm_w4(P(x), 0, 512, P(codes), P(scales), P(zeros), 64, 64, P(y), st) == 2
    assert L.sv_qgemm_w4(P(x), 33, 512, P(codes), P(scales), P(zeros), 64, 64, P(y), st) == 2
    assert L.sv_qgemm_w4(P(x), 4, 500, P(codes), P(scales), P(zeros), 64, 64, P(y), st) == 2
    assert L.sv_qgemm_w4(P(x, 2), 4, 512, P(codes), P(scales), P(zeros), 64, 64, P(y), st) == 3
    assert L.sv_qgemm_w4(None, 4, 512, P(codes), P(scales), P(zeros), 64, 64, P(y), st) == 1


# ---- W8 ---------------------------------------------------------------------

@pytest.mark.parametrize("m,K,N", [(1, 1024, 256), (4, 512, 1024), (16, 4096, 128),
                                   (17, 1024, 64), (32, 2048, 64), (8, 192, 32)])
def test_w8_matches_oracle(m, K, N):
    sv = _sv()
    codes, scales = synth.w8_matrix(N, K, seed=40 + m)
    x = synth.activations(m, K, seed=41 + m)
    y = sv.sv_qgemm_w8(*to_dev(x, codes, scales))
    torch.cuda.synchronize()
    ref = oracle.qgemm_w8(bf16_bits(x), codes.numpy(), scales.numpy())
    assert_rows_close(y.cpu().numpy(), ref, what=f"w8 m={m} K={K} N={N}")


# sv_qgemm_w8 runs the streaming kernel in its 8-bit mode: T = ceil(N / 4096)
# tiles of 16 channels per workgroup, 512-wide chunks of 64-wide blocks,
# MT = 1 or 2 row tiles.  Every T, both MT, a ragged last chunk (K % 512 !=
# 0), waves past K and a short last workgroup.
@pytest.mark.parametrize("m,K,N", [(16, 4672, 512),      # T 1, ragged last chunk
                                   (32, 2560, 256),      # MT 2
                                   (5, 8704, 4112),      # T 2, 17 chunks
                                   (3, 192, 4112),       # waves past K, one chunk
                                   (1, 1024, 11200),     # T 3
                                   (24, 512, 16000),     # MT 2, T 4
                                   (9, 1536, 25616)])    # T 6, last workgroup 5 tiles
def test_w8_streaming_kernel(m, K, N):
    sv = _sv()
    codes, scales = synth.w8_matrix(N, K, seed=50 + m)
    x = synth.activations(m, K, seed=51 + m)
    y = sv.sv_qgemm_w8(*to_dev(x, codes, scales))
    torch.cuda.synchronize()
    ref = oracle.qgemm_w8(bf16_bits(x), codes.numpy(), scales.numpy())
    assert_rows_close(y.cpu().numpy(), ref, what=f"w8 m={m} K={K} N={N}")


def test_w8_one_hot_rows_exact():
    sv = _sv()
    N, K, m = 64, 1024, 32
    codes, scales = synth.w8_matrix(N, K, seed=50)
    codes[0, :8] = torch.tensor([-127, 127, -1, 0, 1, -64, 64, 3], dtype=torch.int8)
    cols = np.concatenate([np.arange(8), np.random.default_rng(5).choice(np.arange(8, K), m - 8,
                                                                         replace=False)])
    x = torch.zeros((m, K), dtype=torch.bfloat16)
    x[torch.arange(m), torch.as_tensor(cols)] = 1.0
    y = sv.sv_qgemm_w8(*to_dev(x, codes, scales))
    torch.cuda.synchronize()
    W = oracle.dequant_w8(codes.numpy(), scales.numpy())
    expect = W[:, cols].T.astype(np.float32)
    assert np.array_equal(y.cpu().numpy(), expect)


@pytest.mark.parametrize("N,K", [(4096, 4096), (12288, 4096), (24576, 4096), (4096, 12288)])
def test_w8_full_size_sampled(N, K):
    sv = _sv()
    for m in (1, 16, 32):
        codes, scales = synth.w8_matrix(N, K, seed=N + K, device=DEV)
        x = synth.activations(m, K, seed=8, device=DEV)
        y = sv.sv_qgemm_w8(x, codes, scales)
        torch.cuda.synchronize()
        rows = np.sort(np.random.default_rng(K).choice(N, size=64, replace=False))
        idx = torch.as_tensor(rows, device=DEV)
        ref = oracle.qgemm_w8(bf16_bits(x), codes[idx].cpu().numpy(), scales[idx].cpu().numpy())
        assert_rows_close(y[:, idx].cpu().numpy(), ref, what=f"w8 full m={m}")


# ---- packed W4 layout (the streaming layout of the verify pass) --------------

def _packed(codes, scales, zeros):
    sv = _sv()
    return sv.sv_w4_pack(*to_dev(codes, scales, zeros))


def packed_block(t, j, KB, ntile):
    """The documented block index of tile t, k block j (tiles grouped by 32)."""
    g = t // 32
    gt = min(32, ntile - 32 * g)
    return 32 * g * KB + j * gt + t % 32


@pytest.mark.parametrize("N,K", [(32, 256), (560, 384)])   # one partial group of tiles
def test_w4_pack_layout_matches_contract(N, K):
    # the documented tile-major layout, rebuilt independently from the contract
    codes, scales, zeros = synth.w4_matrix(N, K, seed=77)
    pc, ps = _packed(codes, scales, zeros)
    torch.cuda.synchronize()
    cu = oracle.unpack_w4(codes.numpy())            # [N, K] codes in natural k order
    KB, nt = K // 128, N // 16
    pcn = pc.cpu().numpy().reshape(nt * KB, 64, 4, 4)
    s, z = scales.numpy(), zeros.numpy()
    psn = ps.cpu().numpy().reshape(nt * KB, 16, 4)
    for t in range(nt):
        for j in range(KB):
            blk = packed_block(t, j, KB, nt)
            for l in range(64):
                n, q = 16 * t + (l & 15), l >> 4
                for wd in range(4):
                    k0 = 128 * j + 64 * (wd // 2) + 16 * q + 8 * (wd % 2)
                    exp = [cu[n, k0 + b] | (cu[n, k0 + b + 4] << 4) for b in range(4)]
                    assert pcn[blk, l, wd].tolist() == exp, (t, j, l, wd)
            for n in range(16):
                row = 16 * t + n
                exp = np.array([s[row, 2 * j], z[row, 2 * j], s[row, 2 * j + 1], z[row, 2 * j + 1]])
                assert np.array_equal(psn[blk, n], exp)


@pytest.mark.parametrize("m,K,N", [(4, 512, 1024),     # the tiny configuration
                                   (1, 4096, 4096), (16, 4096, 8192), (7, 4096, 12288),
                                   (16, 1024, 16384), (32, 4096, 24576), (17, 12288, 4096),
                                   (3, 2176, 48), (32, 128, 16), (12, 8192, 4160)])
def test_w4_packed_matches_oracle(m, K, N):
    sv = _sv()
    x, codes, scales, zeros = _w4_case(m, K, N, seed=90 + m)
    pc, ps = _packed(codes, scales, zeros)
    y = sv.sv_qgemm_w4_packed(x.to(DEV), pc, ps, N)
    torch.cuda.synchronize()
    rows = np.arange(N) if N <= 2048 else np.sort(
        np.random.default_rng(N).choice(N, size=256, replace=False))
    ref = _w4_oracle(x, codes, scales, zeros, rows=rows)
    assert_rows_close(y.cpu().numpy()[:, rows], ref, what=f"w4 packed m={m} K={K} N={N}")


@pytest.mark.parametrize("m", [1, 16, 32])
def test_w4_packed_one_hot_rows_exact(m):
    sv = _sv()
    N, K = 8192, 4096
    codes, scales, zeros = synth.w4_matrix(N, K, seed=5)
    cols = np.random.default_rng(m).choice(K, size=m, replace=False)
    x = torch.zeros((m, K), dtype=torch.bfloat16)
    x[torch.arange(m), torch.as_tensor(cols)] = 1.0
    pc, ps = _packed(codes, scales, zeros)
    y = sv.sv_qgemm_w4_packed(x.to(DEV), pc, ps, N)
    torch.cuda.synchronize()
    W = oracle.dequant_w4(codes.numpy(), scales.numpy(), zeros.numpy())
    expect = W[:, cols].T.astype(np.float32)
    got = y.cpu().numpy()
    bad = np.argwhere(got != expect)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}"


def test_w4_packed_agrees_with_row_major_entry_point():
    sv = _sv()
    m, K, N = 16, 4096, 12288
    x, codes, scales, zeros = to_dev(*_w4_case(m, K, N, seed=123))
    pc, ps = sv.sv_w4_pack(codes, scales, zeros)
    y1 = sv.sv_qgemm_w4_packed(x, pc, ps, N)
    y2 = sv.sv_qgemm_w4(x, codes, scales, zeros)
    y3 = sv.sv_qgemm_w4_packed(x, pc, ps, N)
    torch.cuda.synchronize()
    assert torch.equal(y1, y3)                     # deterministic
    rel = (y1 - y2).norm(dim=1) / y2.norm(dim=1)    # same product, other summation order
    assert float(rel.max()) < 1e-5


def test_w4_packed_argument_errors():
    sv = _sv()
    x, codes, scales, zeros = to_dev(*_w4_case(4, 512, 64, seed=31))
    pc, ps = sv.sv_w4_pack(codes, scales, zeros)
    L, vp = sv.lib, __import__("ctypes").c_void_p
    P = lambda t, off=0: vp(t.data_ptr() + off)
    y = torch.empty((4, 64), dtype=torch.float32, device=DEV)
    st = vp(torch.cuda.current_stream().cuda_stream)
    assert L.sv_qgemm_w4_packed(P(x), 4, 448, P(pc), P(ps), 64, 64, P(y), st) == 2   # K % 128
    assert L.sv_qgemm_w4_packed(P(x), 4, 512, P(pc), P(ps), 64, 128, P(y), st) == 4  # group
    assert L.sv_qgemm_w4_packed(P(x), 4, 512, P(pc, 8), P(ps), 64, 64, P(y), st) == 3
    assert L.sv_w4_pack(P(codes), P(scales), P(zeros), 64, 192, 64, P(pc), P(ps), st) == 2
