"""GPU parity of the verify-pass executor (sv_pass_plan + sv_pass_run).

Every GEMM of a planned pass runs in one launch; each output is compared
with the binary64 oracle (dequantize + matmul) on the same seeded inputs.
"""
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


def _gemm(m, K, N, seed):
    """One seeded GEMM: host copies for the oracle, device tensors for the pass."""
    sv = _sv()
    codes, scales, zeros = synth.w4_matrix(N, K, seed=seed)
    x = synth.activations(m, K, seed=seed + 1)
    pc, ps = sv.sv_w4_pack(*to_dev(codes, scales, zeros))
    y = torch.full((m, N), float("nan"), dtype=torch.float32, device=DEV)
    return dict(host=(x, codes, scales, zeros), dev=(x.to(DEV), pc, ps, N, y))


def _oracle(host, rows=None):
    x, codes, scales, zeros = host
    c, s, z = codes.numpy(), scales.numpy(), zeros.numpy()
    if rows is not None:
        c, s, z = c[rows], s[rows], z[rows]
    return oracle.qgemm_w4(bf16_bits(x), c, s, z)


# Shapes: several chunks and item boundaries, a K that is not a multiple of the
# 256-wide chunk, N that is not a multiple of the 512-channel item, the
# smallest legal matrix, and more items than compute units in total.
MIXED = [(512, 1024), (2176, 48), (640, 4160), (128, 16), (4096, 272), (1152, 8192)]


@pytest.mark.parametrize("m", [1, 4, 16, 17, 32])
def test_pass_matches_oracle_mixed_shapes(m):
    sv = _sv()
    gs = [_gemm(m, K, N, seed=300 + 10 * i + m) for i, (K, N) in enumerate(MIXED)]
    p = sv.sv_pass_plan("w4", [g["dev"] for g in gs])
    assert p.items == sum((N // 16 + 31) // 32 for _, N in MIXED)   # 512-channel items
    sv.sv_pass_run(p)
    torch.cuda.synchronize()
    for (K, N), g in zip(MIXED, gs):
        y = g["dev"][4].cpu().numpy()
        assert np.isfinite(y).all(), f"unwritten outputs K={K} N={N}"
        rows = np.arange(N) if N <= 1024 else np.sort(
            np.random.default_rng(N + K).choice(N, size=512, replace=False))
        assert_rows_close(y[:, rows], _oracle(g["host"], rows),
                          what=f"pass m={m} K={K} N={N}")


def test_pass_tiny_configuration():
    # one linear layer K=512, N=1024 at m=4: fewer items than compute units
    sv = _sv()
    g = _gemm(4, 512, 1024, seed=0)
    p = sv.sv_pass_plan("w4", [g["dev"]])
    assert p.grid == 2 and p.items == 2
    sv.sv_pass_run(p)
    torch.cuda.synchronize()
    assert_rows_close(g["dev"][4].cpu().numpy(), _oracle(g["host"]), what="tiny")


@pytest.mark.parametrize("m", [1, 16, 32])
def test_pass_one_hot_rows_exact(m):
    # a one-hot activation row exposes single dequantized weights: exactly
    # (c - z) * s in binary32 for integer zero points
    sv = _sv()
    shapes = [(4096, 4096), (1024, 2064), (12288, 512)]
    gs, cols = [], []
    for i, (K, N) in enumerate(shapes):
        codes, scales, zeros = synth.w4_matrix(N, K, seed=40 + i)
        c = np.random.default_rng(m + 7 * i).choice(K, size=m, replace=False)
        x = torch.zeros((m, K), dtype=torch.bfloat16)
        x[torch.arange(m), torch.as_tensor(c)] = 1.0
        pc, ps = sv.sv_w4_pack(*to_dev(codes, scales, zeros))
        y = torch.empty((m, N), dtype=torch.float32, device=DEV)
        gs.append(((codes, scales, zeros), (x.to(DEV), pc, ps, N, y)))
        cols.append(c)
    p = sv.sv_pass_plan("w4", [d for _, d in gs])
    sv.sv_pass_run(p)
    torch.cuda.synchronize()
    for ((codes, scales, zeros), d), c in zip(gs, cols):
        W = oracle.dequant_w4(codes.numpy(), scales.numpy(), zeros.numpy())
        expect = W[:, c].T.astype(np.float32)
        got = d[4].cpu().numpy()
        bad = np.argwhere(got != expect)
        assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}"


def test_pass_agrees_with_per_gemm_entry_point_and_is_deterministic():
    sv = _sv()
    m = 16
    shapes = [(4096, 12288), (4096, 4096), (4096, 24576), (12288, 4096)]   # one 9B layer
    gs = [_gemm(m, K, N, seed=500 + i) for i, (K, N) in enumerate(shapes)]
    p = sv.sv_pass_plan("w4", [g["dev"] for g in gs])
    sv.sv_pass_run(p)
    first = [g["dev"][4].clone() for g in gs]
    sv.sv_pass_run(p)
    torch.cuda.synchronize()
    for g, y1 in zip(gs, first):
        x, pc, ps, N, y = g["dev"]
        assert torch.equal(y, y1)                       # deterministic
        ref = sv.sv_qgemm_w4_packed(x, pc, ps, N)
        torch.cuda.synchronize()
        rel = (y - ref).norm(dim=1) / ref.norm(dim=1)   # same product, other summation order
        assert float(rel.max()) < 1e-5


def test_pass_in_a_graph_replays_like_eager():
    sv = _sv()
    gs = [_gemm(16, K, N, seed=700 + i) for i, (K, N) in enumerate([(1024, 4096), (2048, 1024)])]
    p = sv.sv_pass_plan("w4", [g["dev"] for g in gs])
    sv.sv_pass_run(p)
    torch.cuda.synchronize()
    eager = [g["dev"][4].clone() for g in gs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            sv.sv_pass_run(p, stream=s)
    torch.cuda.synchronize()
    for _ in range(3):
        for g in gs:
            g["dev"][4].fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for g, e in zip(gs, eager):
            assert torch.equal(g["dev"][4], e)


@pytest.mark.parametrize("m", [16, 1, 32])
def test_full_9b_stack_pass_sampled_channels(m):
    """The 32-layer, 3.93 GB W4 stack in the launch configuration of the
    benchmark (one pass, one launch) at k = 16, and at the two ends of its k
    sweep; 16 sampled channels per GEMM are checked against the oracle."""
    sv = _sv()
    H, F = 4096, 12288
    x_h = synth.activations(m, H, seed=11, device=DEV)
    x_f = synth.activations(m, F, seed=12, device=DEV)
    shapes = [(3 * H, H), (H, H), (2 * F, H), (H, F)]
    gemms, samples = [], []
    rng = np.random.default_rng(2024)
    for layer in range(32):
        for i, (N, K) in enumerate(shapes):
            c, s, z = synth.w4_matrix(N, K, seed=1000 * layer + i, device=DEV)
            pc, ps = sv.sv_w4_pack(c, s, z)
            rows = np.sort(rng.choice(N, size=16, replace=False))
            ri = torch.as_tensor(rows, device=DEV)
            samples.append((rows, c[ri].cpu(), s[ri].cpu(), z[ri].cpu()))
            del c, s, z
            y = torch.full((m, N), float("nan"), dtype=torch.float32, device=DEV)
            gemms.append((x_h if K == H else x_f, pc, ps, N, y))
    p = sv.sv_pass_plan("w4", gemms)
    sv.sv_pass_run(p)
    torch.cuda.synchronize()
    xb = {H: bf16_bits(x_h.cpu()), F: bf16_bits(x_f.cpu())}
    for (x, pc, ps, N, y), (rows, c, s, z) in zip(gemms, samples):
        K = x.shape[1]
        got = y.cpu().numpy()
        assert np.isfinite(got).all()
        ref = oracle.qgemm_w4(xb[K], c.numpy(), s.numpy(), z.numpy())
        assert_rows_close(got[:, rows], ref, what=f"stack N={N} K={K}")


def test_pass_argument_errors():
    sv = _sv()
    g = _gemm(4, 512, 64, seed=31)
    x, pc, ps, N, y = g["dev"]
    with pytest.raises(ValueError):
        sv.sv_pass_plan("w4", [])
    with pytest.raises(ValueError):      # rows must agree across the pass
        sv.sv_pass_plan("w4", [g["dev"], (x[:2].contiguous(), pc, ps, N, y[:2].contiguous())])
    with pytest.raises(TypeError):
        sv.sv_pass_plan("w4", [(x.float(), pc, ps, N, y)])


# ---- W8 and int8 formats of the executor --------------------------------------

def _w8_gemm(m, K, N, seed):
    sv = _sv()
    codes, scales = synth.w8_matrix(N, K, seed=seed)
    x = synth.activations(m, K, seed=seed + 1)
    pc = sv.sv_w8_pack(codes.to(DEV))
    y = torch.full((m, N), float("nan"), dtype=torch.float32, device=DEV)
    return dict(host=(x, codes, scales), dev=(x.to(DEV), pc, scales.to(DEV), N, y))


def _i8_gemm(m, K, N, seed):
    sv = _sv()
    codes, scales, zeros = synth.w4_matrix(N, K, seed=seed)
    xq, xs = synth.int8_activations(m, K, seed=seed + 1)
    pc, ps = sv.sv_w4_pack(*to_dev(codes, scales, zeros))
    y = torch.full((m, N), float("nan"), dtype=torch.float32, device=DEV)
    return dict(host=(xq, xs, codes, scales, zeros),
                dev=(xq.to(DEV), xs.to(DEV), pc, ps, N, y))


@pytest.mark.parametrize("N,K", [(32, 192), (544, 128)])   # one partial group of tiles
def test_w8_pack_layout_matches_contract(N, K):
    from test_gpu_qgemm import packed_block
    sv = _sv()
    codes, _ = synth.w8_matrix(N, K, seed=5)
    KB, nt = K // 64, N // 16
    pc = sv.sv_w8_pack(codes.to(DEV)).cpu().numpy().reshape(nt * KB, 64, 16)
    c = codes.numpy().view(np.uint8)
    for t in range(nt):
        for j in range(KB):
            blk = packed_block(t, j, KB, nt)
            for l in range(64):
                n, q = 16 * t + (l & 15), l >> 4
                assert np.array_equal(pc[blk, l], c[n, 64 * j + 16 * q: 64 * j + 16 * q + 16])


W8_MIXED = [(512, 1024), (192, 48), (640, 4160), (64, 16), (4096, 272), (1088, 8192)]


@pytest.mark.parametrize("m", [1, 5, 16, 17, 32])
def test_w8_pass_matches_oracle(m):
    sv = _sv()
    gs = [_w8_gemm(m, K, N, seed=900 + 10 * i + m) for i, (K, N) in enumerate(W8_MIXED)]
    p = sv.sv_pass_plan("w8", [g["dev"] for g in gs])
    sv.sv_pass_run(p)
    torch.cuda.synchronize()
    for (K, N), g in zip(W8_MIXED, gs):
        x, codes, scales = g["host"]
        y = g["dev"][4].cpu().numpy()
        assert np.isfinite(y).all(), f"unwritten outputs K={K} N={N}"
        rows = np.arange(N) if N <= 1024 else np.sort(
            np.random.default_rng(N + K).choice(N, size=512, replace=False))
        ref = oracle.qgemm_w8(bf16_bits(x), codes.numpy()[rows], scales.numpy()[rows])
        assert_rows_close(y[:, rows], ref, what=f"w8 pass m={m} K={K} N={N}")


@pytest.mark.parametrize("m", [1, 32])
def test_w8_pass_one_hot_rows_exact(m):
    sv = _sv()
    K, N = 4096, 1040
    codes, scales = synth.w8_matrix(N, K, seed=77)
    cols = np.random.default_rng(m).choice(K, size=m, replace=False)
    x = torch.zeros((m, K), dtype=torch.bfloat16)
    x[torch.arange(m), torch.as_tensor(cols)] = 1.0
    y = torch.empty((m, N), dtype=torch.float32, device=DEV)
    pc = sv.sv_w8_pack(codes.to(DEV))
    p = sv.sv_pass_plan("w8", [(x.to(DEV), pc, scales.to(DEV), N, y)])
    sv.sv_pass_run(p)
    torch.cuda.synchronize()
    W = oracle.dequant_w8(codes.numpy(), scales.numpy())
    assert np.array_equal(y.cpu().numpy(), W[:, cols].T.astype(np.float32))


def test_w8_pass_agrees_with_single_gemm_entry_point():
    sv = _sv()
    g = _w8_gemm(16, 12288, 4096, seed=31)
    x, pc, sc, N, y = g["dev"]
    _, codes, _ = g["host"]
    p = sv.sv_pass_plan("w8", [g["dev"]])
    sv.sv_pass_run(p)
    ref = sv.sv_qgemm_w8(x, codes.to(DEV), sc)
    torch.cuda.synchronize()
    rel = (y - ref).norm(dim=1) / ref.norm(dim=1)
    assert float(rel.max()) < 1e-5


I8_MIXED = [(512, 1024), (2176, 48), (640, 4160), (128, 16), (4096, 272), (1152, 8192)]


@pytest.mark.parametrize("m", [1, 4, 16, 17, 32])
def test_w4_i8_pass_matches_oracle(m):
    sv = _sv()
    gs = [_i8_gemm(m, K, N, seed=700 + 10 * i + m) for i, (K, N) in enumerate(I8_MIXED)]
    p = sv.sv_pass_plan("w4_i8", [g["dev"] for g in gs])
    sv.sv_pass_run(p)
    torch.cuda.synchronize()
    for (K, N), g in zip(I8_MIXED, gs):
        xq, xs, codes, scales, zeros = g["host"]
        y = g["dev"][5].cpu().numpy()
        assert np.isfinite(y).all(), f"unwritten outputs K={K} N={N}"
        rows = np.arange(N) if N <= 1024 else np.sort(
            np.random.default_rng(N + K).choice(N, size=512, replace=False))
        ref = oracle.qgemm_w4_i8(xq.numpy(), xs.numpy(), codes.numpy()[rows],
                                 scales.numpy()[rows], zeros.numpy()[rows])
        assert_rows_close(y[:, rows], ref, what=f"w4_i8 pass m={m} K={K} N={N}")


def test_w4_i8_pass_one_hot_rows_exact():
    sv = _sv()
    m, K, N = 32, 4096, 528
    codes, scales, zeros = synth.w4_matrix(N, K, seed=78)
    cols = np.random.default_rng(3).choice(K, size=m, replace=False)
    xq = torch.zeros((m, K), dtype=torch.int8)
    xq[torch.arange(m), torch.as_tensor(cols)] = 1
    xs = torch.ones((m,), dtype=torch.float32)
    pc, ps = sv.sv_w4_pack(*to_dev(codes, scales, zeros))
    y = torch.empty((m, N), dtype=torch.float32, device=DEV)
    p = sv.sv_pass_plan("w4_i8", [(xq.to(DEV), xs.to(DEV), pc, ps, N, y)])
    sv.sv_pass_run(p)
    torch.cuda.synchronize()
    W = oracle.dequant_w4(codes.numpy(), scales.numpy(), zeros.numpy())
    assert np.array_equal(y.cpu().numpy(), W[:, cols].T.astype(np.float32))


@pytest.mark.parametrize("fmt,m", [("w8", 16), ("w4_i8", 16), ("w8", 32)])
def test_full_9b_stack_pass_other_formats_sampled(fmt, m):
    """The 32-layer stack in the W8 and int8 formats at k = 16 (and W8 at the
    top of its k sweep), one launch, in the benchmark's configuration; 8
    sampled channels per GEMM against the oracle."""
    sv = _sv()
    H, F = 4096, 12288
    shapes = [(3 * H, H), (H, H), (2 * F, H), (H, F)]
    if fmt == "w8":
        xs = {H: synth.activations(m, H, seed=11, device=DEV),
              F: synth.activations(m, F, seed=12, device=DEV)}
    else:
        xs = {H: synth.int8_activations(m, H, seed=13, device=DEV),
              F: synth.int8_activations(m, F, seed=14, device=DEV)}
    gemms, samples = [], []
    rng = np.random.default_rng(99)
    for layer in range(32):
        for i, (N, K) in enumerate(shapes):
            rows = np.sort(rng.choice(N, size=8, replace=False))
            ri = torch.as_tensor(rows, device=DEV)
            y = torch.full((m, N), float("nan"), dtype=torch.float32, device=DEV)
            if fmt == "w8":
                c, s = synth.w8_matrix(N, K, seed=5000 + 1000 * layer + i, device=DEV)
                pc = sv.sv_w8_pack(c)
                samples.append((rows, c[ri].cpu(), s[ri].cpu()))
                gemms.append((xs[K], pc, s, N, y))
                del c
            else:
                c, s, z = synth.w4_matrix(N, K, seed=1000 * layer + i, device=DEV)
                pc, ps = sv.sv_w4_pack(c, s, z)
                samples.append((rows, c[ri].cpu(), s[ri].cpu(), z[ri].cpu()))
                gemms.append((xs[K][0], xs[K][1], pc, ps, N, y))
                del c, s, z
    p = sv.sv_pass_plan(fmt, gemms)
    sv.sv_pass_run(p)
    torch.cuda.synchronize()
    for g, smp in zip(gemms, samples):
        y = g[-1].cpu().numpy()
        assert np.isfinite(y).all()
        rows = smp[0]
        if fmt == "w8":
            K = g[0].shape[1]
            ref = oracle.qgemm_w8(bf16_bits(g[0].cpu()), smp[1].numpy(), smp[2].numpy())
        else:
            K = g[0].shape[1]
            ref = oracle.qgemm_w4_i8(g[0].cpu().numpy(), g[1].cpu().numpy(), smp[1].numpy(),
                                     smp[2].numpy(), smp[3].numpy())
        assert_rows_close(y[:, rows], ref, what=f"{fmt} stack K={K}")
